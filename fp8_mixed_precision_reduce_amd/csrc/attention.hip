// bf16 scaled dot-product attention (no mask) between the fused QKV
// projection and the output projection of the transformer layer: forward and
// backward on the v_mfma_f32_32x32x16_bf16 matrix cores.
//
// Per batch b and head h (head width D = 128):
//   S = Q K^T / sqrt(D),  P = softmax(S) over the keys,  O = P V;
//   backward for dO: dV = P^T dO, dP = dO V^T, dS = P (dP - rowsum(dO * O)),
//   dQ = dS K / sqrt(D), dK = dS^T Q / sqrt(D).
// The pages run this core in bf16 between the FP8 linears ([PT-VI], the
// vision-transformer workload); they do not write it out, so this is the
// textbook form.  Q, K, V are the [Q | K | V] column parts of the projection
// output [B*S][3*H*D] (head h owns columns h*D .. h*D+D-1 of each part); O and
// dO are [B*S][H*D]; dQ, dK, dV are written to the matching parts of
// dqkv [B*S][3*H*D].
//
// Numerics: products of bf16 values are exact in the MFMA and summed in fp32;
// the softmax runs in fp32 in the base-2 domain (x * log2(e) / sqrt(D), then
// v_exp_f32); P and dS are rounded to bf16 (RNE) as operands of the second
// products; the normaliser sums the fp32 P.  The forward saves
// lse2 = m + log2(l) per query (log2 domain) so that the backward recomputes
// P = exp2(S log2(e)/sqrt(D) - lse2) without a second pass.
//
// MFMA operand layout used throughout (32x32x16, 8 bf16 per lane): the first
// operand gives row i = lane % 32, the second column j = lane % 32, and lane
// group g = lane / 32 gives 8 values of the contraction index, the same 8 for
// both operands; accumulator register r of lane l holds
// D[8 (r / 4) + 4 g + r % 4][l % 32].  When a score tile feeds the next product
// (P V, P^T dO, dS K, dS^T Q) its accumulators must hold 8 consecutive keys
// (or queries) per lane group: the row operand of the score product therefore
// reads row sigma(i) for MFMA row i, with sigma swapping bits 2 and 3, so
// register r of group g holds index 16 (r / 8) + 8 g + r % 8.
//
// V (forward), Q, K and dO (backward) are also needed transposed (the token
// index as the contraction index of P V, dO^T P, Q^T dS and K^T dS).  The
// kernels bound by their LDS traffic (the forward and the dK/dV kernel) read
// V^T, Q^T and dO^T tiles that a transpose kernel first writes into the
// caller's workspace (one 16-byte LDS read per fragment instead of two 8-byte
// transposing reads: measured 10 % and 15 % faster); the dQ kernel reads its
// K^T fragments from the row-major K tile with transposing LDS reads
// (ds_read_b64_tr_b16), so K needs no transposed copy.
#include "common.h"

namespace fp8lin {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef float v8f __attribute__((ext_vector_type(8)));

constexpr int kD = 128;            // head width
constexpr int kXcds = 8;

__device__ __forceinline__ int sigma(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

__device__ __forceinline__ v8bf lds16(const uint8_t* p) { return __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(p)); }
__device__ __forceinline__ v8bf as_bf(uint4 u) { return __builtin_bit_cast(v8bf, v4u{u.x, u.y, u.z, u.w}); }

// Eight fp32 accumulators (registers r0 .. r0+7) to eight bf16, RNE.
__device__ __forceinline__ v8bf pack8(const v16f& a, int r0) {
    v8f v = {a[r0], a[r0 + 1], a[r0 + 2], a[r0 + 3], a[r0 + 4], a[r0 + 5], a[r0 + 6], a[r0 + 7]};
    return __builtin_convertvector(v, v8bf);
}

// Lane l and lane l ^ 32 (the two lane groups of an MFMA column) combined
// with one v_permlane32_swap; both lanes get the same value (low half first).
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr float kLazy = 8.0f;   // log2 headroom of the forward's reference maximum

__device__ __forceinline__ v16f mfma(v8bf a, v8bf b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row-major tiles of 256-byte rows (a head's D = 128 bf16): the 16-byte chunk
// index is XOR-swizzled by the row's low 4 bits rotated by two (bits 0-1 to
// 2-3): a bijection of those bits, so 16 rows with distinct low bits (the
// sigma-permuted rows of a quarter wave reading one chunk) hit 16 distinct
// bank groups; and rows r .. r + 3 (r a multiple of 4) put the same four
// consecutive chunks into four different quarters of the banks, so a
// transposing read (four such chunks from each of rows r .. r + 3 and
// r + 8 .. r + 11) hits every bank group twice, its minimum.
__device__ __forceinline__ int swz256(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int off256(int row, int chunk) { return row * 256 + ((chunk ^ swz256(row)) << 4); }
// The forward's and the dK/dV kernel's tiles (no transposing reads) keep the
// plain swizzle by the row's low 4 bits.
__device__ __forceinline__ int off256f(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }
// 64-byte rows (32 tokens): chunk swizzled by (row >> 2) & 3 (four rows span the 64 banks).
__device__ __forceinline__ int off64(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }
// 128-byte rows (64 tokens): chunk swizzled by (row >> 1) & 7 (two rows span the 64 banks).
__device__ __forceinline__ int off128(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;

// One MFMA operand of T^T read from a row-major tile T of 256-byte rows (the
// off256 layout, 128 bf16 per row): lane l receives T[k0 + 8 (l / 32) + e][c0 +
// l % 32] for e = 0..7, by two transposing LDS reads (ds_read_b64_tr_b16).
// Within each 16-lane group such a read hands lane i element i % 4 of the
// 4-element pieces addressed by lanes 4 e + i / 4 of the group (e = 0..3,
// measured); lane k addresses row k / 4 and columns 4 (k % 4) .. + 3 of its
// group's 16, so lane i receives column i of four consecutive rows.  c0 is a
// multiple of 32.
__device__ __forceinline__ v8bf lds_tr(const uint8_t* tile, int k0, int c0, int lane) {
    const int grp = lane >> 4, kk = lane & 15;
    const int col = c0 + 16 * (grp & 1) + 4 * (kk & 3);
    const int r = k0 + 8 * (grp >> 1) + (kk >> 2);
    const int sub = (col & 7) << 1;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(tile + off256(r, col >> 3) + sub));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(tile + off256(r + 4, col >> 3) + sub));
    return __builtin_bit_cast(v8bf, v8s{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// Logical block index: undo the round-robin dealing of workgroups over the 8
// XCDs, so consecutive logical blocks (the same batch and head, which share
// K and V or Q and dO) run on one XCD and share its L2.
__device__ __forceinline__ int xcd_block(int i, int n) {
    const int q = n / kXcds, r = n % kXcds;
    const int xcd = i % kXcds, local = i / kXcds;
    return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

struct AttnShape {
    int32_t batch, seq, heads;
    float c2;              // log2(e) / sqrt(D)
    float scale;           // 1 / sqrt(D)
};

// ------------------------------------------------------------------ forward
// Workgroup: WAVES waves, 32 queries each, of one (b, h).  Key blocks of 64 go
// through three LDS buffers (K [64][256 B] and V^T [128][128 B] each), loaded
// one block ahead by buffer loads that write the LDS directly.
constexpr int kFwdK = 64;
constexpr int kFwdWaves = 8;
constexpr int kFwdBuf = 64 * 256 + 128 * 128;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One wave-instruction of a tile DMA: 16 bytes per lane from the buffer at
// byte offset off land at lds + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const uint8_t* lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, off, 0, 0, 0);
}

template <int WAVES>
__global__ void __launch_bounds__(64 * WAVES, 8 / WAVES)
k_attn_fwd(const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ vt, uint16_t* __restrict__ ctx,
           float* __restrict__ lse, AttnShape sh) {
    constexpr int BQ = 32 * WAVES, NI = 16 / WAVES;   // DMA wave-instructions per tile and wave
    // three key-block buffers as separate arrays, the loop unrolled by three, so
    // the compiler sees that the fragment reads never alias the DMA
    __shared__ __attribute__((aligned(16))) uint8_t smem0[kFwdBuf];
    __shared__ __attribute__((aligned(16))) uint8_t smem1[kFwdBuf];
    __shared__ __attribute__((aligned(16))) uint8_t smem2[kFwdBuf];
    const int S = sh.seq, H = sh.heads;
    const int64_t BS = (int64_t)sh.batch * S, HD = (int64_t)H * kD, ld = 3 * HD;
    const int qblocks = S / BQ;
    const int id = xcd_block(blockIdx.x, gridDim.x);
    const int qb = id % qblocks, h = (id / qblocks) % H, b = id / (qblocks * H);
    const int t = threadIdx.x, lane = t & 63, g = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t tok0 = (int64_t)b * S;
    const int q = qb * BQ + w * 32 + l32;          // this lane's query

    // Q fragments (second operand of S^T = K Q^T): lane's query, d = 16 st + 8 g ..
    v8bf qf[8];
    {
        const uint16_t* qrow = qkv + (tok0 + q) * ld + (int64_t)h * kD;
#pragma unroll
        for (int st = 0; st < 8; ++st) qf[st] = as_bf(*reinterpret_cast<const uint4*>(qrow + 16 * st + 8 * g));
    }
    // Key-block DMA straight into the LDS (16 bytes per lane, lane l at base +
    // 16 l): instruction u of wave w fills K rows 4 (w + WAVES u) .. +3 (256 B
    // each) and V^T rows 8 (w + WAVES u) .. +7 (128 B each), each lane loading
    // the logical chunk whose swizzled place is its own.
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(qkv + tok0 * ld + HD + (int64_t)h * kD), (short)0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vt + (int64_t)h * kD * BS + tok0), (short)0, 0x7FFFFFFF, 0x00020000);
    uint32_t o_k[NI], o_v[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        const int rk_ = 4 * (w + WAVES * u) + (lane >> 4), rv_ = 8 * (w + WAVES * u) + (lane >> 3);
        o_k[u] = (uint32_t)(rk_ * ld + (((lane & 15) ^ (rk_ & 15)) * 8)) * 2;
        o_v[u] = (uint32_t)(rv_ * BS + (((lane & 7) ^ ((rv_ >> 1) & 7)) * 8)) * 2;
    }
    auto dma = [&](int k0, uint8_t* buf) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NI; ++u) {
            dma16(rk, buf + 1024 * (w + WAVES * u), o_k[u] + (uint32_t)k0 * (uint32_t)ld * 2);
            dma16(rv, buf + 64 * 256 + 1024 * (w + WAVES * u), o_v[u] + (uint32_t)k0 * 2);
        }
    };

    v16f o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] = 0.0f;
    float m2 = -__builtin_inff(), lsum = 0.0f;

    // Neighbouring waves run in opposite phases: the odd ("late") waves
    // multiply P V one block behind their scores, so that while one wave runs
    // its softmax (VALU) its neighbour can run products (MFMA) on the matrix
    // core they share.  (Pairing w with w ^ 1 measured 5 % faster than no
    // shift; pairing w with w + 4 gained nothing.)  Three LDS buffers keep
    // block j - 1's V^T for the late waves while block j is used and block
    // j + 1 is loaded.
    const int nblk = S / kFwdK;
    const int row = sigma(l32);
    const bool late = (w & 1) != 0;
    v8bf pl[4];                        // the late waves' P of the previous block
    auto pv = [&](const uint8_t* vb, const v8bf* pb) __attribute__((always_inline)) {
        // O^T += V^T P: keys 16 ks + 8 g + slot = registers 8 (ks & 1) + slot of tile ks / 2
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            v8bf vf[4];
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) vf[dt] = lds16(vb + off128(32 * dt + l32, 2 * ks + g));
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) o[dt] = mfma(vf[dt], pb[ks], o[dt]);
        }
        // reads of step ks + 1 ahead of the MFMAs of step ks
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int ks = 0; ks < 3; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    };
    auto step = [&](int j, const uint8_t* buf, const uint8_t* prev, uint8_t* nxt) __attribute__((always_inline)) {
        if (j + 1 < nblk) dma((j + 1) * kFwdK, nxt);
        if (late && j > 0) pv(prev + 64 * 256, pl);
        // S^T tiles: keys kt * 32 + sigma(i) of the block against the lane's query.
        v16f sc[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) { sc[0][e] = 0.0f; sc[1][e] = 0.0f; }
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            v8bf kf[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) kf[u] = lds16(buf + off256f(32 * (u & 1) + row, 2 * (2 * s2 + (u >> 1)) + g));
#pragma unroll
            for (int u = 0; u < 4; ++u) sc[u & 1] = mfma(kf[u], qf[2 * s2 + (u >> 1)], sc[u & 1]);
        }
        // reads of group s2 + 1 ahead of the MFMAs of group s2
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int s2 = 0; s2 < 3; ++s2) {
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        // block j's maximum; the reference maximum m2 moves only when the block
        // exceeds it by more than kLazy (then every P of the block is <= 2^kLazy,
        // harmless in fp32 and bf16), and O and l are rescaled with it -- exact in
        // the algebra, since both carry the same factor.  max(s * c2) = max(s) * c2
        // (c2 > 0, rounding is monotonic), so the scale goes on the maximum.
        float mx = -__builtin_inff();
#pragma unroll
        for (int e = 0; e < 16; e += 2)
            mx = fmaxf(mx, fmaxf(fmaxf(sc[0][e], sc[0][e + 1]), fmaxf(sc[1][e], sc[1][e + 1])));
        mx = pair_max(mx) * sh.c2;
        if (__any(mx > m2 + kLazy)) {
            const float mnew = mx > m2 + kLazy ? mx : m2;
            const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
            m2 = mnew;
            lsum *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
        }
        float ps = 0.0f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                sc[kt][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kt][e], sh.c2, -m2));
                ps += sc[kt][e];
            }
        lsum += ps;
        v8bf pb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) pb[ks] = pack8(sc[ks >> 1], 8 * (ks & 1));
        if (late) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) pl[ks] = pb[ks];
        } else {
            pv(buf + 64 * 256, pb);
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);     // vmcnt(0): this wave's DMA of the next block landed
        __syncthreads();
    };
    dma(0, smem0);
    __builtin_amdgcn_s_waitcnt(0x0f70);
#pragma unroll
    for (int st = 0; st < 8; ++st) asm volatile("" ::"v"(qf[st]));     // the Q fragments land with the first block
    __syncthreads();
    for (int j = 0; j < nblk; j += 3) {
        step(j, smem0, smem2, smem1);
        if (j + 1 < nblk) step(j + 1, smem1, smem0, smem2);
        if (j + 2 < nblk) step(j + 2, smem2, smem1, smem0);
    }
    if (late) pv((nblk - 1) % 3 == 0 ? smem0 + 64 * 256 : (nblk - 1) % 3 == 1 ? smem1 + 64 * 256 : smem2 + 64 * 256, pl);
    const float ltot = pair_sum(lsum);
    const float inv = 1.0f / ltot;
    uint16_t* orow = ctx + (tok0 + q) * HD + (int64_t)h * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d = 32 * dt + 8 * r4 + 4 * g;
            *reinterpret_cast<uint2*>(orow + d) =
                make_uint2(pack_bf16x2(o[dt][4 * r4] * inv, o[dt][4 * r4 + 1] * inv),
                           pack_bf16x2(o[dt][4 * r4 + 2] * inv, o[dt][4 * r4 + 3] * inv));
        }
    if (g == 0) lse[((int64_t)b * H + h) * S + q] = m2 + __builtin_amdgcn_logf(ltot);
}

// ------------------------------------------------------------ transposes
// out[c][r] = in[r * ld + c] for a rows x cols bf16 view (both multiples of
// 64): 64 x 64 tiles through LDS, 16-byte loads and stores.
__global__ void __launch_bounds__(256)
k_transpose_bf16(const uint16_t* __restrict__ in, int64_t ld, int64_t rows, int64_t cols, uint16_t* __restrict__ out) {
    __shared__ uint16_t tile[64][64 + 2];
    const int64_t tiles_c = cols / 64;
    const int64_t r0 = (int64_t)(blockIdx.x / tiles_c) * 64, c0 = (int64_t)(blockIdx.x % tiles_c) * 64;
    const int t = threadIdx.x;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int c = t + 256 * u, row = c >> 3, cc = (c & 7) * 8;
        const uint4 v = *reinterpret_cast<const uint4*>(in + (r0 + row) * ld + c0 + cc);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            tile[row][cc + 2 * e] = (uint16_t)(w4[e] & 0xFFFFu);
            tile[row][cc + 2 * e + 1] = (uint16_t)(w4[e] >> 16);
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int c = t + 256 * u, orow = c >> 3, rr = (c & 7) * 8;
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w4[e] = (uint32_t)tile[rr + 2 * e][orow] | ((uint32_t)tile[rr + 2 * e + 1][orow] << 16);
        *reinterpret_cast<uint4*>(out + (c0 + orow) * rows + r0 + rr) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
}

// Dq[b][h][s] = sum_d dO * O (fp32): 16 lanes per (token, head), 8 d each,
// then a fixed xor-shuffle tree.
__global__ void __launch_bounds__(256)
k_attn_rowdot(const uint16_t* __restrict__ dctx, const uint16_t* __restrict__ ctx, float* __restrict__ dq_rows,
              AttnShape sh) {
    const int64_t HD = (int64_t)sh.heads * kD;
    const int64_t unit = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;       // (token, head)
    const int sub = threadIdx.x & 15;
    const int64_t n = (int64_t)sh.batch * sh.seq * sh.heads;
    if (unit >= n) return;
    const int64_t tok = unit / sh.heads;
    const int h = (int)(unit % sh.heads);
    const int64_t off = tok * HD + (int64_t)h * kD + sub * 8;
    const uint4 a = *reinterpret_cast<const uint4*>(dctx + off);
    const uint4 c = *reinterpret_cast<const uint4*>(ctx + off);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, cw[4] = {c.x, c.y, c.z, c.w};
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        acc += bf16_to_f32(aw[e] & 0xFFFFu) * bf16_to_f32(cw[e] & 0xFFFFu);
        acc += bf16_to_f32(aw[e] >> 16) * bf16_to_f32(cw[e] >> 16);
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
    if (sub == 0) {
        const int64_t b = tok / sh.seq, s = tok % sh.seq;
        dq_rows[(b * sh.heads + h) * sh.seq + s] = acc;
    }
}

// ------------------------------------------------------------ dK and dV
// Workgroup: 8 waves, 256 keys of one (b, h), 32 per wave (each lane one key;
// its K and V fragments in registers for the whole kernel).  Query blocks of
// 32 go through a double-buffered LDS tile, loaded by buffer loads that write
// the LDS directly: Q and dO [32][256 B], Q^T and dO^T [128][64 B], lse2 and
// Dq [32].
constexpr int kKvKeys = 256, kKvQ = 32, kKvThreads = 512;
constexpr int kKvQt = 32 * 256, kKvBuf = 2 * 32 * 256 + 2 * 128 * 64 + 2 * 32 * 4;

__global__ void __launch_bounds__(kKvThreads, 1)
k_attn_bwd_kv(const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ dctx, const uint16_t* __restrict__ qt,
              const uint16_t* __restrict__ dot, const float* __restrict__ lse, const float* __restrict__ dq_rows,
              uint16_t* __restrict__ dqkv, AttnShape sh) {
    // two query-block buffers as separate arrays, the loop unrolled by two, so
    // the compiler sees that the fragment reads of one never alias the DMA into
    // the other
    __shared__ __attribute__((aligned(16))) uint8_t smem0[kKvBuf];
    __shared__ __attribute__((aligned(16))) uint8_t smem1[kKvBuf];
    const int S = sh.seq, H = sh.heads;
    const int64_t BS = (int64_t)sh.batch * S, HD = (int64_t)H * kD, ld = 3 * HD;
    const int kblocks = S / kKvKeys;
    const int id = xcd_block(blockIdx.x, gridDim.x);
    const int kb = id % kblocks, h = (id / kblocks) % H, b = id / (kblocks * H);
    const int t = threadIdx.x, lane = t & 63, g = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t tok0 = (int64_t)b * S;
    const int key = kb * kKvKeys + w * 32 + l32;

    // the wave's keys: K and V fragments in registers for the whole kernel
    v8bf kf[8], vf[8];
    {
        const uint16_t* krow = qkv + (tok0 + key) * ld + HD + (int64_t)h * kD;
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            kf[st] = as_bf(*reinterpret_cast<const uint4*>(krow + 16 * st + 8 * g));
            vf[st] = as_bf(*reinterpret_cast<const uint4*>(krow + HD + 16 * st + 8 * g));
        }
    }
    // Query-block DMA straight into the LDS (16 bytes per lane, lane l at
    // base + 16 l): wave w fills Q and dO rows 4 w .. 4 w + 3 (256 B each) and
    // Q^T and dO^T rows 16 w .. 16 w + 15 (64 B each); lane l loads the logical
    // chunk whose swizzled place is its own.  Wave 0's lanes 0..15 also load the
    // block's 32 lse2 and 32 Dq values.
    const auto rs = [](const void* p) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, 0x7FFFFFFF, 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t rq = rs(qkv + tok0 * ld + (int64_t)h * kD);
    const __amdgpu_buffer_rsrc_t rdo = rs(dctx + tok0 * HD + (int64_t)h * kD);
    const __amdgpu_buffer_rsrc_t rqt = rs(qt + (int64_t)h * kD * BS + tok0);
    const __amdgpu_buffer_rsrc_t rdot = rs(dot + (int64_t)h * kD * BS + tok0);
    const __amdgpu_buffer_rsrc_t rl = rs(lse + ((int64_t)b * H + h) * S);
    const __amdgpu_buffer_rsrc_t rd = rs(dq_rows + ((int64_t)b * H + h) * S);
    const int r256 = 4 * w + (lane >> 4), c256 = (lane & 15) ^ (r256 & 15);
    const int r64 = 16 * w + (lane >> 2), c64 = (lane & 3) ^ ((r64 >> 2) & 3);
    const uint32_t o_q = (uint32_t)(r256 * ld + c256 * 8) * 2, o_do = (uint32_t)(r256 * HD + c256 * 8) * 2;
    const uint32_t o_t = (uint32_t)(r64 * BS + c64 * 8) * 2;
    auto dma = [&](int q0, uint8_t* buf) __attribute__((always_inline)) {
        const uint32_t qrow = (uint32_t)q0;
        dma16(rq, buf + 1024 * w, o_q + qrow * (uint32_t)ld * 2);
        dma16(rdo, buf + kKvQt + 1024 * w, o_do + qrow * (uint32_t)HD * 2);
        dma16(rqt, buf + 2 * kKvQt + 1024 * w, o_t + qrow * 2);
        dma16(rdot, buf + 2 * kKvQt + 128 * 64 + 1024 * w, o_t + qrow * 2);
        // (a buffer resource is wave-uniform: lse2 by lanes 0..7, Dq by lanes 8..15,
        // which land 128 bytes further)
        if (w == 0 && lane < 8)
            dma16(rl, buf + 2 * kKvQt + 2 * 128 * 64, (qrow + 4 * (uint32_t)lane) * 4);
        if (w == 0 && lane >= 8 && lane < 16)
            dma16(rd, buf + 2 * kKvQt + 2 * 128 * 64, (qrow + 4 * (uint32_t)(lane - 8)) * 4);
    };

    v16f dk[4], dv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) { dk[i][e] = 0.0f; dv[i][e] = 0.0f; }

    const int nblk = S / kKvQ;
    auto block = [&](int j, const uint8_t* buf, uint8_t* nxt) __attribute__((always_inline)) {
        const uint8_t* sq = buf;
        const uint8_t* sdo = buf + kKvQt;
        const uint8_t* sqt = buf + 2 * kKvQt;
        const uint8_t* sdot = sqt + 128 * 64;
        const float* sl = reinterpret_cast<const float*>(sqt + 2 * 128 * 64);
        if (j + 1 < nblk) dma((j + 1) * kKvQ, nxt);
        // S and dP tiles, rows = queries sigma(i) of the block, column = the lane's key.
        v16f s, dp;
#pragma unroll
        for (int e = 0; e < 16; ++e) { s[e] = 0.0f; dp[e] = 0.0f; }
        const int row = sigma(l32);
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            s = mfma(lds16(sq + off256f(row, 2 * st + g)), kf[st], s);
            dp = mfma(lds16(sdo + off256f(row, 2 * st + g)), vf[st], dp);
        }
        // register r holds query 16 (r / 8) + 8 g + r % 8 of the block: P and
        // dS for registers 8 hb .. 8 hb + 7 from 8 consecutive lse2 and Dq values
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const float4 la = *reinterpret_cast<const float4*>(sl + 16 * hb + 8 * g);
            const float4 lc = *reinterpret_cast<const float4*>(sl + 16 * hb + 8 * g + 4);
            const float4 da = *reinterpret_cast<const float4*>(sl + 32 + 16 * hb + 8 * g);
            const float4 dc = *reinterpret_cast<const float4*>(sl + 32 + 16 * hb + 8 * g + 4);
            const float lq[8] = {la.x, la.y, la.z, la.w, lc.x, lc.y, lc.z, lc.w};
            const float dq[8] = {da.x, da.y, da.z, da.w, dc.x, dc.y, dc.z, dc.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * hb + e], sh.c2, -lq[e]));
                s[8 * hb + e] = p;
                dp[8 * hb + e] = p * (dp[8 * hb + e] - dq[e]);
            }
        }
        // dV^T += dO^T P and dK^T += Q^T dS: queries 16 ks + 8 g + slot = registers 8 ks + slot.
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const v8bf pb = pack8(s, 8 * ks), sb = pack8(dp, 8 * ks);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                dv[dt] = mfma(lds16(sdot + off64(32 * dt + l32, 2 * ks + g)), pb, dv[dt]);
                dk[dt] = mfma(lds16(sqt + off64(32 * dt + l32, 2 * ks + g)), sb, dk[dt]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);     // vmcnt(0): this wave's DMA of the next block landed
        __syncthreads();
    };
    dma(0, smem0);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    for (int j = 0; j < nblk; j += 2) {
        block(j, smem0, smem1);
        if (j + 1 < nblk) block(j + 1, smem1, smem0);
    }
    // register r of tile dt holds d = 32 dt + 8 (r / 4) + 4 g + r % 4 of the lane's key
    uint16_t* krow = dqkv + (tok0 + key) * ld + HD + (int64_t)h * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d = 32 * dt + 8 * r4 + 4 * g;
            const float c = sh.scale;
            *reinterpret_cast<uint2*>(krow + d) =
                make_uint2(pack_bf16x2(dk[dt][4 * r4] * c, dk[dt][4 * r4 + 1] * c),
                           pack_bf16x2(dk[dt][4 * r4 + 2] * c, dk[dt][4 * r4 + 3] * c));
            *reinterpret_cast<uint2*>(krow + HD + d) =
                make_uint2(pack_bf16x2(dv[dt][4 * r4], dv[dt][4 * r4 + 1]),
                           pack_bf16x2(dv[dt][4 * r4 + 2], dv[dt][4 * r4 + 3]));
        }
}

// ------------------------------------------------------------------- dQ
// Workgroup: 8 waves, 256 queries of one (b, h), 32 per wave (Q and dO
// fragments in registers).  Key blocks of 32: K and V [32][256 B].
constexpr int kQQ = 256, kQK = 32, kQThreads = 512;
constexpr int kQKt = 32 * 256, kQBuf = 2 * 32 * 256;

__global__ void __launch_bounds__(kQThreads, 1)
k_attn_bwd_q(const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ dctx, const float* __restrict__ lse,
             const float* __restrict__ dq_rows, uint16_t* __restrict__ dqkv,
             AttnShape sh) {
    __shared__ __attribute__((aligned(16))) uint8_t smem0[kQBuf];
    __shared__ __attribute__((aligned(16))) uint8_t smem1[kQBuf];
    const int S = sh.seq, H = sh.heads;
    const int64_t BS = (int64_t)sh.batch * S, HD = (int64_t)H * kD, ld = 3 * HD;
    const int qblocks = S / kQQ;
    const int id = xcd_block(blockIdx.x, gridDim.x);
    const int qb = id % qblocks, h = (id / qblocks) % H, b = id / (qblocks * H);
    const int t = threadIdx.x, lane = t & 63, g = lane >> 5, l32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t tok0 = (int64_t)b * S;
    const int q = qb * kQQ + w * 32 + l32;

    v8bf qf[8], df[8];
    {
        const uint16_t* qrow = qkv + (tok0 + q) * ld + (int64_t)h * kD;
        const uint16_t* drow = dctx + (tok0 + q) * HD + (int64_t)h * kD;
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            qf[st] = as_bf(*reinterpret_cast<const uint4*>(qrow + 16 * st + 8 * g));
            df[st] = as_bf(*reinterpret_cast<const uint4*>(drow + 16 * st + 8 * g));
        }
    }
    float lq = lse[((int64_t)b * H + h) * S + q];
    float dd = dq_rows[((int64_t)b * H + h) * S + q];
    // Key-block DMA straight into the LDS: wave w fills K and V rows 4 w .. 4 w + 3
    // (256 B each), each lane loading the logical chunk whose swizzled place is
    // its own (K^T fragments are read from the K tile by transposing reads).
    const auto rs = [](const void* p) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, 0x7FFFFFFF, 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t rk = rs(qkv + tok0 * ld + HD + (int64_t)h * kD);
    const int r256 = 4 * w + (lane >> 4), c256 = (lane & 15) ^ swz256(r256);
    const uint32_t o_k = (uint32_t)(r256 * ld + c256 * 8) * 2;
    auto dma = [&](int k0, uint8_t* buf) __attribute__((always_inline)) {
        const uint32_t kr = (uint32_t)k0;
        dma16(rk, buf + 1024 * w, o_k + kr * (uint32_t)ld * 2);
        dma16(rk, buf + kQKt + 1024 * w, o_k + kr * (uint32_t)ld * 2 + (uint32_t)HD * 2);
    };

    v16f acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;

    const int nblk = S / kQK;
    auto block = [&](int j, const uint8_t* buf, uint8_t* nxt) __attribute__((always_inline)) {
        if (j + 1 < nblk) dma((j + 1) * kQK, nxt);
        v16f s, dp;
#pragma unroll
        for (int e = 0; e < 16; ++e) { s[e] = 0.0f; dp[e] = 0.0f; }
        const int row = sigma(l32);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            v8bf f[4];      // K and V fragments of steps 2 s2 and 2 s2 + 1
#pragma unroll
            for (int u = 0; u < 4; ++u) f[u] = lds16(buf + (u & 1) * kQKt + off256(row, 2 * (2 * s2 + (u >> 1)) + g));
#pragma unroll
            for (int u = 0; u < 4; u += 2) {
                s = mfma(f[u], qf[2 * s2 + (u >> 1)], s);
                dp = mfma(f[u + 1], df[2 * s2 + (u >> 1)], dp);
            }
        }
        // reads of group s2 + 1 ahead of the MFMAs of group s2
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int s2 = 0; s2 < 3; ++s2) {
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
#pragma unroll
        for (int e = 0; e < 16; ++e) dp[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], sh.c2, -lq)) * (dp[e] - dd);
        // dQ^T += K^T dS: keys 16 ks + 8 g + slot = registers 8 ks + slot
        v8bf kt_f[2][4];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) kt_f[ks][dt] = lds_tr(buf, 16 * ks, 32 * dt, lane);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const v8bf sb = pack8(dp, 8 * ks);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) acc[dt] = mfma(kt_f[ks][dt], sb, acc[dt]);
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);     // vmcnt(0): this wave's DMA of the next block landed
        __syncthreads();
    };
    dma(0, smem0);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    // The per-query fragments and row statistics land together with the first
    // block: left to the scheduler, their loads move past this barrier and the
    // loop's first uses wait on the memory counter, which then (in every
    // iteration) also waits for the next block's DMA in the middle of the
    // products.
#pragma unroll
    for (int st = 0; st < 8; ++st) asm volatile("" ::"v"(qf[st]), "v"(df[st]));
    asm volatile("" : "+v"(lq), "+v"(dd));
    __syncthreads();
    for (int j = 0; j < nblk; j += 2) {
        block(j, smem0, smem1);
        if (j + 1 < nblk) block(j + 1, smem1, smem0);
    }
    uint16_t* qrow = dqkv + (tok0 + q) * ld + (int64_t)h * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d = 32 * dt + 8 * r4 + 4 * g;
            const float c = sh.scale;
            *reinterpret_cast<uint2*>(qrow + d) =
                make_uint2(pack_bf16x2(acc[dt][4 * r4] * c, acc[dt][4 * r4 + 1] * c),
                           pack_bf16x2(acc[dt][4 * r4 + 2] * c, acc[dt][4 * r4 + 3] * c));
        }
}

AttnShape make_shape(int64_t batch, int64_t seq, int64_t heads) {
    AttnShape sh;
    sh.batch = (int32_t)batch; sh.seq = (int32_t)seq; sh.heads = (int32_t)heads;
    sh.scale = (float)(1.0 / 11.313708498984761);                 // 1 / sqrt(128)
    sh.c2 = (float)(1.4426950408889634 / 11.313708498984761);     // log2(e) / sqrt(128)
    return sh;
}

hipError_t transpose(const uint16_t* in, int64_t ld, int64_t rows, int64_t cols, uint16_t* out, hipStream_t s) {
    const int64_t tiles = (rows / 64) * (cols / 64);
    hipLaunchKernelGGL(k_transpose_bf16, dim3((unsigned)tiles), dim3(256), 0, s, in, ld, rows, cols, out);
    return hipGetLastError();
}

}  // namespace

// Shapes are validated by the caller: seq a multiple of 256, head width 128,
// batch * seq * heads * 128 elements within the int32 index range of a tile.
hipError_t launch_attention_fwd(const uint16_t* qkv, int64_t batch, int64_t seq, int64_t heads, uint16_t* ctx,
                                float* lse, uint16_t* vt_ws, hipStream_t s) {
    const AttnShape sh = make_shape(batch, seq, heads);
    const int64_t BS = batch * seq, HD = heads * kD;
    timing_before(kKindOther, s);
    hipError_t e = transpose(qkv + 2 * HD, 3 * HD, BS, HD, vt_ws, s);
    timing_after(s);
    if (e != hipSuccess) return e;
    timing_before(kKindAttn, s);
    constexpr int waves = kFwdWaves;
    const int64_t blocks = batch * heads * (seq / (32 * waves));
    hipLaunchKernelGGL(k_attn_fwd<waves>, dim3((unsigned)blocks), dim3(64 * waves), 0, s, qkv, vt_ws, ctx, lse, sh);
    e = hipGetLastError();
    timing_after(s);
    return e;
}

hipError_t launch_attention_bwd(const uint16_t* qkv, const uint16_t* ctx, const float* lse, const uint16_t* dctx,
                                int64_t batch, int64_t seq, int64_t heads, uint16_t* dqkv, uint16_t* qt_ws,
                                uint16_t* dot_ws, float* rows_ws, hipStream_t s) {
    const AttnShape sh = make_shape(batch, seq, heads);
    const int64_t BS = batch * seq, HD = heads * kD;
    timing_before(kKindOther, s);
    hipError_t e = transpose(qkv, 3 * HD, BS, HD, qt_ws, s);
    if (e == hipSuccess) e = transpose(dctx, HD, BS, HD, dot_ws, s);
    if (e == hipSuccess) {
        const int64_t units = BS * heads;
        hipLaunchKernelGGL(k_attn_rowdot, dim3((unsigned)((units * 16 + 255) / 256)), dim3(256), 0, s, dctx, ctx,
                           rows_ws, sh);
        e = hipGetLastError();
    }
    timing_after(s);
    if (e != hipSuccess) return e;
    timing_before(kKindAttn, s);
    hipLaunchKernelGGL(k_attn_bwd_kv, dim3((unsigned)(batch * heads * (seq / kKvKeys))), dim3(kKvThreads), 0, s, qkv,
                       dctx, qt_ws, dot_ws, lse, rows_ws, dqkv, sh);
    e = hipGetLastError();
    timing_after(s);
    if (e != hipSuccess) return e;
    timing_before(kKindAttn, s);
    hipLaunchKernelGGL(k_attn_bwd_q, dim3((unsigned)(batch * heads * (seq / kQQ))), dim3(kQThreads), 0, s, qkv, dctx,
                       lse, rows_ws, dqkv, sh);
    e = hipGetLastError();
    timing_after(s);
    return e;
}

}  // namespace fp8lin
