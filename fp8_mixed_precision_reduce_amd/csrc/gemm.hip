// FP8 x FP8 GEMM with fp32 accumulation on CDNA4 matrix cores and a fused
// epilogue.
//
//   y[i][j] = (sum_k dec(A[i][k]) * dec(B[j][k])) * sinv_a * sinv_b + bias[j]
//   D[i][j] = gelu(y) | y | D[i][j] + y, plus an optional residual R[i][j],
//   rounded to fp32 or bf16; optional pre-GeLU copy and the amax of D as
//   written.
//
// Pages (titles in include/fp8lin.h): [PT-VI] torch._scaled_mm example (two
// FP8 operands, the second transposed, their scales, optional bias, output
// type, output amax); [MP-KR] "Accumulation into FP32"; [TE-RU] section 3
// (inverse scaling after the GEMM).
//
// Two inner products, chosen per call:
//  * exact (default): each FP8 fragment is decoded to f16 in registers after
//    the LDS read (v_cvt_scalef32_pk_f16_fp8/bf8, exact: every E4M3 and E5M2
//    value is an f16 value) and multiplied with v_mfma_f32_32x32x16_f16, whose
//    products are exact and whose sums keep fp32 precision.  This meets an
//    fp32-accumulation bound.
//  * fast (FP8LIN_EPI_FAST_ACCUM): v_mfma_f32_32x32x64_f8f6f4 on the codes
//    directly, twice the MFMA rate.  Measured on gfx950: the instruction adds
//    its products in groups of 8 consecutive k aligned to the group's largest
//    product and keeps about 14 bits there (a product 2^-14 below the group
//    maximum is dropped); partial sums across groups and into the accumulator
//    are fp32.  This is the same kind of reduced-precision FP8 accumulation
//    the H100 example on the Transformer Engine page exhibits.
//
// Tiling.  Both operands are contiguous along k ("TN").  A workgroup of
// WM x WN waves computes a BM x BN tile; each wave owns MB x NB blocks of
// 32 x 32.  The kernel is persistent: one resident wave of workgroups loops
// over the tiles (a tile's output stores are still in flight when the next
// tile's first stage is fetched; vector-memory operations retire in issue
// order, so that stage's wait covers them).  k advances in stages of 128 bytes through a double-buffered LDS
// tile.  The next stage is fetched while the current one is multiplied, with
// buffer loads that write straight into LDS (buffer_load_dwordx4 ... lds: no
// staging registers, out-of-range rows and the k tail read as zero).  LDS rows
// are 128 bytes with the 16-byte chunk index XOR-swizzled by (row >> 1) & 7,
// so a DMA wave-instruction fills 8 rows and the 16-byte fragment reads of 16
// consecutive rows (one LDS cycle on gfx950's 64 banks) hit 16 distinct bank
// groups; with a (row & 7) swizzle the counters showed 2-way conflicts.  Each lane reads 16 bytes
// of k per fragment: the exact path splits them into two f16 MFMAs (bytes
// 0-7 and 8-15; A and B use the same split, so the k order inside an MFMA is
// only permuted), the fast path reads 32 bytes per 64-k MFMA.  Fragments of
// the next k block are read before the current block's MFMAs are issued
// (exact path; the fast path reads each block's fragments just before its
// MFMAs).  The two LDS stages are separate arrays and the k loop is unrolled
// by two, so the compiler sees that a stage's fragment reads never alias the
// DMA into the other stage and inserts no wait for that DMA before them; the
// whole next-stage DMA is issued at the start of a stage (the longest lead).
// The MFMA takes the B tile as
// its first operand, so each lane's accumulators run along n: four
// consecutive outputs of one row.  The outputs (bf16, fp32, and the pre-GeLU
// copy) are first staged in the LDS, which is free after the k loop, and then
// written by the whole workgroup in 16-byte pieces that cover complete row
// segments, with non-temporal stores (only fp32 outputs with GeLU are written
// straight from the registers, 32 bytes per row per store).  A launch may
// cover a column range of a wider output (its row stride is then the full
// width).  Tiles are rasterised in groups of 8 tile-rows, and the
// workgroup index is remapped so that each XCD (workgroups are dealt
// round-robin over 8 XCDs) works on a contiguous range of tiles that share
// operands in its own L2.
#include <atomic>

#include "common.h"

namespace fp8lin {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

constexpr int kBK = 128;
constexpr int kGroupM = 8;
constexpr int kXcds = 8;
constexpr int kEpiFastAccum = 4;
constexpr int kOutDirect = 0, kOutF32Staged = 1;     // epilogue kinds (kernel template)

struct GemmParams {
    const uint8_t* a;
    const uint8_t* b;
    int64_t m, n, k;
    int64_t ldd;               // row stride (elements) of d, aux and residual; n unless a launch covers a column range
    const float* sinv_a;
    const float* sinv_b;
    const void* bias;
    void* d;
    void* aux;
    const void* residual;
    float* amax;
    const float* q_scale;      // FP8 copy of the output (bf16 outputs only): scale, codes, transposed codes
    uint8_t* q;
    uint8_t* qt;
    int32_t q_fmt;
    int32_t tiles_m, tiles_n;
    int32_t bias_dtype, d_dtype, epilogue;
};

// WM x WN waves, each owning MB x NB blocks of 32 x 32.
template <int WM, int WN, int MB, int NB>
struct TileCfg {
    static constexpr int WAVES = WM * WN;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int BM = WM * 32 * MB;
    static constexpr int BN = WN * 32 * NB;
    static constexpr int STAGE = (BM + BN) * kBK;           // LDS bytes per stage
    static constexpr int A_DMA = BM / 8 / WAVES;            // 1 KiB DMA wave-instructions per stage
    static constexpr int B_DMA = BN / 8 / WAVES;
};

// Byte offset of the 16-byte chunk `chunk` of LDS row `row`.  The LDS serves
// 16 lanes of a 16-byte read per cycle from 64 banks (256 bytes, two rows);
// swizzling by (row >> 1) & 7 puts the same logical chunk of 16 consecutive
// rows into 16 distinct bank groups.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * kBK + ((chunk ^ swz(row)) << 4); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Eight FP8 codes (k order) to eight f16 values, exactly.
template <int FMT>
__device__ __forceinline__ v8h dec8_f16(uint2 raw) {
    v2h a, b, c, d;
    if constexpr (FMT == kE4M3) {
        a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)raw.x, 1.0f, false);
        b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)raw.x, 1.0f, true);
        c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)raw.y, 1.0f, false);
        d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)raw.y, 1.0f, true);
    } else {
        a = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8((int)raw.x, 1.0f, false);
        b = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8((int)raw.x, 1.0f, true);
        c = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8((int)raw.y, 1.0f, false);
        d = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8((int)raw.y, 1.0f, true);
    }
    return v8h{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// One wave-instruction of the stage DMA: lane l's 16 bytes land at
// lds_base + 16 * l.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds_base, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_base, 16, off, 0, 0, 0);
}

// 4 x 4 byte transpose: a..d are four rows of four bytes; c0..c3 are the four
// columns (byte i of column j = byte j of row i).
__device__ __forceinline__ void transpose4x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t& c0,
                                             uint32_t& c1, uint32_t& c2, uint32_t& c3) {
    const uint32_t ab_lo = __builtin_amdgcn_perm(b, a, 0x05010400u);   // a0 b0 a1 b1
    const uint32_t ab_hi = __builtin_amdgcn_perm(b, a, 0x07030602u);   // a2 b2 a3 b3
    const uint32_t cd_lo = __builtin_amdgcn_perm(d, c, 0x05010400u);   // c0 d0 c1 d1
    const uint32_t cd_hi = __builtin_amdgcn_perm(d, c, 0x07030602u);   // c2 d2 c3 d3
    c0 = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u);             // a0 b0 c0 d0
    c1 = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u);
    c2 = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u);
    c3 = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u);
}

// MFMA format selector of an FP8 operand.
template <int FMT> struct MfmaFmt;
template <> struct MfmaFmt<kE4M3> { static constexpr int value = 0; };
template <> struct MfmaFmt<kE5M2> { static constexpr int value = 1; };

// Logical tile index of this workgroup: undo the round-robin XCD dealing,
// then raster in groups of kGroupM tile-rows.
__device__ __forceinline__ void tile_coords(int i, int32_t tiles_m, int32_t tiles_n, int& tm, int& tn) {
    const int nwg = tiles_m * tiles_n;
    const int q = nwg / kXcds, r = nwg % kXcds;
    const int xcd = i % kXcds, local = i / kXcds;
    const int pid = xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
    const int in_group = kGroupM * tiles_n;
    const int gid = pid / in_group;
    const int first_m = gid * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    const int rem = pid % in_group;
    tm = first_m + rem % gsize;
    tn = rem / gsize;
}

template <int WM, int WN, int MB, int NB, int AF, int BF, bool FAST, bool QOUT, int OUT>
__global__ void __launch_bounds__(64 * WM * WN, (WM * WN * MB * NB >= 64 ? (WM * WN) / 4 : 2))
k_gemm(GemmParams p) {
    using C = TileCfg<WM, WN, MB, NB>;
    // The two stages are separate arrays, and the k loop is unrolled by two so
    // that every LDS access names its stage statically: the compiler can then
    // see that the fragment reads of one stage never alias the DMA into the
    // other, and does not wait for that DMA before each read (the explicit
    // wait and barrier at the end of each stage order the two).
    __shared__ __attribute__((aligned(16))) uint8_t smem0[C::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t smem1[C::STAGE];
    __shared__ uint32_t red[C::WAVES];

    const int64_t M = p.m, N = p.n, K = p.k, LDD = p.ldd;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int g = lane >> 5, r32 = lane & 31;
    // Stage DMA: wave-instruction i of wave w fills rows 8 (w + W i) .. +7 (W =
    // waves per workgroup); lane l lands at physical chunk l % 8 of row
    // row = 8 (w + W i) + l / 8, i.e. it loads logical chunk (l % 8) ^ swz(row).
    const int lrow = lane >> 3, lpc = lane & 7;
    constexpr int NDMA = C::A_DMA + C::B_DMA;
    const int nk = (int)((K + kBK - 1) / kBK);
    const int ntiles = p.tiles_m * p.tiles_n;
    const float sc = (*p.sinv_a) * (*p.sinv_b);
    uint32_t amax = 0;

    // Persistent: each workgroup takes tiles blockIdx.x, + gridDim.x, ....
    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    int tm, tn;
    tile_coords(tile, p.tiles_m, p.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;

    // Buffer resources over this tile's rows of A and B.
    const uint32_t rows_a = (uint32_t)min<int64_t>(C::BM, M - m0), rows_b = (uint32_t)min<int64_t>(C::BN, N - n0);
    const __amdgpu_buffer_rsrc_t ra_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.a + m0 * K), (short)0, (int)(rows_a * (uint32_t)K), 0x00020000);
    const __amdgpu_buffer_rsrc_t rb_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.b + n0 * K), (short)0, (int)(rows_b * (uint32_t)K), 0x00020000);

    // DMA wave-instruction q of a stage: q < A_DMA fills A rows, the rest B rows.
    auto dma_part = [&](int kt, uint8_t* sa, int q0, int q1) {
        uint8_t* sb = sa + C::BM * kBK;
        const uint32_t k0 = (uint32_t)kt * kBK;
#pragma unroll
        for (int q = 0; q < C::A_DMA + C::B_DMA; ++q) {
            if (q < q0 || q >= q1) continue;
            const bool is_a = q < C::A_DMA;
            const int i = is_a ? q : q - C::A_DMA;
            const int row = 8 * (wave + C::WAVES * i) + lrow;
            const uint32_t kb = k0 + (uint32_t)((lpc ^ swz(row)) << 4);
            const uint32_t off = (uint32_t)row * (uint32_t)K + kb;
            dma16(is_a ? ra_rsrc : rb_rsrc, (is_a ? sa : sb) + (row - lrow) * kBK,
                  kb < (uint32_t)K ? off : 0x80000000u);
        }
    };
    // The next stage's DMA during the k loop.  On the FP8-MFMA path with eight
    // waves, waves w and w ^ 4 share a SIMD; in each stage one of them issues
    // both waves' DMA wave-instructions (alternating by stage) while the other
    // goes straight on to its fragment reads and MFMAs, so one wave keeps the
    // SIMD's matrix core fed while the other waits to issue into a backed-up
    // memory pipeline (every GEMM 1-2 % faster, same data in the same
    // LDS places; on the exact path, whose converts already fill the other
    // wave's time, it measured 1-2 % slower, so that path keeps every wave
    // issuing its own share).  The pair's rows are those of wave
    // w & 3 and the same rows + 32 (the swizzle repeats every 16 rows), so the
    // second offset is the first + 32 K; every offset stays in the vector
    // offset, which the buffer range check covers (a k-tail lane's 2^31 + 32 K
    // is past every tile's rows * K and below 2^32, since K < 2^23).
    auto dma_stage = [&](int kt, uint8_t* sa) {
        if constexpr (FAST && C::WAVES == 8) {
            static_assert(C::A_DMA * 8 * C::WAVES == C::BM && C::B_DMA * 8 * C::WAVES == C::BN, "DMA row layout");
            if (((wave >> 2) ^ (kt & 1)) != 0) return;
            const int wb = wave & 3;
            const uint32_t dk = 32u * (uint32_t)K;
            uint8_t* sb = sa + C::BM * kBK;
            const uint32_t k0 = (uint32_t)kt * kBK;
#pragma unroll
            for (int q = 0; q < NDMA; ++q) {
                const bool is_a = q < C::A_DMA;
                const int i = is_a ? q : q - C::A_DMA;
                const int row = 8 * (wb + C::WAVES * i) + lrow;
                const uint32_t kb = k0 + (uint32_t)((lpc ^ swz(row)) << 4);
                const uint32_t off = kb < (uint32_t)K ? (uint32_t)row * (uint32_t)K + kb : 0x80000000u;
                uint8_t* dst = (is_a ? sa : sb) + (row - lrow) * kBK;
                const __amdgpu_buffer_rsrc_t r = is_a ? ra_rsrc : rb_rsrc;
                dma16(r, dst, off);
                dma16(r, dst + 32 * kBK, off + dk);
            }
        } else {
            dma_part(kt, sa, 0, NDMA);
        }
    };

    v16f acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    if (nk > 0) {
        dma_part(0, smem0, 0, NDMA);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    // One stage: multiply the tile in `cur` while the DMA of stage kt + 1 fills `nxt`.
    auto stage_step = [&](int kt, const uint8_t* cur, uint8_t* nxt) {
        // the next stage's DMA is issued all at once at the start of the stage
        // (the fragment reads of this stage do not wait for it)
        const bool more = kt + 1 < nk;
        const uint8_t* sa = cur;
        const uint8_t* sb = sa + C::BM * kBK;
        if constexpr (FAST) {
            // 64-k blocks: lane group g holds k = 64 kb + 32 g .. +31 (chunks 4 kb + 2 g, +1).
            // The fragments of a block are read right before its MFMAs (no
            // register prefetch of the next block: the second wave on the SIMD
            // covers the LDS latency, and the registers are not there to spare).
#pragma unroll
            for (int kb = 0; kb < kBK / 64; ++kb) {
                const int c0 = kb * 4 + g * 2;
                v8i af[MB], bf[NB];
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    const int row = wm * MB * 32 + i * 32 + r32;
                    const uint4 lo = *reinterpret_cast<const uint4*>(sa + lds_off(row, c0));
                    const uint4 hi = *reinterpret_cast<const uint4*>(sa + lds_off(row, c0 + 1));
                    af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                }
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int row = wn * NB * 32 + j * 32 + r32;
                    const uint4 lo = *reinterpret_cast<const uint4*>(sb + lds_off(row, c0));
                    const uint4 hi = *reinterpret_cast<const uint4*>(sb + lds_off(row, c0 + 1));
                    bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                }
                if (more && kb == 0) dma_stage(kt + 1, nxt);
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            bf[j], af[i], acc[i][j], MfmaFmt<BF>::value, MfmaFmt<AF>::value, 0, 0, 0, 0);
            }
        } else {
            // 32-k blocks: lane group g holds k = 32 kb + 16 g .. +15 (chunk 2 kb + g);
            // bytes 0-7 feed the first f16 MFMA ("h1"), bytes 8-15 the second ("h2").
            // Software pipeline: the h2 converts of block kb run beside its h1
            // MFMAs, and the h1 converts of block kb + 1 beside its h2 MFMAs, so
            // a wave keeps the matrix core and the VALU busy at the same time.
            uint4 ar[MB], br[NB];
            v8h a0[MB], a1[MB], b0[NB], b1[NB];
            auto rd = [&](int kb) {
                const int c = kb * 2 + g;
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    ar[i] = *reinterpret_cast<const uint4*>(sa + lds_off(wm * MB * 32 + i * 32 + r32, c));
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    br[j] = *reinterpret_cast<const uint4*>(sb + lds_off(wn * NB * 32 + j * 32 + r32, c));
            };
            auto cvt_h1 = [&]() {
#pragma unroll
                for (int i = 0; i < MB; ++i) a0[i] = dec8_f16<AF>(make_uint2(ar[i].x, ar[i].y));
#pragma unroll
                for (int j = 0; j < NB; ++j) b0[j] = dec8_f16<BF>(make_uint2(br[j].x, br[j].y));
            };
            auto cvt_h2 = [&]() {
#pragma unroll
                for (int i = 0; i < MB; ++i) a1[i] = dec8_f16<AF>(make_uint2(ar[i].z, ar[i].w));
#pragma unroll
                for (int j = 0; j < NB; ++j) b1[j] = dec8_f16<BF>(make_uint2(br[j].z, br[j].w));
            };
            constexpr int NMF = MB * NB;              // MFMAs per half block
            constexpr int NCV = 4 * (MB + NB);        // converts per half block
            rd(0);
            cvt_h1();
#pragma unroll
            for (int kb = 0; kb < kBK / 32; ++kb) {
                cvt_h2();
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0[j], a0[i], acc[i][j], 0, 0, 0);
                // one MFMA, then a share of the converts, repeated
#pragma unroll
                for (int q = 0; q < NMF; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, (NCV + NMF - 1) / NMF, 0);
                }
                if (more && kb == 0) dma_stage(kt + 1, nxt);
                if (kb + 1 < kBK / 32) {
                    rd(kb + 1);
                    cvt_h1();
                }
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b1[j], a1[i], acc[i][j], 0, 0, 0);
                if (kb + 1 < kBK / 32) {
                    // the next block's fragment reads first, two MFMAs to cover
                    // their latency, then MFMAs and its h1 converts interleaved
                    __builtin_amdgcn_sched_group_barrier(0x100, MB + NB, 1);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
#pragma unroll
                    for (int q = 2; q < NMF; ++q) {
                        __builtin_amdgcn_sched_group_barrier(0x002, (NCV + NMF - 3) / (NMF - 2), 1);
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                    }
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    for (int kt = 0; kt < nk; kt += 2) {
        stage_step(kt, smem0, smem1);
        if (kt + 1 < nk) stage_step(kt + 1, smem1, smem0);
    }

    // ---------------------------------------------------------------- epilogue
    // The epilogue's lane indices come from an opaque copy of the thread index
    // made inside the tile loop: otherwise the compiler hoists the epilogue's
    // per-lane LDS addresses out of the tile loop, where they stay live across
    // the k loop and are spilled to scratch (one reload per store, each
    // followed by a wait for all of the wave's memory operations).
    int te = t;
    asm volatile("" : "+v"(te));
    const int lane_e = te & 63, r32e = lane_e & 31, ge = lane_e >> 5;
    // y = acc * sinv_a * sinv_b + bias, in place.  Lane (r32e, ge) of block (i, j)
    // holds row i * 32 + r32e and, for q4 = 0..3, the four columns
    // j * 32 + 8 q4 + 4 ge .. + 3 of its wave's sub-tile.
    const bool gelu = p.epilogue & 1, accum = p.epilogue & 2;
    const bool want_amax = p.amax != nullptr;      // the output amax costs VALU work per element
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int64_t ncol = n0 + wn * NB * 32 + j * 32 + 8 * q4 + 4 * ge;
            float b[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (p.bias && ncol < N) {
                if (p.bias_dtype == kF32) {
                    const float4 bv = *reinterpret_cast<const float4*>(static_cast<const float*>(p.bias) + ncol);
                    b[0] = bv.x; b[1] = bv.y; b[2] = bv.z; b[3] = bv.w;
                } else {
                    const uint2 bv = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.bias) + ncol);
                    b[0] = bf16_to_f32(bv.x & 0xFFFFu); b[1] = bf16_to_f32(bv.x >> 16);
                    b[2] = bf16_to_f32(bv.y & 0xFFFFu); b[3] = bf16_to_f32(bv.y >> 16);
                }
            }
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][4 * q4 + e] = acc[i][j][4 * q4 + e] * sc + b[e];
        }
    }

    if (OUT == kOutDirect && p.d_dtype == kBF16) {     // (OUT folds at compile time)
        // bf16 outputs go through LDS (free after the k loop) so that the global
        // stores write whole row segments: rows of the wave-row wm go to stage
        // array wm, BN * 2 bytes per row, 8-byte units XOR-swizzled by row.
        // The stores are non-temporal: all workgroups store a tile at about
        // the same time, and the burst drained that way measured 5-14 %
        // faster on the fast path's bf16-output GEMMs (1-3 % on the exact
        // path's), outputs unchanged.
        static_assert(WM == 2 && (C::BM / 2) * C::BN * 2 <= C::STAGE, "bf16 staging must fit one stage array");
        constexpr int UPR = C::BN / 4;                  // 8-byte units per LDS row
        auto lds_unit = [&](int lr, int unit) { return lr * (C::BN * 2) + ((unit ^ (((lr & 15) << 1) & (UPR - 1))) << 3); };
        uint8_t* const half = wm == 0 ? smem0 : smem1;
        auto stage_store = [&](void* dst) {
            __syncthreads();
            constexpr int CPR = C::BN / 8;              // 16-byte chunks per row
            constexpr int RPP = C::THREADS / CPR;       // rows per pass
            constexpr int NPASS = C::BM / RPP, NH = NPASS / 2;
            static_assert(NPASS % 2 == 0 && RPP % 16 == 0, "passes split over the two stage arrays");
            const int c = te % CPR, r0 = te / CPR;
            // Every LDS read of the thread first (rows r0 + RPP pass: the
            // first half from stage array 0, the second from array 1, at
            // constant offsets from one address), one wait, then the stores.
            v4u v[NPASS];
#pragma unroll
            for (int pass = 0; pass < NPASS; ++pass)
                v[pass] = *reinterpret_cast<const v4u*>((pass < NH ? smem0 : smem1) +
                                                        lds_unit(r0 + RPP * (pass % NH), 2 * c));
            // (the reads stay here, not sunk into the conditional stores)
#pragma unroll
            for (int pass = 0; pass < NPASS; ++pass) asm volatile("" : "+v"(v[pass]));
            const int64_t col = n0 + 8 * c;
            uint16_t* const out = static_cast<uint16_t*>(dst) + (m0 + r0) * LDD + col;
#pragma unroll
            for (int pass = 0; pass < NPASS; ++pass)
                if (m0 + r0 + RPP * pass < M && col < N)
                    __builtin_nontemporal_store(v[pass], reinterpret_cast<v4u*>(out + (int64_t)(RPP * pass) * LDD));
            __syncthreads();
        };
        if (gelu && p.aux) {
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int lr = i * 32 + r32e;
                        const int unit = (wn * NB * 32 + j * 32 + 8 * q4 + 4 * ge) / 4;
                        *reinterpret_cast<uint2*>(half + lds_unit(lr, unit)) =
                            make_uint2(pack_bf16x2(acc[i][j][4 * q4], acc[i][j][4 * q4 + 1]),
                                       pack_bf16x2(acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]));
                    }
            stage_store(p.aux);
        }
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const int64_t mrow = m0 + wm * MB * 32 + i * 32 + r32e;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int64_t ncol = n0 + wn * NB * 32 + j * 32 + 8 * q4 + 4 * ge;
                    const bool inside = mrow < M && ncol < N;
                    float y[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = gelu ? gelu_f32(acc[i][j][4 * q4 + e]) : acc[i][j][4 * q4 + e];
                    if (p.residual && inside) {
                        const uint2 rv =
                            *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.residual) + mrow * LDD + ncol);
                        y[0] += bf16_to_f32(rv.x & 0xFFFFu); y[1] += bf16_to_f32(rv.x >> 16);
                        y[2] += bf16_to_f32(rv.y & 0xFFFFu); y[3] += bf16_to_f32(rv.y >> 16);
                    }
                    const uint2 o = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
                    if (want_amax && inside)
                        amax = max(amax, max(max(abs_bits(bf16_to_f32(o.x & 0xFFFFu)), abs_bits(bf16_to_f32(o.x >> 16))),
                                             max(abs_bits(bf16_to_f32(o.y & 0xFFFFu)), abs_bits(bf16_to_f32(o.y >> 16)))));
                    const int unit = (wn * NB * 32 + j * 32 + 8 * q4 + 4 * ge) / 4;
                    *reinterpret_cast<uint2*>(half + lds_unit(i * 32 + r32e, unit)) = o;
                }
            }
        }
        if constexpr (!QOUT) {
            stage_store(p.d);
        } else {
            // The output as written (bf16) is also cast to FP8 with the scale of the
            // tensor it becomes: codes = enc(fl32(bf16 value * scale)), the same
            // arithmetic as a separate cast of d.  The bf16 values and the row-major
            // codes are stored straight from the staged values (non-temporal, whole
            // row segments, as the other staged outputs); for the transposed codes each
            // segment of SEG rows goes through a byte tile in an LDS region of its
            // own (16 KiB; 4-byte words XOR-swizzled by an even function of the
            // row, so 8-byte pairs stay together) and 4 x 4 byte transposes, as in
            // the cast-transpose kernel.
            constexpr int CPR = C::BN / 8;              // 16-byte bf16 chunks (8 values) per row
            constexpr int RPP = C::THREADS / CPR;       // rows per pass
            constexpr int HALF = C::BM / 2;
            constexpr int SEG = (16384 / C::BN) < HALF ? (16384 / C::BN) : HALF;
            constexpr int NPASS = SEG / RPP;            // passes per segment
            constexpr int WPR = C::BN / 4;              // 4-byte words per code row
            static_assert(SEG % RPP == 0 && SEG % 16 == 0 && HALF % SEG == 0, "code segment layout");
            __shared__ __attribute__((aligned(16))) uint8_t codes[SEG * C::BN];
            auto code_word = [&](int r, int w) { return r * C::BN + ((w ^ (((r >> 4) << 1) & (WPR - 1))) << 2); };
            const float qs = *p.q_scale;
            const int c = te % CPR;
            __syncthreads();
#pragma unroll
            for (int sg = 0; sg < C::BM / SEG; ++sg) {
#pragma unroll
                for (int pass = 0; pass < NPASS; ++pass) {
                    const int lr = te / CPR + RPP * pass;        // row within the segment
                    const int r = sg * SEG + lr;
                    const uint4 v = *reinterpret_cast<const uint4*>((r < HALF ? smem0 : smem1) + lds_unit(r % HALF, 2 * c));
                    const int64_t row = m0 + r, col = n0 + 8 * c;
                    const bool inside = row < M && col < N;
                    if (p.d && inside)
                        __builtin_nontemporal_store(__builtin_bit_cast(v4u, v),
                                                    reinterpret_cast<v4u*>(static_cast<uint16_t*>(p.d) + row * LDD + col));
                    const float f[8] = {bf16_to_f32(v.x & 0xFFFFu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xFFFFu),
                                        bf16_to_f32(v.y >> 16),     bf16_to_f32(v.z & 0xFFFFu), bf16_to_f32(v.z >> 16),
                                        bf16_to_f32(v.w & 0xFFFFu), bf16_to_f32(v.w >> 16)};
                    const uint2 q8 = p.q_fmt == kE4M3
                        ? make_uint2(enc4<kE4M3>(f[0] * qs, f[1] * qs, f[2] * qs, f[3] * qs),
                                     enc4<kE4M3>(f[4] * qs, f[5] * qs, f[6] * qs, f[7] * qs))
                        : make_uint2(enc4<kE5M2>(f[0] * qs, f[1] * qs, f[2] * qs, f[3] * qs),
                                     enc4<kE5M2>(f[4] * qs, f[5] * qs, f[6] * qs, f[7] * qs));
                    if (p.q && inside) __builtin_nontemporal_store(__builtin_bit_cast(v2u, q8), reinterpret_cast<v2u*>(p.q + row * N + col));
                    if (p.qt) *reinterpret_cast<uint2*>(codes + code_word(lr, 2 * c)) = q8;
                }
                if (p.qt) {
                    __syncthreads();
                    constexpr int STRIPS = SEG / 16;
                    for (int u = te; u < WPR * STRIPS; u += C::THREADS) {
                        const int cg = u / STRIPS, strip = u % STRIPS;
                        uint32_t w[16];
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            w[i] = *reinterpret_cast<const uint32_t*>(codes + code_word(strip * 16 + i, cg));
                        uint32_t o4[4][4];
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk)
                            transpose4x4(w[4 * kk], w[4 * kk + 1], w[4 * kk + 2], w[4 * kk + 3], o4[0][kk], o4[1][kk],
                                         o4[2][kk], o4[3][kk]);
                        const int64_t ocol = m0 + sg * SEG + strip * 16;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int64_t orow = n0 + 4 * cg + j;
                            if (orow < N && ocol < M)
                                *reinterpret_cast<uint4*>(p.qt + orow * M + ocol) =
                                    make_uint4(o4[j][0], o4[j][1], o4[j][2], o4[j][3]);
                        }
                    }
                    __syncthreads();       // the code tile is rewritten by the next segment
                }
            }
            __syncthreads();               // the staged values are read; the next tile may DMA
        }
    } else if (OUT == kOutF32Staged) {
        // fp32 outputs go through LDS as well (written from registers, each
        // wave store would put 32 bytes into each of 32 rows).  One wave-row
        // (BM / 2 rows) per pass, its rows split over the two stage arrays,
        // 1 KiB per row for BN = 256, 16-byte units XOR-swizzled by the row's
        // low 4 bits; then the whole workgroup applies the residual and the
        // accumulate in the same order as the register path and writes
        // complete row segments with non-temporal stores.  Never launched with
        // GeLU.
        static_assert(WM == 2 && (C::BM / 4) * C::BN * 4 <= C::STAGE && C::BN >= 64, "fp32 staging layout");
        constexpr int UPR = C::BN / 4;                  // 16-byte units (4 floats) per row
        constexpr int QR = C::BM / 4;                   // rows per stage array in one pass
        constexpr int RPP = C::THREADS / UPR;           // rows per store step
        auto f32_unit = [&](int lr, int unit) {
            return (lr < QR ? smem0 : smem1) + (lr % QR) * (C::BN * 4) + ((unit ^ (lr & 15)) << 4);
        };
        const int c = te % UPR;
#pragma unroll
        for (int pass = 0; pass < WM; ++pass) {
            __syncthreads();
            if (wm == pass) {
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int j = 0; j < NB; ++j)
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4)
                            *reinterpret_cast<float4*>(f32_unit(i * 32 + r32e, (wn * NB * 32 + j * 32 + 8 * q4 + 4 * ge) / 4)) =
                                make_float4(acc[i][j][4 * q4], acc[i][j][4 * q4 + 1], acc[i][j][4 * q4 + 2],
                                            acc[i][j][4 * q4 + 3]);
            }
            __syncthreads();
#pragma unroll
            for (int st = 0; st < (C::BM / 2) / RPP; ++st) {
                const int lr = te / UPR + RPP * st;
                const int64_t mrow = m0 + pass * (C::BM / 2) + lr, ncol = n0 + 4 * c;
                if (mrow >= M || ncol >= N) continue;
                const float4 v = *reinterpret_cast<const float4*>(f32_unit(lr, c));
                float y[4] = {v.x, v.y, v.z, v.w};
                const int64_t off = mrow * LDD + ncol;
                if (p.residual) {
                    const float4 rv = *reinterpret_cast<const float4*>(static_cast<const float*>(p.residual) + off);
                    y[0] += rv.x; y[1] += rv.y; y[2] += rv.z; y[3] += rv.w;
                }
                float4* dp = reinterpret_cast<float4*>(static_cast<float*>(p.d) + off);
                if (accum) {
                    const float4 old = *dp;
                    y[0] = old.x + y[0]; y[1] = old.y + y[1]; y[2] = old.z + y[2]; y[3] = old.w + y[3];
                }
                __builtin_nontemporal_store(v4f{y[0], y[1], y[2], y[3]}, reinterpret_cast<v4f*>(dp));
                if (want_amax)
                    amax = max(amax, max(max(abs_bits(y[0]), abs_bits(y[1])), max(abs_bits(y[2]), abs_bits(y[3]))));
            }
        }
        __syncthreads();     // the next tile's DMA rewrites the LDS
    } else {
        // fp32 outputs from registers: lane (r32e, ge) writes four consecutive
        // columns of its row per 32 x 32 block.
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const int64_t mrow = m0 + wm * MB * 32 + i * 32 + r32e;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int64_t ncol = n0 + wn * NB * 32 + j * 32 + 8 * q4 + 4 * ge;
                    if (mrow >= M || ncol >= N) continue;
                    float y[4];
                    const int64_t off = mrow * LDD + ncol;
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = acc[i][j][4 * q4 + e];
                    if (gelu) {
                        if (p.aux)
                            *reinterpret_cast<float4*>(static_cast<float*>(p.aux) + off) = make_float4(y[0], y[1], y[2], y[3]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[e] = gelu_f32(y[e]);
                    }
                    if (p.residual) {
                        const float4 rv = *reinterpret_cast<const float4*>(static_cast<const float*>(p.residual) + off);
                        y[0] += rv.x; y[1] += rv.y; y[2] += rv.z; y[3] += rv.w;
                    }
                    float4* dp = reinterpret_cast<float4*>(static_cast<float*>(p.d) + off);
                    if (accum) {
                        const float4 old = *dp;
                        y[0] = old.x + y[0]; y[1] = old.y + y[1]; y[2] = old.z + y[2]; y[3] = old.w + y[3];
                    }
                    *dp = make_float4(y[0], y[1], y[2], y[3]);
                    if (want_amax)
                        amax = max(amax, max(max(abs_bits(y[0]), abs_bits(y[1])), max(abs_bits(y[2]), abs_bits(y[3]))));
                }
            }
        }
        __syncthreads();     // the next tile's DMA rewrites the LDS
    }
    }   // tile loop
    if (p.amax) block_amax_merge(amax, p.amax, red);
}


template <typename Kern>
int resident_per_cu(Kern kern, int threads) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, threads, 0) != hipSuccess || n < 1) n = 1;
    return n;
}

template <int WM, int WN, int MB, int NB, int AF, int BF, bool FAST, bool QOUT, int OUT>
hipError_t launch_out(const GemmParams& p, hipStream_t s) {
    using C = TileCfg<WM, WN, MB, NB>;
    static const int per_cu = resident_per_cu(k_gemm<WM, WN, MB, NB, AF, BF, FAST, QOUT, OUT>, C::THREADS);
    // One resident wave of workgroups, each looping over tiles; a multiple of
    // 8 so that every workgroup stays on the same XCD's tile range.
    const int64_t ntiles = (int64_t)p.tiles_m * p.tiles_n;
    int64_t grid = (int64_t)cu_count() * per_cu;
    if (grid >= 8) grid -= grid % 8;
    if (grid > ntiles) grid = ntiles;
    hipLaunchKernelGGL((k_gemm<WM, WN, MB, NB, AF, BF, FAST, QOUT, OUT>), dim3((unsigned)grid), dim3(C::THREADS), 0, s,
                       p);
    return hipGetLastError();
}

// The staged fp32 epilogue is an instance of its own: with it in the same
// kernel as the bf16 and register fp32 epilogues, the register allocation of
// the whole kernel changed (37 spilled registers instead of 14 on the exact
// path) and bf16-output GEMMs measured 2-5% slower.  Every fp32 output without
// GeLU takes it: its whole-row, non-temporal stores measured 8-17 % faster on
// the fast path's weight gradients and 1.5-3 % on the exact path's, against
// the register path's 32-byte pieces (which non-temporal stores make slower
// still: partial lines then miss the L2's write combining).
template <int WM, int WN, int MB, int NB, int AF, int BF, bool FAST, bool QOUT = false>
hipError_t launch_fmt(const GemmParams& p, hipStream_t s) {
    if constexpr (QOUT) {
        return launch_out<WM, WN, MB, NB, AF, BF, FAST, true, kOutDirect>(p, s);     // bf16 outputs only
    } else {
        if (p.d_dtype == kF32 && !(p.epilogue & 1))
            return launch_out<WM, WN, MB, NB, AF, BF, FAST, false, kOutF32Staged>(p, s);
        return launch_out<WM, WN, MB, NB, AF, BF, FAST, false, kOutDirect>(p, s);
    }
}

template <int WM, int WN, int MB, int NB, bool FAST>
hipError_t launch_cfg(const GemmParams& base, int afmt, int bfmt, hipStream_t s) {
    using C = TileCfg<WM, WN, MB, NB>;
    GemmParams p = base;
    p.tiles_m = (int32_t)((p.m + C::BM - 1) / C::BM);
    p.tiles_n = (int32_t)((p.n + C::BN - 1) / C::BN);
    // the FP8 copy of the output is built for the forward GEMMs (E4M3 x E4M3) only
    if (p.q_scale) return launch_fmt<WM, WN, MB, NB, kE4M3, kE4M3, FAST, true>(p, s);
    if (afmt == kE4M3 && bfmt == kE4M3) return launch_fmt<WM, WN, MB, NB, kE4M3, kE4M3, FAST>(p, s);
    if (afmt == kE5M2 && bfmt == kE4M3) return launch_fmt<WM, WN, MB, NB, kE5M2, kE4M3, FAST>(p, s);
    if (afmt == kE4M3) return launch_fmt<WM, WN, MB, NB, kE4M3, kE5M2, FAST>(p, s);
    return launch_fmt<WM, WN, MB, NB, kE5M2, kE5M2, FAST>(p, s);
}

// Workgroups of one resident wave of the 256 x 256 configuration.
template <bool FAST>
int64_t big_grid() {
    using C = TileCfg<2, 4, 4, 2>;
    static const int per_cu = resident_per_cu(k_gemm<2, 4, 4, 2, kE4M3, kE4M3, FAST, false, kOutDirect>, C::THREADS);
    int64_t grid = (int64_t)cu_count() * per_cu;
    if (grid >= 8) grid -= grid % 8;
    return grid;
}

template <bool FAST>
hipError_t launch_path(const GemmParams& p, int afmt, int bfmt, hipStream_t s) {
    // Tile choice: 256 x 256 when that still gives every CU work, else smaller
    // tiles.  At 256 x 256 both paths run 8 waves (2 per SIMD, 128 x 64 each)
    // so one wave's LDS reads and converts overlap the other's MFMAs; 128 x 128
    // per wave would need 256 accumulator registers, which the persistent
    // loop's state no longer leaves room for.
    const int64_t tm = (p.m + 255) / 256, tn = (p.n + 255) / 256;
    const int64_t big = tm * tn;
    const int64_t mid = ((p.m + 127) / 128) * ((p.n + 127) / 128);
    if (big >= 256) {
        // A last round at most half full (e.g. 896 tiles on 256 workgroups)
        // leaves CUs idle: the tile rows of the full rounds run on 256 x 256
        // tiles, the remaining rows (at most 8 tile rows) on 128 x 128 tiles,
        // four times as many, in a second launch.  Every output element is
        // computed exactly as in one launch (same k order); the output amax is
        // merged by both.  Not for the FP8-output epilogue (its codes are
        // indexed by the full M and N).
        const int64_t grid = big_grid<FAST>();
        const int64_t rem = big % grid;
        if (rem != 0 && rem <= grid / 2 && !p.q_scale) {
            const int64_t esz = p.d_dtype == kF32 ? 4 : 2;
            int64_t tm1 = tm - 1;
            while (tm1 > 0 && (tm1 * tn) % grid != 0) --tm1;
            if (tm1 > 0 && tm - tm1 <= 8) {
                const int64_t r0 = tm1 * 256;
                GemmParams top = p, rest = p;
                top.m = r0;
                rest.m = p.m - r0;
                rest.a = p.a + r0 * p.k;
                rest.d = static_cast<uint8_t*>(p.d) + r0 * p.ldd * esz;
                if (p.aux) rest.aux = static_cast<uint8_t*>(p.aux) + r0 * p.ldd * esz;
                if (p.residual) rest.residual = static_cast<const uint8_t*>(p.residual) + r0 * p.ldd * esz;
                const hipError_t e = launch_cfg<2, 4, 4, 2, FAST>(top, afmt, bfmt, s);
                if (e != hipSuccess) return e;
                return launch_cfg<2, 2, 2, 2, FAST>(rest, afmt, bfmt, s);
            }
            // A wide output (e.g. 4096 x 14336) splits by columns instead: the
            // first tile columns on 256 x 256 tiles, the last (at most 8) on
            // 128 x 128 tiles, both writing into the full-width output through
            // its row stride.
            int64_t tn1 = tn - 1;
            while (tn1 > 0 && (tm * tn1) % grid != 0) --tn1;
            if (tn1 > 0 && tn - tn1 <= 8) {
                const int64_t c0 = tn1 * 256;
                const int64_t bsz = p.bias_dtype == kF32 ? 4 : 2;
                GemmParams left = p, right = p;
                left.n = c0;
                right.n = p.n - c0;
                right.b = p.b + c0 * p.k;
                if (p.bias) right.bias = static_cast<const uint8_t*>(p.bias) + c0 * bsz;
                right.d = static_cast<uint8_t*>(p.d) + c0 * esz;
                if (p.aux) right.aux = static_cast<uint8_t*>(p.aux) + c0 * esz;
                if (p.residual) right.residual = static_cast<const uint8_t*>(p.residual) + c0 * esz;
                const hipError_t e = launch_cfg<2, 4, 4, 2, FAST>(left, afmt, bfmt, s);
                if (e != hipSuccess) return e;
                return launch_cfg<2, 2, 2, 2, FAST>(right, afmt, bfmt, s);
            }
        }
        return launch_cfg<2, 4, 4, 2, FAST>(p, afmt, bfmt, s);
    }
    if (mid >= 256) return launch_cfg<2, 2, 2, 2, FAST>(p, afmt, bfmt, s);
    return launch_cfg<2, 2, 1, 1, FAST>(p, afmt, bfmt, s);
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a, int afmt, const uint8_t* b, int bfmt, int64_t m, int64_t n, int64_t k,
                       const float* sinv_a, const float* sinv_b, const void* bias, int bias_dtype, int epilogue,
                       void* d, int d_dtype, void* aux, const void* residual, float* amax, const float* q_scale,
                       uint8_t* q, uint8_t* qt, int q_fmt, hipStream_t s) {
    if (m == 0 || n == 0) return hipSuccess;
    GemmParams p{};
    p.a = a; p.b = b; p.m = m; p.n = n; p.k = k; p.ldd = n;
    p.sinv_a = sinv_a; p.sinv_b = sinv_b; p.bias = bias; p.d = d; p.aux = aux; p.residual = residual; p.amax = amax;
    p.q_scale = q_scale; p.q = q; p.qt = qt; p.q_fmt = q_fmt;
    p.bias_dtype = bias_dtype; p.d_dtype = d_dtype; p.epilogue = epilogue;
    timing_before(kKindGemm, s);
    const hipError_t e = (epilogue & kEpiFastAccum) ? launch_path<true>(p, afmt, bfmt, s)
                                                    : launch_path<false>(p, afmt, bfmt, s);
    timing_after(s);
    return e;
}

}  // namespace fp8lin
