// Fused amax + cast + transpose (+ bias-gradient partial sums, + GeLU backward).
//
// Pages (titles in include/fp8lin.h): [TE-KR] "FP8 자동변환(Autocasting)"
// (cast, amax and factor in one step) and "Backward Pass 처리" (the backward
// GEMMs consume the FP8 copies made here); [PT-VI] torch._scaled_mm example
// (the second GEMM operand enters transposed).
//
// One workgroup (256 threads, 4 waves) owns a 128 x 128 tile of the
// [rows][cols] input and loops over tiles; the grid is one resident round of
// workgroups (the occupancy the compiled kernel allows, times the CU count),
// so the amax merge costs one, usually skipped, atomic per workgroup.
//
// Load phase: the tile is read as 16-byte vectors (8 bf16 or 4 fp32
// elements); thread t owns vector column t % V of rows t / V + (256 / V) p
// (V vectors per tile row), so each load instruction of a wave covers whole
// 256- or 512-byte row segments.  Every access is a buffer access relative to
// the tile with 32-bit offsets, bounded by the tile (out-of-range lanes load
// zeros and drop their stores), so the loads carry no branches: every load of
// the tile (and of z for the GeLU backward) is issued before any is used, and
// each vector is encoded as soon as its own load has returned.  Each vector's
// codes go to q with one 8- or 4-byte store and to an LDS tile [128][128]
// bytes.
//
// Transpose phase: thread t owns input columns 4 cg .. 4 cg + 3 (cg = t / 8)
// of the 16-row strip s = t % 8: it reads one 4-byte LDS word from each of the
// strip's 16 rows, transposes the 16 x 4 bytes with byte permutes (4 x 4
// blocks, 8 permutes each) and writes four 16-byte vectors, one to each of
// the four q_t rows; the 8 lanes of a column group write the 128 contiguous
// bytes the tile contributes to a q_t row.  LDS word w of row r is stored at
// word w ^ (((r >> 5) & 3) << 3), which spreads the four strips a half-wave
// reads over distinct banks.
//
// Rows and cols are multiples of 16, so a 16-row strip or a 4-column group is
// either entirely inside the tensor or entirely outside.
//
// The GeLU-backward variant on bf16 input is bound by the arithmetic of
// gelu'(z), not by memory; since z is a bf16 value, each workgroup tabulates
// gelu' for the 3072 bf16 patterns with 2^-8 <= |z| < 16 in LDS once (same
// function, so a lookup is bit-identical to computing it) and computes it only
// for the others (measured 8192 x 14336: about 10% faster).
//
// The dual-format variant encodes every element with two scales, to E4M3 and
// to E5M2, from one read of the input: four outputs (both formats, both
// layouts) through two LDS tiles, and one amax for both tensors' metas.
#include <mutex>

#include "common.h"

namespace fp8lin {
namespace {

constexpr int kTile = 128;
constexpr int kThreads = 256;

constexpr int kGeluExpLo = 119, kGeluExps = 12;                  // bf16 exponent fields of the gelu' table
constexpr int kGeluTabHalf = kGeluExps * 128, kGeluTabN = 2 * kGeluTabHalf;

// Buffer accesses (raw, unswizzled): an access whose offset is at or past the
// resource's num_records loads zeros or stores nothing.
constexpr uint32_t kOob = 0x80000000u;       // an offset past every bound in use (all below 2^31)
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)num_bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}

template <int DT> struct CtVec {
    static constexpr int E = DT == kF32 ? 4 : 8;       // elements per 16-byte vector
    static constexpr int V = kTile / E;                // vectors per tile row
    static constexpr int RS = kThreads / V;            // rows between a thread's vectors
    static constexpr int NP = kTile / RS;              // vectors per thread
};

// The elements of one 16-byte vector as fp32.
template <int DT>
__device__ __forceinline__ void unpack_vec(uint4 w, float v[CtVec<DT>::E]) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    if constexpr (DT == kF32) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = __uint_as_float(u[j]);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(u[j] << 16);
            v[2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
        }
    }
}

template <int DT>
__device__ __forceinline__ uint4 pack_vec(const float v[CtVec<DT>::E]) {
    if constexpr (DT == kF32)
        return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
    else
        return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                          pack_bf16x2(v[6], v[7]));
}

// Codes of one vector: 4 codes in a word, or 8 codes in two words.  any_nan:
// some scaled value v * s is NaN (always so when some v is NaN).
template <int FMT, int E>
__device__ __forceinline__ uint2 enc_vec(const float v[E], float s, bool& any_nan) {
    bool n0, n1 = false;
    const uint32_t lo = enc4<FMT>(v[0] * s, v[1] * s, v[2] * s, v[3] * s, n0);
    const uint32_t hi = E == 4 ? 0u : enc4<FMT>(v[4] * s, v[5] * s, v[6] * s, v[7] * s, n1);
    any_nan = n0 | n1;
    return make_uint2(lo, hi);
}
template <int FMT, int E>
__device__ __forceinline__ uint2 enc_vec(const float v[E], float s) {
    bool any_nan;
    return enc_vec<FMT, E>(v, s, any_nan);
}

// Byte offset in the LDS tile of the 4-byte word `w` (0..31) of tile row `r`.
__device__ __forceinline__ int lds_word(int r, int w) { return r * kTile + ((w ^ (((r >> 5) & 3) << 3)) << 2); }

// 4 x 4 byte transpose: a..d are four rows of four bytes; c0..c3 are the four
// columns (byte i of column j = byte j of row i).
__device__ __forceinline__ void transpose4x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t& c0,
                                             uint32_t& c1, uint32_t& c2, uint32_t& c3) {
    const uint32_t ab_lo = __builtin_amdgcn_perm(b, a, 0x05010400u);   // a0 b0 a1 b1
    const uint32_t ab_hi = __builtin_amdgcn_perm(b, a, 0x07030602u);   // a2 b2 a3 b3
    const uint32_t cd_lo = __builtin_amdgcn_perm(d, c, 0x05010400u);   // c0 d0 c1 d1
    const uint32_t cd_hi = __builtin_amdgcn_perm(d, c, 0x07030602u);   // c2 d2 c3 d3
    c0 = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u);             // a0 b0 c0 d0
    c1 = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u);             // a1 b1 c1 d1
    c2 = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u);
    c3 = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u);
}

// Outputs of the dual-format variant (its second format is always E5M2).
struct Second {
    const float* scale;
    uint8_t* q;
    uint8_t* qt;
    float* amax_slot;
};

// A second tensor of the same element type and format, cast by the same
// launch (the pair variant): the workgroups' tile indices past the first
// tensor's tiles address this one.
struct CtJob {
    const void* x;
    int64_t rows, cols, tiles_c;
    const float* scale;
    uint8_t* q;
    uint8_t* qt;
    float* amax_slot;
};

// The scale update the dual-format variant can finish with: the metas of its
// two formats (0: E4M3, 1: E5M2) in one bank, hist [2][L]; ticket == nullptr:
// no update.
struct DualUpdate {
    float* hist;
    float* scale;
    float* sinv;
    int32_t L, margin;
    unsigned int* ticket;
};

// The optimizer step the SGD variant applies to an fp32 weight matrix before
// casting it: w <- w - lr * (g * (1 / S)) in place (the arithmetic of
// k_sgd), skipped when the step found Inf/NaN gradients (state[2] != 0).
struct SgdPre {
    float* w;
    const float* g;
    float lr;
    const float* state;
};

template <int DT, int FMT, bool DGELU, bool DBIAS, bool DUAL, bool PAIR = false, bool SGD = false>
__global__ void __launch_bounds__(kThreads)
k_cast_transpose(const void* __restrict__ x_a, const void* __restrict__ z, int64_t rows_a, int64_t cols_a,
                 int64_t tiles_ca, const float* __restrict__ scale_p, uint8_t* __restrict__ q_a,
                 uint8_t* __restrict__ qt_a, float* amax_slot, float* __restrict__ dbias_ws,
                 void* __restrict__ dz_out, Second sec, SinvSnap snap, CtJob job_b, DualUpdate upd, SatCounts sat,
                 SgdPre sgd) {
    static_assert(!PAIR || (!DGELU && !DBIAS && !DUAL), "the pair variant is a plain cast-transpose");
    static_assert(!SGD || (DT == kF32 && !PAIR && !DGELU && !DBIAS && !DUAL), "the SGD variant casts fp32 weights");
    using C = CtVec<DT>;
    constexpr int E = C::E, NP = C::NP;
    constexpr int NF = DUAL ? 2 : 1;
    __shared__ __attribute__((aligned(16))) uint8_t tile[NF * kTile * kTile];
    __shared__ uint32_t red[kThreads / 64];
    // GeLU backward on bf16 Z: gelu'(z) of every bf16 pattern with
    // 2^-8 <= |z| < 16 (exponent fields 119 .. 130, both signs), computed once
    // per workgroup by the same function the other elements use, so a lookup
    // returns exactly what the arithmetic would.
    constexpr bool kGeluTable = DGELU && DT == kBF16;
    __shared__ float gtab[kGeluTable ? kGeluTabN : 1];
    take_snapshot(snap);
    if constexpr (kGeluTable) {
        for (int i = threadIdx.x; i < kGeluTabN; i += kThreads) {
            const uint32_t bits = ((uint32_t)(i / kGeluTabHalf) << 15) | (uint32_t)(i % kGeluTabHalf + (kGeluExpLo << 7));
            gtab[i] = gelu_grad_f32(__uint_as_float(bits << 16));
        }
        __syncthreads();
    }

    const int t = threadIdx.x;
    const int vc = t % C::V;          // vector column in the tile
    const int r_first = t / C::V;     // first tile row; then every C::RS rows
    const int cg = t >> 3, strip = t & 7;   // transpose phase
    const float s_a = *scale_p;
    const float s_b = PAIR ? *job_b.scale : 0.0f;
    const float s2 = DUAL ? *sec.scale : 0.0f;
    const bool sgd_update = SGD && sgd.state[2] == 0.0f;                    // uniform: the step's found_inf
    const float sgd_inv = SGD ? __fdiv_rn(1.0f, sgd.state[3]) : 0.0f;
    const int64_t ntiles_a = ((rows_a + kTile - 1) / kTile) * tiles_ca;
    const int64_t ntiles = ntiles_a + (PAIR ? ((job_b.rows + kTile - 1) / kTile) * job_b.tiles_c : 0);
    uint32_t m_a = 0, m_b = 0;
    uint32_t n_a = 0, n_b = 0;        // saturated elements (of the second tensor or format: n_b)
    for (int64_t tile_id = blockIdx.x; tile_id < ntiles; tile_id += gridDim.x) {
        const bool second = PAIR && tile_id >= ntiles_a;        // uniform per workgroup
        const void* const x = second ? job_b.x : x_a;
        const int64_t rows = second ? job_b.rows : rows_a, cols = second ? job_b.cols : cols_a;
        const uint32_t tiles_c = (uint32_t)(second ? job_b.tiles_c : tiles_ca);
        const float s = second ? s_b : s_a;
        uint8_t* const q = second ? job_b.q : q_a;
        uint8_t* const qt = second ? job_b.qt : qt_a;
        const uint32_t local_id = (uint32_t)(second ? tile_id - ntiles_a : tile_id);
        const bool count = (second ? sat.b : sat.a) != nullptr;      // uniform per workgroup
        // The tile's amax as the unsigned max of |v|'s bit patterns: for a
        // vector without NaN that is the float max of |v| (non-negative
        // floats order as their bits), taken two elements per instruction;
        // a vector whose scaled values hold a NaN (so every vector with a NaN
        // element) adds its exact bit patterns instead.
        float mf = 0.0f;
        uint32_t mb = 0;
        const uint32_t tr = local_id / tiles_c, tc = local_id - tr * tiles_c;
        const int64_t r0 = (int64_t)tr * kTile, c0 = (int64_t)tc * kTile;
        const uint32_t trows = (uint32_t)min(rows - r0, (int64_t)kTile), tcols = (uint32_t)min(cols - c0, (int64_t)kTile);
        const uint32_t ucols = (uint32_t)cols, urows = (uint32_t)rows;

        // Every global access of the tile is a buffer access relative to the
        // tile's first element, bounded by the tile's rows (num_records): a
        // lane past the last row lands beyond the bound, a lane past the last
        // column is given the offset kOob; such loads return zeros and such
        // stores are dropped.  Offsets stay below 2^32 (the launcher admits
        // cols < 2^22 and rows < 2^24).
        const uint32_t e0 = vc * E < tcols ? (uint32_t)r_first * ucols + vc * E : kOob;   // element offset
        const uint32_t estep = C::RS * ucols;                                            // between vectors
        const int64_t tile0 = r0 * cols + c0;
        constexpr uint32_t XB = DT == kF32 ? 4 : 2;
        const uint32_t xnum = trows * ucols * XB;
        auto xoff = [&](int p) { return e0 == kOob ? kOob : (e0 + (uint32_t)p * estep) * XB; };
        auto qoff = [&](int p) { return e0 == kOob ? kOob : e0 + (uint32_t)p * estep; };
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(static_cast<const uint8_t*>(SGD ? (const void*)sgd.w : x) + tile0 * XB, xnum);
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(q ? q + tile0 : nullptr, q ? trows * ucols : 0u);

        uint4 rv[NP], rz[DGELU ? NP : 1];
#pragma unroll
        for (int p = 0; p < NP; ++p) rv[p] = buf_load16(rx, xoff(p));
        if constexpr (SGD) {
            // the weights (read and written through sgd.w, not x) and their gradients
            if (sgd_update) {
                const __amdgpu_buffer_rsrc_t rg = make_rsrc(reinterpret_cast<const uint8_t*>(sgd.g) + tile0 * 4, xnum);
                uint4 rg_v[NP];
#pragma unroll
                for (int p = 0; p < NP; ++p) rg_v[p] = buf_load16(rg, xoff(p));
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    float4 wv = __builtin_bit_cast(float4, rv[p]);
                    const float4 gv = __builtin_bit_cast(float4, rg_v[p]);
                    wv.x = wv.x - sgd.lr * (gv.x * sgd_inv);
                    wv.y = wv.y - sgd.lr * (gv.y * sgd_inv);
                    wv.z = wv.z - sgd.lr * (gv.z * sgd_inv);
                    wv.w = wv.w - sgd.lr * (gv.w * sgd_inv);
                    rv[p] = __builtin_bit_cast(uint4, wv);
                    buf_store16(rx, xoff(p), rv[p]);
                }
            }
        }
        if constexpr (DGELU) {
            const __amdgpu_buffer_rsrc_t rzs = make_rsrc(static_cast<const uint8_t*>(z) + tile0 * XB, xnum);
#pragma unroll
            for (int p = 0; p < NP; ++p) rz[p] = buf_load16(rzs, xoff(p));
        }
        const __amdgpu_buffer_rsrc_t rdz = make_rsrc(DGELU && dz_out ? static_cast<uint8_t*>(dz_out) + tile0 * XB : nullptr,
                                                     DGELU && dz_out ? xnum : 0u);

        float csum[E];
#pragma unroll
        for (int j = 0; j < E; ++j) csum[j] = 0.0f;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int lrow = r_first + C::RS * p;
            float v[E];
            unpack_vec<DT>(rv[p], v);
            if constexpr (DGELU) {
                float zz[E];
                unpack_vec<DT>(rz[p], zz);
#pragma unroll
                for (int j = 0; j < E; ++j) {
                    float gz;
                    if constexpr (kGeluTable) {
                        const uint32_t u = __float_as_uint(zz[j]) >> 16;                // the bf16 bits
                        const bool in = ((u >> 7) & 0xFFu) - (uint32_t)kGeluExpLo < (uint32_t)kGeluExps;
                        const uint32_t idx = (u >> 15) * kGeluTabHalf + (u & 0x7FFFu) - (kGeluExpLo << 7);
                        gz = gtab[in ? idx : 0];
                        if (!in) gz = gelu_grad_f32(zz[j]);
                    } else {
                        gz = gelu_grad_f32(zz[j]);
                    }
                    const float g = v[j] * gz;
                    v[j] = DT == kF32 ? g : round_to_bf16(g);
                }
                if (dz_out) buf_store16(rdz, xoff(p), pack_vec<DT>(v));
            }
            const int lds = lds_word(lrow, vc * (E / 4));
            bool vnan;
            const uint2 codes = enc_vec<FMT, E>(v, s, vnan);
            float vm = mf;
#pragma unroll
            for (int j = 0; j < E; ++j) {
                vm = fmaxf(vm, fabsf(v[j]));
                if constexpr (DBIAS) csum[j] += v[j];
            }
            mf = vnan ? mf : vm;
            asm volatile("" : "+v"(mf));      // keeps the max here (not sunk to the tile's end with every |v| live)
            if (vnan) {
#pragma unroll
                for (int j = 0; j < E; ++j) mb = max(mb, abs_bits(v[j]));
            }
            if (count) {
                const uint32_t c = sat_count<FMT, E>(v, s);
                if (second) n_b += c;
                else n_a += c;
            }
            if constexpr (DUAL) {
                if (sat.b) n_b += sat_count<kE5M2, E>(v, s2);
            }
            if constexpr (E == 8) {
                if (q) buf_store8(rq, qoff(p), codes);
                if (qt) *reinterpret_cast<uint2*>(tile + lds) = codes;
            } else {
                if (q) buf_store4(rq, qoff(p), codes.x);
                if (qt) *reinterpret_cast<uint32_t*>(tile + lds) = codes.x;
            }
            if constexpr (DUAL) {
                const __amdgpu_buffer_rsrc_t rq2 = make_rsrc(sec.q ? sec.q + tile0 : nullptr, sec.q ? trows * ucols : 0u);
                const uint2 c2 = enc_vec<kE5M2, E>(v, s2);
                if constexpr (E == 8) {
                    if (sec.q) buf_store8(rq2, qoff(p), c2);
                    if (sec.qt) *reinterpret_cast<uint2*>(tile + kTile * kTile + lds) = c2;
                } else {
                    if (sec.q) buf_store4(rq2, qoff(p), c2.x);
                    if (sec.qt) *reinterpret_cast<uint32_t*>(tile + kTile * kTile + lds) = c2.x;
                }
            }
        }
        __syncthreads();

        // Transposed write: four q_t rows (input columns c0 + 4 cg ..) x one
        // 16-byte strip (input rows r0 + 16 strip ..) per thread and format,
        // as buffer stores relative to q_t's element (c0, r0) bounded by the
        // tile's columns; a strip past the last row gets kOob.
        const uint32_t t0 = (uint32_t)strip * 16 < trows ? (uint32_t)(4 * cg) * urows + strip * 16 : kOob;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            uint8_t* const qtf = f == 0 ? qt : sec.qt;
            if (!qtf) continue;
            const __amdgpu_buffer_rsrc_t rt = make_rsrc(qtf + c0 * rows + r0, tcols * urows);
            const uint8_t* const tf = tile + f * kTile * kTile;
            uint32_t w[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) w[i] = *reinterpret_cast<const uint32_t*>(tf + lds_word(strip * 16 + i, cg));
            uint32_t o[4][4];       // o[j][k]: word k of the vector for column 4 cg + j
#pragma unroll
            for (int k = 0; k < 4; ++k)
                transpose4x4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3], o[0][k], o[1][k], o[2][k], o[3][k]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                buf_store16(rt, t0 == kOob ? kOob : t0 + (uint32_t)j * urows, make_uint4(o[j][0], o[j][1], o[j][2], o[j][3]));
        }

        if constexpr (DBIAS) {
            // Column partial sums of this tile in a fixed order: per thread over
            // its NP rows, then over the RS threads that share its columns.
            // Reuses the LDS tile as fp32 [RS][128].
            __syncthreads();
            float* fs = reinterpret_cast<float*>(tile);
#pragma unroll
            for (int j = 0; j < E; ++j) fs[r_first * kTile + vc * E + j] = csum[j];
            __syncthreads();
            if (t < kTile) {
                float acc = 0.0f;
                for (int g = 0; g < C::RS; ++g) acc += fs[g * kTile + t];
                if (c0 + t < cols) dbias_ws[tr * cols + c0 + t] = acc;
            }
        }
        __syncthreads();             // the LDS tile is rewritten by the next tile
        const uint32_t m = max(__float_as_uint(mf), mb);
        if (second) m_b = max(m_b, m);
        else m_a = max(m_a, m);
    }
    if constexpr (DUAL) {
        if (upd.ticket) {
            // The last workgroup to finish updates both metas ([TE-KR]
            // "FP8 자동변환(Autocasting)": cast, amax and factor as one step).
            // Thread 0 merges the workgroup's amax into both slots with
            // returning atomics and takes its ticket only once both have
            // returned (the ticket increment depends on their results), so
            // every merge is performed at the device's coherence point before
            // the last ticket is taken; no release fence (on this chip an
            // agent-scope release writes the L2 back, in every workgroup).
            // The last workgroup then reads the histories with device-scope
            // loads after an acquire fence, and leaves the ticket at zero.
            // Every workgroup read the scales before taking its ticket.
            const uint32_t wm = wave_max_u32(m_a);
            if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = wm;
            __syncthreads();
            __shared__ uint32_t last;
            if (threadIdx.x == 0) {
                uint32_t bm = 0;
                for (int w = 0; w < kThreads / 64; ++w) bm = max(bm, red[w]);
                const uint32_t o4 = atomicMax(reinterpret_cast<unsigned int*>(amax_slot), bm);
                const uint32_t o5 = atomicMax(reinterpret_cast<unsigned int*>(sec.amax_slot), bm);
                uint32_t dep;
                asm volatile("v_and_b32 %0, 0, %1" : "=v"(dep) : "v"(o4 ^ o5));
                last = atomicAdd(upd.ticket, 1u + dep) == gridDim.x - 1 ? 1u : 0u;
            }
            __syncthreads();
            if (last) {
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                float* fred = reinterpret_cast<float*>(red);
                scale_update_block<true>(upd.hist, upd.scale, upd.sinv, 448.0f, upd.L, upd.margin, fred);
                scale_update_block<true>(upd.hist + upd.L, upd.scale + 1, upd.sinv + 1, 57344.0f, upd.L, upd.margin,
                                         fred);
                if (threadIdx.x == 0) __hip_atomic_store(upd.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        } else {
            if (amax_slot) block_amax_merge(m_a, amax_slot, red);
            if (sec.amax_slot) {
                __syncthreads();     // red[] is reused
                block_amax_merge(m_a, sec.amax_slot, red);
            }
        }
    } else {
        if (amax_slot) block_amax_merge(m_a, amax_slot, red);
    }
    if constexpr (PAIR) {
        if (job_b.amax_slot) {
            __syncthreads();
            block_amax_merge(m_b, job_b.amax_slot, red);
        }
    }
    if (sat.a) wave_count_add(n_a, sat.a);
    if constexpr (DUAL || PAIR) {
        if (sat.b) wave_count_add(n_b, sat.b);
    }
}

// dbias[c] = sum over row tiles of the partials, in row-tile order.
__global__ void __launch_bounds__(256)
k_dbias_reduce(const float* __restrict__ ws, int64_t tiles_r, int64_t cols, float* __restrict__ dbias) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= cols) return;
    float acc = 0.0f;
    for (int64_t r = 0; r < tiles_r; ++r) acc += ws[r * cols + c];
    dbias[c] = acc;
}

// Grid of a cast-transpose instance: the workgroups that are resident at once
// (its occupancy times the compute units), at most one per tile.  Each
// workgroup loops over tiles with the grid as stride, so every workgroup takes
// within one as many tiles as any other (a grid of more than one resident
// wave of workgroups would leave the last wave part-empty).
template <int DT, int FMT, bool DGELU, bool DBIAS, bool DUAL, bool PAIR, bool SGD>
dim3 ct_grid(int64_t ntiles) {
    static const int per_cu = [] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_cast_transpose<DT, FMT, DGELU, DBIAS, DUAL, PAIR, SGD>,
                                                         kThreads, 0) != hipSuccess || n < 1)
            n = 1;
        return n;
    }();
    const int64_t resident = (int64_t)cu_count() * per_cu;
    return dim3((unsigned)(ntiles < resident ? ntiles : resident));
}

template <int DT, int FMT>
hipError_t launch_dt_fmt(const void* x, const void* z, int64_t rows, int64_t cols, const float* scale,
                         uint8_t* q, uint8_t* qt, float* slot, float* dbias_ws, void* dz_out, hipStream_t s,
                         SinvSnap snap, SatCounts sat) {
    const int64_t tiles_r = (rows + kTile - 1) / kTile, tiles_c = (cols + kTile - 1) / kTile;
    const int64_t ntiles = tiles_r * tiles_c;
    const dim3 block(kThreads);
    const bool dgelu = z != nullptr, dbias = dbias_ws != nullptr;
    const Second none{nullptr, nullptr, nullptr, nullptr};
    if (!dgelu && !dbias)
        hipLaunchKernelGGL((k_cast_transpose<DT, FMT, false, false, false>),
                           (ct_grid<DT, FMT, false, false, false, false, false>(ntiles)), block, 0, s, x, z, rows, cols,
                           tiles_c, scale, q, qt, slot, dbias_ws, dz_out, none, snap, CtJob{}, DualUpdate{}, sat, SgdPre{});
    else if (!dgelu)
        hipLaunchKernelGGL((k_cast_transpose<DT, FMT, false, true, false>),
                           (ct_grid<DT, FMT, false, true, false, false, false>(ntiles)), block, 0, s, x, z, rows, cols,
                           tiles_c, scale, q, qt, slot, dbias_ws, dz_out, none, snap, CtJob{}, DualUpdate{}, sat, SgdPre{});
    else if (!dbias)
        hipLaunchKernelGGL((k_cast_transpose<DT, FMT, true, false, false>),
                           (ct_grid<DT, FMT, true, false, false, false, false>(ntiles)), block, 0, s, x, z, rows, cols,
                           tiles_c, scale, q, qt, slot, dbias_ws, dz_out, none, snap, CtJob{}, DualUpdate{}, sat, SgdPre{});
    else
        hipLaunchKernelGGL((k_cast_transpose<DT, FMT, true, true, false>),
                           (ct_grid<DT, FMT, true, true, false, false, false>(ntiles)), block, 0, s, x, z, rows, cols,
                           tiles_c, scale, q, qt, slot, dbias_ws, dz_out, none, snap, CtJob{}, DualUpdate{}, sat, SgdPre{});
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dual_dt(const void* x, int64_t rows, int64_t cols, const float* scale4, uint8_t* q4,
                          uint8_t* q4t, float* slot4, const Second& sec, hipStream_t s, DualUpdate upd, SatCounts sat) {
    const int64_t tiles_r = (rows + kTile - 1) / kTile, tiles_c = (cols + kTile - 1) / kTile;
    const int64_t ntiles = tiles_r * tiles_c;
    const dim3 grid = ct_grid<DT, kE4M3, false, false, true, false, false>(ntiles), block(kThreads);
    hipLaunchKernelGGL((k_cast_transpose<DT, kE4M3, false, false, true>), grid, block, 0, s, x, nullptr, rows,
                       cols, tiles_c, scale4, q4, q4t, slot4, nullptr, nullptr, sec, SinvSnap{}, CtJob{}, upd, sat, SgdPre{});
    return hipGetLastError();
}

template <int DT, int FMT>
hipError_t launch_pair_dt_fmt(const void* xa, int64_t rows, int64_t cols, const float* scale, uint8_t* q, uint8_t* qt,
                              float* slot, const CtJob& b, hipStream_t s, SinvSnap snap, SatCounts sat) {
    const int64_t tiles_c = (cols + kTile - 1) / kTile;
    const int64_t ntiles = ((rows + kTile - 1) / kTile) * tiles_c + ((b.rows + kTile - 1) / kTile) * b.tiles_c;
    const dim3 grid = ct_grid<DT, FMT, false, false, false, true, false>(ntiles), block(kThreads);
    const Second none{nullptr, nullptr, nullptr, nullptr};
    hipLaunchKernelGGL((k_cast_transpose<DT, FMT, false, false, false, true>), grid, block, 0, s, xa, nullptr, rows,
                       cols, tiles_c, scale, q, qt, slot, nullptr, nullptr, none, snap, b, DualUpdate{}, sat, SgdPre{});
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sgd_cast_transpose(float* w, const float* g, int64_t rows, int64_t cols, float lr,
                                     const float* state, const float* scale, uint8_t* q, uint8_t* qt, float* slot,
                                     hipStream_t s, SatCounts sat) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const int64_t tiles_r = (rows + kTile - 1) / kTile, tiles_c = (cols + kTile - 1) / kTile;
    const int64_t ntiles = tiles_r * tiles_c;
    const dim3 grid = ct_grid<kF32, kE4M3, false, false, false, false, true>(ntiles), block(kThreads);
    const Second none{nullptr, nullptr, nullptr, nullptr};
    timing_before(kKindSgd, s);
    hipLaunchKernelGGL((k_cast_transpose<kF32, kE4M3, false, false, false, false, true>), grid, block, 0, s, w,
                       nullptr, rows, cols, tiles_c, scale, q, qt, slot, nullptr, nullptr, none, SinvSnap{}, CtJob{},
                       DualUpdate{}, sat, SgdPre{w, g, lr, state});
    timing_after(s);
    return hipGetLastError();
}

int64_t cast_transpose_dbias_ws_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    return ((rows + kTile - 1) / kTile) * cols * (int64_t)sizeof(float);
}

// Scratch of the cast-transpose that allocates nothing: the bias gradient's
// per-row-tile partial sums (every entry is written before it is read, so
// nothing needs clearing).  Each device holds its own copy until the process
// ends; calls that overlap on one device share it and race.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

hipError_t noalloc_scratch(hipStream_t s, float** out) {
    static std::mutex mu;
    static float* ptr[kMaxDevices] = {};
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    dev = cur;
    if (s && (e = hipStreamGetDevice(s, &dev)) != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!ptr[dev]) {
        // the symbol's address on the stream's device, looked up with that
        // device current (each device has its own copy of the array)
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        ptr[dev] = static_cast<float*>(p);
    }
    *out = ptr[dev];
    return hipSuccess;
}

hipError_t launch_cast_transpose(const void* x, const void* z, int dtype, int64_t rows, int64_t cols, int fmt,
                                 const float* scale, uint8_t* q, uint8_t* qt, float* slot, float* dbias,
                                 float* dbias_ws, void* dz_out, hipStream_t s, SinvSnap snap, SatCounts sat) {
    if (rows == 0 || cols == 0) {
        if (dbias && cols > 0) return launch_zero_f32(dbias, cols, s);
        return hipSuccess;
    }
    float* ws = dbias ? dbias_ws : nullptr;
    hipError_t e;
    timing_before(kKindCastT, s);
    if (dtype == kF32 && fmt == kE4M3)
        e = launch_dt_fmt<kF32, kE4M3>(x, z, rows, cols, scale, q, qt, slot, ws, dz_out, s, snap, sat);
    else if (dtype == kF32)
        e = launch_dt_fmt<kF32, kE5M2>(x, z, rows, cols, scale, q, qt, slot, ws, dz_out, s, snap, sat);
    else if (fmt == kE4M3)
        e = launch_dt_fmt<kBF16, kE4M3>(x, z, rows, cols, scale, q, qt, slot, ws, dz_out, s, snap, sat);
    else
        e = launch_dt_fmt<kBF16, kE5M2>(x, z, rows, cols, scale, q, qt, slot, ws, dz_out, s, snap, sat);
    timing_after(s);
    if (e != hipSuccess || !dbias) return e;
    const int64_t tiles_r = (rows + kTile - 1) / kTile;
    timing_before(kKindDbias, s);
    hipLaunchKernelGGL(k_dbias_reduce, dim3((unsigned)((cols + 255) / 256)), dim3(256), 0, s, ws, tiles_r, cols,
                       dbias);
    timing_after(s);
    return hipGetLastError();
}

hipError_t launch_cast_transpose_dual(const void* x, int dtype, int64_t rows, int64_t cols, const float* scale_e4m3,
                                      uint8_t* q_e4m3, uint8_t* q_e4m3_t, float* slot_e4m3, const float* scale_e5m2,
                                      uint8_t* q_e5m2, uint8_t* q_e5m2_t, float* slot_e5m2, hipStream_t s,
                                      SatCounts sat) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const Second sec{scale_e5m2, q_e5m2, q_e5m2_t, slot_e5m2};
    timing_before(kKindCastT, s);
    const hipError_t e = dtype == kF32
        ? launch_dual_dt<kF32>(x, rows, cols, scale_e4m3, q_e4m3, q_e4m3_t, slot_e4m3, sec, s, DualUpdate{}, sat)
        : launch_dual_dt<kBF16>(x, rows, cols, scale_e4m3, q_e4m3, q_e4m3_t, slot_e4m3, sec, s, DualUpdate{}, sat);
    timing_after(s);
    return e;
}

hipError_t launch_cast_transpose_dual_update(const void* x, int dtype, int64_t rows, int64_t cols, uint8_t* q_e4m3,
                                             uint8_t* q_e4m3_t, uint8_t* q_e5m2, uint8_t* q_e5m2_t, float* hist,
                                             float* scale, float* sinv, int32_t L, int32_t margin,
                                             unsigned int* ticket, hipStream_t s, SatCounts sat) {
    if (rows == 0 || cols == 0) {      // nothing to cast: the update alone
        const uint8_t fmts[2] = {kE4M3, kE5M2};
        return launch_scale_update(hist, scale, sinv, fmts, 2, L, margin, s);
    }
    const Second sec{scale + 1, q_e5m2, q_e5m2_t, hist + L};
    const DualUpdate upd{hist, scale, sinv, L, margin, ticket};
    timing_before(kKindCastT, s);
    const hipError_t e = dtype == kF32
        ? launch_dual_dt<kF32>(x, rows, cols, scale, q_e4m3, q_e4m3_t, hist, sec, s, upd, sat)
        : launch_dual_dt<kBF16>(x, rows, cols, scale, q_e4m3, q_e4m3_t, hist, sec, s, upd, sat);
    timing_after(s);
    return e;
}

hipError_t launch_cast_transpose_pair(const void* xa, const void* xb, int dtype, int64_t rows_a, int64_t cols_a,
                                      int64_t rows_b, int64_t cols_b, int fmt, const float* scale_a, uint8_t* q_a,
                                      uint8_t* qt_a, float* slot_a, const float* scale_b, uint8_t* q_b, uint8_t* qt_b,
                                      float* slot_b, hipStream_t s, SinvSnap snap, SatCounts sat) {
    const CtJob b{xb, rows_b, cols_b, (cols_b + kTile - 1) / kTile, scale_b, q_b, qt_b, slot_b};
    hipError_t e;
    timing_before(kKindCastT, s);
    if (dtype == kF32 && fmt == kE4M3)
        e = launch_pair_dt_fmt<kF32, kE4M3>(xa, rows_a, cols_a, scale_a, q_a, qt_a, slot_a, b, s, snap, sat);
    else if (dtype == kF32)
        e = launch_pair_dt_fmt<kF32, kE5M2>(xa, rows_a, cols_a, scale_a, q_a, qt_a, slot_a, b, s, snap, sat);
    else if (fmt == kE4M3)
        e = launch_pair_dt_fmt<kBF16, kE4M3>(xa, rows_a, cols_a, scale_a, q_a, qt_a, slot_a, b, s, snap, sat);
    else
        e = launch_pair_dt_fmt<kBF16, kE5M2>(xa, rows_a, cols_a, scale_a, q_a, qt_a, slot_a, b, s, snap, sat);
    timing_after(s);
    return e;
}

}  // namespace fp8lin
