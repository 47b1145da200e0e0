// Fused amax + cast + transpose (+ bias-gradient partial sums, + GeLU backward).
//
// Pages (titles in include/fp8lin.h): [TE-KR] "FP8 자동변환(Autocasting)"
// (cast, amax and factor in one step) and "Backward Pass 처리" (the backward
// GEMMs consume the FP8 copies made here); [PT-VI] torch._scaled_mm example
// (the second GEMM operand enters transposed).
//
// One workgroup (256 threads, 4 waves) owns a 128 x 128 tile of the
// [rows][cols] input.  Load phase: thread t reads 16 consecutive columns of
// rows (t/8) + 32p, p = 0..3 (all loads issued before any use), merges |x|
// into its amax, encodes, writes the 16 codes to q with one 16-byte store and
// to an LDS tile [128][128] with one 16-byte LDS store; the 16-byte chunk of
// LDS row r is stored at chunk position chunk ^ ((r >> 4) & 7).  Transpose
// phase: lane l takes the 16-row strip l & 7 of output row (input column)
// l >> 3, reads that column's 16 bytes one by one (the swizzle spreads the 8
// strips of a wave over 8 bank groups, so the byte reads are conflict-free),
// packs them and writes one 16-byte store; 8 consecutive lanes thereby write
// the 128 contiguous bytes this tile contributes to one q_t row.  Rows and
// cols are multiples of 16, so a 16-element chunk is either entirely inside
// the tensor or entirely outside.  At most 2048 workgroups run; each loops
// over tiles, so the amax merge costs one (usually skipped) atomic per
// workgroup rather than one per tile.
//
// The dual-format variant encodes every element with two scales, to E4M3 and
// to E5M2, from one read of the input: four outputs (both formats, both
// layouts) through two LDS tiles, and one amax for both tensors' metas.
#include "common.h"

namespace fp8lin {
namespace {

constexpr int kTile = 128;
constexpr int kThreads = 256;
constexpr int64_t kMaxGrid = 256 * 8;     // workgroups loop over tiles beyond this

// 16 elements from their raw 16-byte words (4 words of f32 or 2 of bf16).
template <int DT>
__device__ __forceinline__ void unpack16(const uint4* w, float v[16]) {
    if constexpr (DT == kF32) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[4 * j + 0] = __uint_as_float(w[j].x); v[4 * j + 1] = __uint_as_float(w[j].y);
            v[4 * j + 2] = __uint_as_float(w[j].z); v[4 * j + 3] = __uint_as_float(w[j].w);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t u[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[8 * j + 2 * h + 0] = __uint_as_float(u[h] << 16);
                v[8 * j + 2 * h + 1] = __uint_as_float(u[h] & 0xFFFF0000u);
            }
        }
    }
}

template <int DT>
__device__ __forceinline__ void store16(void* base, int64_t idx, const float v[16]) {
    if constexpr (DT == kF32) {
        uint4* p = reinterpret_cast<uint4*>(static_cast<float*>(base) + idx);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            p[j] = make_uint4(__float_as_uint(v[4 * j]), __float_as_uint(v[4 * j + 1]),
                              __float_as_uint(v[4 * j + 2]), __float_as_uint(v[4 * j + 3]));
    } else {
        uint4* p = reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + idx);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            p[j] = make_uint4(pack_bf16x2(v[8 * j], v[8 * j + 1]), pack_bf16x2(v[8 * j + 2], v[8 * j + 3]),
                              pack_bf16x2(v[8 * j + 4], v[8 * j + 5]), pack_bf16x2(v[8 * j + 6], v[8 * j + 7]));
    }
}

// Outputs of the dual-format variant (its second format is always E5M2).
struct Second {
    const float* scale;
    uint8_t* q;
    uint8_t* qt;
    float* amax_slot;
};

template <int DT, int FMT, bool DGELU, bool DBIAS, bool DUAL>
__global__ void __launch_bounds__(kThreads)
k_cast_transpose(const void* __restrict__ x, const void* __restrict__ z, int64_t rows, int64_t cols,
                 int64_t tiles_c, const float* __restrict__ scale_p, uint8_t* __restrict__ q,
                 uint8_t* __restrict__ qt, float* amax_slot, float* __restrict__ dbias_ws,
                 void* __restrict__ dz_out, Second sec) {
    constexpr int NF = DUAL ? 2 : 1;
    __shared__ __attribute__((aligned(16))) uint8_t tile[NF * kTile * kTile];
    __shared__ uint32_t red[kThreads / 64];

    const int t = threadIdx.x;
    const int cc = t & 7;        // 16-column chunk within the tile
    const int rr = t >> 3;       // 0..31
    const float s = *scale_p;
    const float s2 = DUAL ? *sec.scale : 0.0f;
    const int64_t ntiles = ((rows + kTile - 1) / kTile) * tiles_c;
    uint32_t m = 0;
    for (int64_t tile_id = blockIdx.x; tile_id < ntiles; tile_id += gridDim.x) {
    const int64_t tr = tile_id / tiles_c, tc = tile_id % tiles_c;
    const int64_t r0 = tr * kTile, c0 = tc * kTile;
    const int64_t col = c0 + cc * 16;
    const bool col_ok = col < cols;

    // Issue every load of the tile (and of z for the GeLU backward) before
    // touching any of them, then unpack.
    constexpr int NV = DT == kF32 ? 4 : 2;              // 16-byte loads per 16 elements
    uint4 rv[4][NV], rz[DGELU ? 4 : 1][NV];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int64_t row = r0 + rr + 32 * p;
        const bool ok = col_ok && row < rows;
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(x) +
                                                          (row * cols + col) * (DT == kF32 ? 4 : 2));
#pragma unroll
        for (int j = 0; j < NV; ++j) rv[p][j] = ok ? src[j] : make_uint4(0, 0, 0, 0);
    }
    if constexpr (DGELU) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int64_t row = r0 + rr + 32 * p;
            const bool ok = col_ok && row < rows;
            const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(z) +
                                                              (row * cols + col) * (DT == kF32 ? 4 : 2));
#pragma unroll
            for (int j = 0; j < NV; ++j) rz[p][j] = ok ? src[j] : make_uint4(0, 0, 0, 0);
        }
    }
    float v[4][16];
#pragma unroll
    for (int p = 0; p < 4; ++p) unpack16<DT>(rv[p], v[p]);
    if constexpr (DGELU) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int64_t row = r0 + rr + 32 * p;
            float zz[16];
            unpack16<DT>(rz[p], zz);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float g = v[p][j] * gelu_grad_f32(zz[j]);
                v[p][j] = DT == kF32 ? g : round_to_bf16(g);
            }
            if (dz_out && col_ok && row < rows) store16<DT>(dz_out, row * cols + col, v[p]);
        }
    }

    float csum[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) csum[j] = 0.0f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int lrow = rr + 32 * p;
        const int64_t row = r0 + lrow;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            m = max(m, abs_bits(v[p][j]));
            if constexpr (DBIAS) csum[j] += v[p][j];
        }
        const int lds = lrow * kTile + ((cc ^ ((lrow >> 4) & 7)) << 4);
        const uint4 codes = scale_enc16<FMT>(v[p], s);
        if (q && col_ok && row < rows) *reinterpret_cast<uint4*>(q + row * cols + col) = codes;
        if (qt) *reinterpret_cast<uint4*>(tile + lds) = codes;
        if constexpr (DUAL) {
            const uint4 c2 = scale_enc16<kE5M2>(v[p], s2);
            if (sec.q && col_ok && row < rows) *reinterpret_cast<uint4*>(sec.q + row * cols + col) = c2;
            if (sec.qt) *reinterpret_cast<uint4*>(tile + kTile * kTile + lds) = c2;
        }
    }
    __syncthreads();

    // Transposed write: 128 output rows (input columns) x 8 strips of 16 bytes,
    // per format.
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        uint8_t* const qtf = f == 0 ? qt : sec.qt;
        const uint8_t* const tf = tile + f * kTile * kTile;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (!qtf) break;
            const int idx = t + kThreads * i;
            const int rc = idx & 7;                 // 16-row strip 0..7
            const int oc = idx >> 3;                // output row within the tile (input column)
            const int64_t orow = c0 + oc, ocol = r0 + rc * 16;
            const int colp = (((oc >> 4) ^ rc) << 4) | (oc & 15);   // swizzled byte column of strip rc
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint8_t* src = tf + (rc * 16 + 4 * j) * kTile + colp;
                w[j] = (uint32_t)src[0] | ((uint32_t)src[kTile] << 8) | ((uint32_t)src[2 * kTile] << 16) |
                       ((uint32_t)src[3 * kTile] << 24);
            }
            if (orow < cols && ocol < rows)
                *reinterpret_cast<uint4*>(qtf + orow * rows + ocol) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }

    if constexpr (DBIAS) {
        // Column partial sums of this tile in a fixed order: per thread over its
        // four rows, then over the 32 row groups.  Reuses the LDS tile as fp32.
        __syncthreads();
        float* fs = reinterpret_cast<float*>(tile);      // [32][128] floats = 16 KiB
#pragma unroll
        for (int j = 0; j < 16; ++j) fs[rr * kTile + cc * 16 + j] = csum[j];
        __syncthreads();
        if (t < kTile) {
            float acc = 0.0f;
            for (int g = 0; g < 32; ++g) acc += fs[g * kTile + t];
            if (c0 + t < cols) dbias_ws[tr * cols + c0 + t] = acc;
        }
    }
    __syncthreads();             // the LDS tile is rewritten by the next tile
    }
    if (amax_slot) block_amax_merge(m, amax_slot, red);
    if constexpr (DUAL) {
        if (sec.amax_slot) {
            __syncthreads();     // red[] is reused
            block_amax_merge(m, sec.amax_slot, red);
        }
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

template <int DT, int FMT>
hipError_t launch_dt_fmt(const void* x, const void* z, int64_t rows, int64_t cols, const float* scale,
                         uint8_t* q, uint8_t* qt, float* slot, float* dbias_ws, void* dz_out, hipStream_t s) {
    const int64_t tiles_r = (rows + kTile - 1) / kTile, tiles_c = (cols + kTile - 1) / kTile;
    const int64_t ntiles = tiles_r * tiles_c;
    const dim3 grid((unsigned)(ntiles < kMaxGrid ? ntiles : kMaxGrid)), block(kThreads);
    const bool dgelu = z != nullptr, dbias = dbias_ws != nullptr;
    const Second none{nullptr, nullptr, nullptr, nullptr};
    if (!dgelu && !dbias)
        hipLaunchKernelGGL((k_cast_transpose<DT, FMT, false, false, false>), grid, block, 0, s, x, z, rows, cols,
                           tiles_c, scale, q, qt, slot, dbias_ws, dz_out, none);
    else if (!dgelu)
        hipLaunchKernelGGL((k_cast_transpose<DT, FMT, false, true, false>), grid, block, 0, s, x, z, rows, cols,
                           tiles_c, scale, q, qt, slot, dbias_ws, dz_out, none);
    else if (!dbias)
        hipLaunchKernelGGL((k_cast_transpose<DT, FMT, true, false, false>), grid, block, 0, s, x, z, rows, cols,
                           tiles_c, scale, q, qt, slot, dbias_ws, dz_out, none);
    else
        hipLaunchKernelGGL((k_cast_transpose<DT, FMT, true, true, false>), grid, block, 0, s, x, z, rows, cols,
                           tiles_c, scale, q, qt, slot, dbias_ws, dz_out, none);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dual_dt(const void* x, int64_t rows, int64_t cols, const float* scale4, uint8_t* q4,
                          uint8_t* q4t, float* slot4, const Second& sec, hipStream_t s) {
    const int64_t tiles_r = (rows + kTile - 1) / kTile, tiles_c = (cols + kTile - 1) / kTile;
    const int64_t ntiles = tiles_r * tiles_c;
    const dim3 grid((unsigned)(ntiles < kMaxGrid ? ntiles : kMaxGrid)), block(kThreads);
    hipLaunchKernelGGL((k_cast_transpose<DT, kE4M3, false, false, true>), grid, block, 0, s, x, nullptr, rows,
                       cols, tiles_c, scale4, q4, q4t, slot4, nullptr, nullptr, sec);
    return hipGetLastError();
}

}  // namespace

int64_t cast_transpose_dbias_ws_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    return ((rows + kTile - 1) / kTile) * cols * (int64_t)sizeof(float);
}

hipError_t launch_cast_transpose(const void* x, const void* z, int dtype, int64_t rows, int64_t cols, int fmt,
                                 const float* scale, uint8_t* q, uint8_t* qt, float* slot, float* dbias,
                                 float* dbias_ws, void* dz_out, hipStream_t s) {
    if (rows == 0 || cols == 0) {
        if (dbias && cols > 0) return launch_zero_f32(dbias, cols, s);
        return hipSuccess;
    }
    float* ws = dbias ? dbias_ws : nullptr;
    hipError_t e;
    timing_before(kKindCastT, s);
    if (dtype == kF32 && fmt == kE4M3) e = launch_dt_fmt<kF32, kE4M3>(x, z, rows, cols, scale, q, qt, slot, ws, dz_out, s);
    else if (dtype == kF32) e = launch_dt_fmt<kF32, kE5M2>(x, z, rows, cols, scale, q, qt, slot, ws, dz_out, s);
    else if (fmt == kE4M3) e = launch_dt_fmt<kBF16, kE4M3>(x, z, rows, cols, scale, q, qt, slot, ws, dz_out, s);
    else e = launch_dt_fmt<kBF16, kE5M2>(x, z, rows, cols, scale, q, qt, slot, ws, dz_out, s);
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
                                      uint8_t* q_e5m2, uint8_t* q_e5m2_t, float* slot_e5m2, hipStream_t s) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const Second sec{scale_e5m2, q_e5m2, q_e5m2_t, slot_e5m2};
    timing_before(kKindCastT, s);
    const hipError_t e = dtype == kF32
        ? launch_dual_dt<kF32>(x, rows, cols, scale_e4m3, q_e4m3, q_e4m3_t, slot_e4m3, sec, s)
        : launch_dual_dt<kBF16>(x, rows, cols, scale_e4m3, q_e4m3, q_e4m3_t, slot_e4m3, sec, s);
    timing_after(s);
    return e;
}

}  // namespace fp8lin
