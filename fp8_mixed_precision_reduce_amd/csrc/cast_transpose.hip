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
// to an LDS tile [128][128] with one 16-byte LDS store (8 lanes of a row hit
// 8 distinct 16-byte bank groups).  Transpose phase: a wave reads 64
// consecutive LDS columns of one 16-row strip byte by byte (consecutive
// bytes: no bank conflicts), packs each column's 16 bytes and writes them to
// q_t with one 16-byte store; each q_t row receives 128 contiguous bytes per
// tile.  Rows and cols are multiples of 16, so a 16-element chunk is either
// entirely inside the tensor or entirely outside.
#include "common.h"

namespace fp8lin {
namespace {

constexpr int kTile = 128;
constexpr int kThreads = 256;

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

template <int DT, int FMT, bool DGELU, bool DBIAS>
__global__ void __launch_bounds__(kThreads)
k_cast_transpose(const void* __restrict__ x, const void* __restrict__ z, int64_t rows, int64_t cols,
                 int64_t tiles_c, const float* __restrict__ scale_p, uint8_t* __restrict__ q,
                 uint8_t* __restrict__ qt, float* amax_slot, float* __restrict__ dbias_ws,
                 void* __restrict__ dz_out) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[kTile * kTile];
    __shared__ uint32_t red[kThreads / 64];

    const int64_t tr = blockIdx.x / tiles_c, tc = blockIdx.x % tiles_c;
    const int64_t r0 = tr * kTile, c0 = tc * kTile;
    const int t = threadIdx.x;
    const int cc = t & 7;        // 16-column chunk within the tile
    const int rr = t >> 3;       // 0..31
    const int64_t col = c0 + cc * 16;
    const bool col_ok = col < cols;
    const float s = *scale_p;

    float v[4][16];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int64_t row = r0 + rr + 32 * p;
        if (col_ok && row < rows) {
            load16<DT>(x, row * cols + col, v[p]);
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) v[p][j] = 0.0f;
        }
    }
    if constexpr (DGELU) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int64_t row = r0 + rr + 32 * p;
            float zz[16];
            if (col_ok && row < rows) load16<DT>(z, row * cols + col, zz);
            else {
#pragma unroll
                for (int j = 0; j < 16; ++j) zz[j] = 0.0f;
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float g = v[p][j] * gelu_grad_f32(zz[j]);
                v[p][j] = DT == kF32 ? g : round_to_bf16(g);
            }
            if (dz_out && col_ok && row < rows) store16<DT>(dz_out, row * cols + col, v[p]);
        }
    }

    uint32_t m = 0;
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
        const uint4 codes = scale_enc16<FMT>(v[p], s);
        if (q && col_ok && row < rows) *reinterpret_cast<uint4*>(q + row * cols + col) = codes;
        if (qt) *reinterpret_cast<uint4*>(tile + lrow * kTile + cc * 16) = codes;
    }
    __syncthreads();

    // Transposed write: 128 output rows (input columns) x 8 strips of 16 bytes.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (!qt) break;
        const int idx = t + kThreads * i;
        const int oc = idx & (kTile - 1);       // output row within the tile (input column)
        const int rc = idx >> 7;                // 16-row strip 0..7
        const int64_t orow = c0 + oc, ocol = r0 + rc * 16;
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint8_t* src = tile + (rc * 16 + 4 * j) * kTile + oc;
            w[j] = (uint32_t)src[0] | ((uint32_t)src[kTile] << 8) | ((uint32_t)src[2 * kTile] << 16) |
                   ((uint32_t)src[3 * kTile] << 24);
        }
        if (orow < cols && ocol < rows)
            *reinterpret_cast<uint4*>(qt + orow * rows + ocol) = make_uint4(w[0], w[1], w[2], w[3]);
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
    if (amax_slot) block_amax_merge(m, amax_slot, red);
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
    const dim3 grid((unsigned)(tiles_r * tiles_c)), block(kThreads);
    const bool dgelu = z != nullptr, dbias = dbias_ws != nullptr;
    if (!dgelu && !dbias)
        hipLaunchKernelGGL((k_cast_transpose<DT, FMT, false, false>), grid, block, 0, s, x, z, rows, cols,
                           tiles_c, scale, q, qt, slot, dbias_ws, dz_out);
    else if (!dgelu)
        hipLaunchKernelGGL((k_cast_transpose<DT, FMT, false, true>), grid, block, 0, s, x, z, rows, cols,
                           tiles_c, scale, q, qt, slot, dbias_ws, dz_out);
    else if (!dbias)
        hipLaunchKernelGGL((k_cast_transpose<DT, FMT, true, false>), grid, block, 0, s, x, z, rows, cols,
                           tiles_c, scale, q, qt, slot, dbias_ws, dz_out);
    else
        hipLaunchKernelGGL((k_cast_transpose<DT, FMT, true, true>), grid, block, 0, s, x, z, rows, cols,
                           tiles_c, scale, q, qt, slot, dbias_ws, dz_out);
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

}  // namespace fp8lin
