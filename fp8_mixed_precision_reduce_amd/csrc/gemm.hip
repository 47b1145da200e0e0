// FP8 x FP8 GEMM with fp32 accumulation on CDNA4 matrix cores and a fused
// epilogue.
//
//   y[i][j] = (sum_k dec(A[i][k]) * dec(B[j][k])) * sinv_a * sinv_b + bias[j]
//   D[i][j] = gelu(y) | y | D[i][j] + y, rounded to fp32 or bf16; optional
//   pre-GeLU copy and the amax of D as written.
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
// Tiling.  Both operands are contiguous along k ("TN").  A workgroup of 4
// waves (2 x 2) computes a BM x BN tile; each wave owns MB x NB blocks of
// 32 x 32.  k advances in stages of 128 bytes through a double-buffered LDS
// tile; global loads for the next stage go through buffer resources
// (out-of-range rows and the k tail read as zero) into registers while the
// current stage is multiplied.  LDS rows are 128 bytes; the 16-byte chunk
// index is XOR-swizzled with (row & 7) and the 8-byte half with bit 3 of the
// row, so 16-byte accesses of 8 consecutive rows and 8-byte accesses of 16
// consecutive rows each touch distinct banks.  The MFMA takes the B tile as
// its first operand, so each lane's accumulators run along n: four
// consecutive outputs of one row, written with one 16-byte (fp32) or 8-byte
// (bf16) store.  Tiles are rasterised in groups of 8 tile-rows, and the
// workgroup index is remapped so that each XCD (workgroups are dealt
// round-robin over 8 XCDs) works on a contiguous range of tiles that share
// operands in its own L2.
#include "common.h"

namespace fp8lin {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kBK = 128;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;
constexpr int kXcds = 8;
constexpr int kEpiFastAccum = 4;

struct GemmParams {
    const uint8_t* a;
    const uint8_t* b;
    int64_t m, n, k;
    const float* sinv_a;
    const float* sinv_b;
    const void* bias;
    void* d;
    void* aux;
    float* amax;
    int32_t tiles_m, tiles_n;
    int32_t bias_dtype, d_dtype, epilogue;
};

template <int MB, int NB>
struct TileCfg {
    static constexpr int BM = 2 * 32 * MB;
    static constexpr int BN = 2 * 32 * NB;
    static constexpr int A_LD = BM * kBK / 16 / kThreads;   // 16-byte chunks per thread per stage
    static constexpr int B_LD = BN * kBK / 16 / kThreads;
    static constexpr int STAGE = (BM + BN) * kBK;           // LDS bytes per stage
};

// Byte offset of the 16-byte chunk `chunk` of LDS row `row`; the two 8-byte
// halves of a chunk are stored swapped when bit 3 of the row is set.
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 4); }
__device__ __forceinline__ int half_swap(int row) { return (row >> 3) & 1; }
__device__ __forceinline__ uint4 swap_halves(uint4 v, int sw) { return sw ? make_uint4(v.z, v.w, v.x, v.y) : v; }

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

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// MFMA format selector of an FP8 operand.
template <int FMT> struct MfmaFmt;
template <> struct MfmaFmt<kE4M3> { static constexpr int value = 0; };
template <> struct MfmaFmt<kE5M2> { static constexpr int value = 1; };

// Logical tile index of this workgroup: undo the round-robin XCD dealing,
// then raster in groups of kGroupM tile-rows.
__device__ __forceinline__ void tile_coords(int32_t tiles_m, int32_t tiles_n, int& tm, int& tn) {
    const int nwg = tiles_m * tiles_n;
    const int i = blockIdx.x;
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

template <int MB, int NB, int AF, int BF, bool FAST>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(1, 1)))
k_gemm(GemmParams p) {
    using C = TileCfg<MB, NB>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];
    __shared__ uint32_t red[kThreads / 64];

    int tm, tn;
    tile_coords(p.tiles_m, p.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
    const int64_t M = p.m, N = p.n, K = p.k;

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int g = lane >> 5, r32 = lane & 31;

    // Buffer resources over this tile's rows of A and B.
    const uint32_t rows_a = (uint32_t)min<int64_t>(C::BM, M - m0), rows_b = (uint32_t)min<int64_t>(C::BN, N - n0);
    const __amdgpu_buffer_rsrc_t ra_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.a + m0 * K), (short)0, (int)(rows_a * (uint32_t)K), 0x00020000);
    const __amdgpu_buffer_rsrc_t rb_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.b + n0 * K), (short)0, (int)(rows_b * (uint32_t)K), 0x00020000);

    const int chunk = t & 7, row_base = t >> 3;     // this thread's chunk column and first row
    uint4 ga[C::A_LD], gb[C::B_LD];

    auto gload = [&](int kt) {
        const uint32_t kb = (uint32_t)kt * kBK + chunk * 16;
        const bool kok = kb < (uint32_t)K;
#pragma unroll
        for (int i = 0; i < C::A_LD; ++i) {
            const uint32_t row = row_base + 32 * i;
            ga[i] = buf_load16(ra_rsrc, kok ? row * (uint32_t)K + kb : 0x80000000u);
        }
#pragma unroll
        for (int i = 0; i < C::B_LD; ++i) {
            const uint32_t row = row_base + 32 * i;
            gb[i] = buf_load16(rb_rsrc, kok ? row * (uint32_t)K + kb : 0x80000000u);
        }
    };
    auto lstore = [&](int stage) {
        uint8_t* sa = smem + stage * C::STAGE;
        uint8_t* sb = sa + C::BM * kBK;
#pragma unroll
        for (int i = 0; i < C::A_LD; ++i) {
            const int row = row_base + 32 * i;
            *reinterpret_cast<uint4*>(sa + lds_off(row, chunk)) = swap_halves(ga[i], half_swap(row));
        }
#pragma unroll
        for (int i = 0; i < C::B_LD; ++i) {
            const int row = row_base + 32 * i;
            *reinterpret_cast<uint4*>(sb + lds_off(row, chunk)) = swap_halves(gb[i], half_swap(row));
        }
    };

    v16f acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int nk = (int)((K + kBK - 1) / kBK);
    if (nk > 0) {
        gload(0);
        lstore(0);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int stage = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const uint8_t* sa = smem + stage * C::STAGE;
        const uint8_t* sb = sa + C::BM * kBK;
        if constexpr (FAST) {
#pragma unroll
            for (int ks = 0; ks < kBK / 64; ++ks) {
                v8i af[MB], bf[NB];
                const int c0 = ks * 4 + g * 2;
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    const int row = wm * MB * 32 + i * 32 + r32;
                    const uint4 lo = swap_halves(*reinterpret_cast<const uint4*>(sa + lds_off(row, c0)), half_swap(row));
                    const uint4 hi = swap_halves(*reinterpret_cast<const uint4*>(sa + lds_off(row, c0 + 1)), half_swap(row));
                    af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                }
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int row = wn * NB * 32 + j * 32 + r32;
                    const uint4 lo = swap_halves(*reinterpret_cast<const uint4*>(sb + lds_off(row, c0)), half_swap(row));
                    const uint4 hi = swap_halves(*reinterpret_cast<const uint4*>(sb + lds_off(row, c0 + 1)), half_swap(row));
                    bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                }
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            bf[j], af[i], acc[i][j], MfmaFmt<BF>::value, MfmaFmt<AF>::value, 0, 0, 0, 0);
            }
        } else {
            // k steps of 16: lane group g holds k = 8g .. 8g+7 of the step.
#pragma unroll
            for (int ks = 0; ks < kBK / 16; ++ks) {
                v8h af[MB], bf[NB];
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    const int row = wm * MB * 32 + i * 32 + r32;
                    const uint2 raw = *reinterpret_cast<const uint2*>(sa + lds_off(row, ks) + ((g ^ half_swap(row)) << 3));
                    af[i] = dec8_f16<AF>(raw);
                }
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int row = wn * NB * 32 + j * 32 + r32;
                    const uint2 raw = *reinterpret_cast<const uint2*>(sb + lds_off(row, ks) + ((g ^ half_swap(row)) << 3));
                    bf[j] = dec8_f16<BF>(raw);
                }
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[j], af[i], acc[i][j], 0, 0, 0);
            }
        }
        if (kt + 1 < nk) lstore(stage ^ 1);
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    const float sc = (*p.sinv_a) * (*p.sinv_b);
    const bool gelu = p.epilogue & 1, accum = p.epilogue & 2;
    const bool out_bf16 = p.d_dtype == kBF16;
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        const int64_t mrow = m0 + wm * MB * 32 + i * 32 + r32;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int64_t ncol = n0 + wn * NB * 32 + j * 32 + 8 * q4 + 4 * g;
                if (mrow >= M || ncol >= N) continue;
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = acc[i][j][4 * q4 + e] * sc;
                if (p.bias) {
                    if (p.bias_dtype == kF32) {
                        const float4 bv = *reinterpret_cast<const float4*>(static_cast<const float*>(p.bias) + ncol);
                        y[0] += bv.x; y[1] += bv.y; y[2] += bv.z; y[3] += bv.w;
                    } else {
                        const uint2 bv = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.bias) + ncol);
                        y[0] += bf16_to_f32(bv.x & 0xFFFFu); y[1] += bf16_to_f32(bv.x >> 16);
                        y[2] += bf16_to_f32(bv.y & 0xFFFFu); y[3] += bf16_to_f32(bv.y >> 16);
                    }
                }
                const int64_t off = mrow * N + ncol;
                if (gelu) {
                    if (p.aux) {
                        if (out_bf16)
                            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.aux) + off) =
                                make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
                        else
                            *reinterpret_cast<float4*>(static_cast<float*>(p.aux) + off) = make_float4(y[0], y[1], y[2], y[3]);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = gelu_f32(y[e]);
                }
                if (out_bf16) {
                    const uint2 o = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.d) + off) = o;
                    amax = max(amax, max(max(abs_bits(bf16_to_f32(o.x & 0xFFFFu)), abs_bits(bf16_to_f32(o.x >> 16))),
                                         max(abs_bits(bf16_to_f32(o.y & 0xFFFFu)), abs_bits(bf16_to_f32(o.y >> 16)))));
                } else {
                    float4* dp = reinterpret_cast<float4*>(static_cast<float*>(p.d) + off);
                    if (accum) {
                        const float4 old = *dp;
                        y[0] = old.x + y[0]; y[1] = old.y + y[1]; y[2] = old.z + y[2]; y[3] = old.w + y[3];
                    }
                    *dp = make_float4(y[0], y[1], y[2], y[3]);
                    amax = max(amax, max(max(abs_bits(y[0]), abs_bits(y[1])), max(abs_bits(y[2]), abs_bits(y[3]))));
                }
            }
        }
    }
    if (p.amax) block_amax_merge(amax, p.amax, red);
}

template <int MB, int NB, bool FAST>
hipError_t launch_cfg(const GemmParams& base, int afmt, int bfmt, hipStream_t s) {
    using C = TileCfg<MB, NB>;
    GemmParams p = base;
    p.tiles_m = (int32_t)((p.m + C::BM - 1) / C::BM);
    p.tiles_n = (int32_t)((p.n + C::BN - 1) / C::BN);
    const dim3 grid((unsigned)p.tiles_m * (unsigned)p.tiles_n), block(kThreads);
    if (afmt == kE4M3 && bfmt == kE4M3) hipLaunchKernelGGL((k_gemm<MB, NB, kE4M3, kE4M3, FAST>), grid, block, 0, s, p);
    else if (afmt == kE5M2 && bfmt == kE4M3) hipLaunchKernelGGL((k_gemm<MB, NB, kE5M2, kE4M3, FAST>), grid, block, 0, s, p);
    else if (afmt == kE4M3) hipLaunchKernelGGL((k_gemm<MB, NB, kE4M3, kE5M2, FAST>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_gemm<MB, NB, kE5M2, kE5M2, FAST>), grid, block, 0, s, p);
    return hipGetLastError();
}

template <bool FAST>
hipError_t launch_path(const GemmParams& p, int afmt, int bfmt, hipStream_t s) {
    // Tile choice: 256 x 256 when that still gives every CU work, else smaller tiles.
    const int64_t big = ((p.m + 255) / 256) * ((p.n + 255) / 256);
    const int64_t mid = ((p.m + 127) / 128) * ((p.n + 127) / 128);
    if (big >= 256) return launch_cfg<4, 4, FAST>(p, afmt, bfmt, s);
    if (mid >= 256) return launch_cfg<2, 2, FAST>(p, afmt, bfmt, s);
    return launch_cfg<1, 1, FAST>(p, afmt, bfmt, s);
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a, int afmt, const uint8_t* b, int bfmt, int64_t m, int64_t n, int64_t k,
                       const float* sinv_a, const float* sinv_b, const void* bias, int bias_dtype, int epilogue,
                       void* d, int d_dtype, void* aux, float* amax, hipStream_t s) {
    if (m == 0 || n == 0) return hipSuccess;
    GemmParams p{};
    p.a = a; p.b = b; p.m = m; p.n = n; p.k = k;
    p.sinv_a = sinv_a; p.sinv_b = sinv_b; p.bias = bias; p.d = d; p.aux = aux; p.amax = amax;
    p.bias_dtype = bias_dtype; p.d_dtype = d_dtype; p.epilogue = epilogue;
    timing_before(kKindGemm, s);
    const hipError_t e = (epilogue & kEpiFastAccum) ? launch_path<true>(p, afmt, bfmt, s)
                                                    : launch_path<false>(p, afmt, bfmt, s);
    timing_after(s);
    return e;
}

}  // namespace fp8lin
