// Device helpers and launcher declarations shared by the kernels of libfp8lin.
//
// Everything here is written for gfx950 (CDNA4): 64-lane waves, the OCP FP8
// hardware converts, DPP lane shuffles, buffer resources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8lin {

enum Dtype : int32_t { kF32 = 0, kBF16 = 1, kE4M3 = 2, kE5M2 = 3 };

// Kinds of kernels, as reported by the event timer.
enum Kind : int32_t { kKindAmax = 0, kKindCast = 1, kKindCastT = 2, kKindDequant = 3,
                      kKindScaleUpdate = 4, kKindGemm = 5, kKindDbias = 6, kKindOther = 7, kKindSgd = 8,
                      kKindAttn = 9, kKindStream = 10 };

// Host side: record events around a launch when timing is enabled.
void timing_before(int kind, hipStream_t stream);
void timing_after(hipStream_t stream);

// A cast kernel can also take the forward's snapshot of the two inverse scales
// (the backward uses the values the forward multiplied with): workgroup 0,
// thread 0 copies *a and *b to dst[0], dst[1].  dst == nullptr: no snapshot.
struct SinvSnap {
    const float* a;
    const float* b;
    float* dst;
};
// Saturation counters of a cast (fp8lin_count_saturation): device counters
// that the cast adds its number of saturated elements to -- those whose scaled
// value fl32(x * scale) exceeds the format's largest finite magnitude, the
// values the saturating encode clamps.  nullptr: not counted.
struct SatCounts {
    uint32_t* a = nullptr;     // the tensor (dual cast: its E4M3 copy; pair cast: the first tensor)
    uint32_t* b = nullptr;     // dual cast: the E5M2 copy; pair cast: the second tensor
};
#ifdef __HIPCC__
__device__ __forceinline__ void take_snapshot(const SinvSnap& snap) {
    if (snap.dst && blockIdx.x == 0 && threadIdx.x == 0) {
        snap.dst[0] = *snap.a;
        snap.dst[1] = *snap.b;
    }
}
#endif

// Compute units of the current device (the persistent kernels size their grids by it).
int cu_count();

// ------------------------------------------------------------------ launchers
// Each returns the hipError_t of its launch.  Arguments are validated by the
// C entry points before these are called.
hipError_t launch_amax(const void* x, int dtype, int64_t n, float* slot, hipStream_t s);
hipError_t launch_cast(const void* x, int dtype, int64_t n, int fmt, const float* scale,
                       uint8_t* q, float* slot, hipStream_t s, SinvSnap snap = {}, SatCounts sat = {});
hipError_t launch_dequant(const uint8_t* q, int fmt, int64_t n, const float* sinv, void* out,
                          int out_dtype, hipStream_t s);
hipError_t launch_scale_update(float* hist, float* scale, float* sinv, const uint8_t* fmts,
                               int32_t n, int32_t L, int32_t margin, hipStream_t s);
hipError_t launch_scale_from_current(const float* hist, int64_t stride, float* scale, float* sinv,
                                     const uint8_t* fmts, int32_t n, int32_t margin, hipStream_t s);
hipError_t launch_copy_scalars(const float* a, const float* b, float* dst2, hipStream_t s);
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s);
hipError_t launch_clock_sample(unsigned long long* out, int64_t ticks, hipStream_t s);
hipError_t launch_stream_probe(const void* src, void* dst, int64_t bytes, int mode, hipStream_t s);
hipError_t launch_cast_transpose(const void* x, const void* z, int dtype, int64_t rows, int64_t cols,
                                 int fmt, const float* scale, uint8_t* q, uint8_t* qt, float* slot,
                                 float* dbias, float* dbias_ws, void* dz_out, hipStream_t s, SinvSnap snap = {},
                                 SatCounts sat = {});
// The fp32 weight matrix w [rows][cols] updated by SGD (as launch_sgd) and
// cast-transposed to E4M3 in the same pass (the cast the next forward needs).
hipError_t launch_sgd_cast_transpose(float* w, const float* g, int64_t rows, int64_t cols, float lr,
                                     const float* state, const float* scale, uint8_t* q, uint8_t* qt, float* slot,
                                     hipStream_t s, SatCounts sat = {});
// Two non-empty tensors of one element type cast to one format in one launch.
hipError_t launch_cast_transpose_pair(const void* xa, const void* xb, int dtype, int64_t rows_a, int64_t cols_a,
                                      int64_t rows_b, int64_t cols_b, int fmt, const float* scale_a, uint8_t* q_a,
                                      uint8_t* qt_a, float* slot_a, const float* scale_b, uint8_t* q_b, uint8_t* qt_b,
                                      float* slot_b, hipStream_t s, SinvSnap snap, SatCounts sat = {});
hipError_t launch_cast_transpose_dual(const void* x, int dtype, int64_t rows, int64_t cols, const float* scale_e4m3,
                                      uint8_t* q_e4m3, uint8_t* q_e4m3_t, float* slot_e4m3, const float* scale_e5m2,
                                      uint8_t* q_e5m2, uint8_t* q_e5m2_t, float* slot_e5m2, hipStream_t s,
                                      SatCounts sat = {});
// The dual-format cast-transpose into a bank of two metas (0: E4M3, 1: E5M2,
// histories hist[2][L]) whose last workgroup then runs the scale update of
// both; `ticket` is a device counter that is zero before and after.
hipError_t launch_cast_transpose_dual_update(const void* x, int dtype, int64_t rows, int64_t cols, uint8_t* q_e4m3,
                                             uint8_t* q_e4m3_t, uint8_t* q_e5m2, uint8_t* q_e5m2_t, float* hist,
                                             float* scale, float* sinv, int32_t L, int32_t margin,
                                             unsigned int* ticket, hipStream_t s, SatCounts sat = {});
int64_t cast_transpose_dbias_ws_bytes(int64_t rows, int64_t cols);
// The scratch array of fp8_cast_transpose_dbias_noalloc on the device of
// stream s (its address is looked up once per device).
constexpr int64_t kNoAllocScratchBytes = int64_t(8) << 20;
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(hipStream_t s, float** out);
hipError_t launch_gemm(const uint8_t* a, int afmt, const uint8_t* b, int bfmt, int64_t m, int64_t n,
                       int64_t k, const float* sinv_a, const float* sinv_b, const void* bias,
                       int bias_dtype, int epilogue, void* d, int d_dtype, void* aux, const void* residual,
                       float* amax, const float* q_scale, uint8_t* q, uint8_t* qt, int q_fmt, hipStream_t s);
hipError_t launch_loss_scale_update(const float* amaxes, int32_t n, int64_t stride, float* state,
                                    int32_t interval, float backoff, float growth, hipStream_t s);
hipError_t launch_sgd(float* w, const float* g, int64_t n, float lr, const float* state, hipStream_t s);
hipError_t launch_scale_by(const void* x, int dtype, int64_t n, const float* state, void* out, hipStream_t s);
hipError_t launch_attention_fwd(const uint16_t* qkv, int64_t batch, int64_t seq, int64_t heads, uint16_t* ctx,
                                float* lse, uint16_t* vt_ws, hipStream_t s);
hipError_t launch_attention_bwd(const uint16_t* qkv, const uint16_t* ctx, const float* lse, const uint16_t* dctx,
                                int64_t batch, int64_t seq, int64_t heads, uint16_t* dqkv, uint16_t* qt_ws,
                                uint16_t* dot_ws, float* rows_ws, hipStream_t s);

#ifdef __HIPCC__
// ------------------------------------------------------------ device helpers

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Two fp32 values to two bf16 (round to nearest-even) packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float round_to_bf16(float v) {
    return bf16_to_f32(pack_bf16x2(v, 0.0f) & 0xFFFFu);
}

template <int FMT> struct Fp8Max;
template <> struct Fp8Max<kE4M3> { static constexpr float value = 448.0f; };
template <> struct Fp8Max<kE5M2> { static constexpr float value = 57344.0f; };

// Number of the E values whose product with s exceeds the format's largest
// finite magnitude (the same fp32 products the encode rounds; NaN not counted).
template <int FMT, int E>
__device__ __forceinline__ uint32_t sat_count(const float* v, float s) {
    uint32_t n = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) n += fabsf(v[j] * s) > Fp8Max<FMT>::value ? 1u : 0u;
    return n;
}

// Sum a per-thread count over the wave and add it to a device counter (one
// atomic per wave, none for a zero sum).  Every lane of the wave must call it.
__device__ __forceinline__ void wave_count_add(uint32_t v, uint32_t* ctr) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0 && v != 0u) atomicAdd(ctr, v);
}

// Saturating clamp, one median-of-three: |p| >= max -> +-max, any other
// non-NaN p (-0 and subnormals included) unchanged.  A NaN p comes out as some
// finite value; the encoders below replace its code.
template <int FMT>
__device__ __forceinline__ float sat_fp8(float p) {
    return __builtin_amdgcn_fmed3f(p, -Fp8Max<FMT>::value, Fp8Max<FMT>::value);
}

// Encode four fp32 values (already scaled) into four codes, byte i = value i.
// The hardware converts round to nearest-even; the clamp gives saturation and
// NaN is mapped to sign|0x7F explicitly.  any_nan: set when one of the four
// values is NaN.
template <int FMT>
__device__ __forceinline__ uint32_t enc4(float a, float b, float c, float d, bool& any_nan) {
    const float sa = sat_fp8<FMT>(a), sb = sat_fp8<FMT>(b), sc = sat_fp8<FMT>(c), sd = sat_fp8<FMT>(d);
    int v;
    if constexpr (FMT == kE4M3) {
        v = __builtin_amdgcn_cvt_pk_fp8_f32(sa, sb, 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(sc, sd, v, true);
    } else {
        v = __builtin_amdgcn_cvt_pk_bf8_f32(sa, sb, 0, false);
        v = __builtin_amdgcn_cvt_pk_bf8_f32(sc, sd, v, true);
    }
    uint32_t r = (uint32_t)v;
    const bool na = a != a, nb = b != b, nc = c != c, nd = d != d;
    any_nan = na | nb | nc | nd;
    if (__builtin_expect(any_nan, 0)) {
        const uint32_t nan_mask = (na ? 0xFFu : 0u) | (nb ? 0xFF00u : 0u) | (nc ? 0xFF0000u : 0u) |
                                  (nd ? 0xFF000000u : 0u);
        const uint32_t signs = ((__float_as_uint(a) >> 31) << 7) | ((__float_as_uint(b) >> 31) << 15) |
                               ((__float_as_uint(c) >> 31) << 23) | ((__float_as_uint(d) >> 31) << 31);
        r = (r & ~nan_mask) | (nan_mask & (0x7F7F7F7Fu | signs));
    }
    return r;
}
template <int FMT>
__device__ __forceinline__ uint32_t enc4(float a, float b, float c, float d) {
    bool any_nan;
    return enc4<FMT>(a, b, c, d, any_nan);
}

// Decode four codes (bytes of w) to fp32, exactly.
template <int FMT>
__device__ __forceinline__ void dec4(uint32_t w, float out[4]) {
    f32x2 lo, hi;
    if constexpr (FMT == kE4M3) {
        lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
        hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    } else {
        lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
        hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
    }
    out[0] = lo.x; out[1] = lo.y; out[2] = hi.x; out[3] = hi.y;
}

// Global wave index and wave count of a 1-D launch.
__device__ __forceinline__ int64_t wave_id() {
    return (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
}
__device__ __forceinline__ int64_t wave_count() { return (int64_t)gridDim.x * (blockDim.x >> 6); }

// Non-temporal (streaming) 16-byte global store: for outputs that no kernel
// of the same step reads back soon (measured: dequant of 2^28 codes to bf16
// 147 -> 118 us; no gain for the casts that feed the next GEMM).
typedef unsigned int ntu4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt(uint4* p, uint4 v) {
    __builtin_nontemporal_store(ntu4{v.x, v.y, v.z, v.w}, reinterpret_cast<ntu4*>(p));
}

// |x| as an unsigned bit pattern: the amax statistic compares these.
__device__ __forceinline__ uint32_t abs_bits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// The delayed-scaling scale rule: s = fl32(fl32(fp8_max / a) * 2^-margin),
// FLT_MAX if that overflowed; 0 means "keep the old scale" (a not > 0, or s
// underflowed).
__device__ __forceinline__ float scale_rule(float a, float fmax, int32_t margin) {
    if (!(a > 0.0f)) return 0.0f;
    float s = __fdiv_rn(fmax, a);
    s = ldexpf(s, -margin);
    if (isinf(s)) s = 3.402823466e+38f;
    return s;
}

// The per-step update of one tensor's meta by one workgroup (every thread
// calls it): the max over the finite history entries, the scale rule, then
// the roll h[i] <- h[i-1], h[0] <- 0, done top-down in chunks of blockDim.x
// so every read of a chunk precedes the writes that could clobber it.
// COHERENT reads the history with device-scope loads (for entries other
// workgroups of the same launch merged into).  red: LDS, blockDim.x / 64 floats.
template <bool COHERENT>
__device__ __forceinline__ float load_hist(const float* p) {
    if constexpr (COHERENT)
        return __uint_as_float(__hip_atomic_load(reinterpret_cast<const unsigned int*>(p), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT));
    else
        return *p;
}

template <bool COHERENT>
__device__ __forceinline__ void scale_update_block(float* h, float* scale, float* sinv, float fmax, int32_t L,
                                                   int32_t margin, float* red) {
    const int nt = (int)blockDim.x;
    float m = -INFINITY;
    for (int i = threadIdx.x; i < L; i += nt) {
        const float v = load_hist<COHERENT>(h + i);
        if (isfinite(v)) m = fmaxf(m, v);
    }
    // wave then block max (floats; -inf marks "no finite entry")
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float a = red[0];
        for (int w = 1; w < nt / 64; ++w) a = fmaxf(a, red[w]);
        const float s = scale_rule(a, fmax, margin);
        if (s > 0.0f) {
            *scale = s;
            *sinv = __fdiv_rn(1.0f, s);
        }
    }
    __syncthreads();
    for (int base = ((L - 1) / nt) * nt; base >= 0; base -= nt) {
        const int i = base + threadIdx.x;
        float prev = 0.0f;
        if (i < L && i > 0) prev = load_hist<COHERENT>(h + i - 1);
        __syncthreads();
        if (i < L) h[i] = prev;
        __syncthreads();
    }
}

// Max over the 64 lanes of a wave: DPP within each row of 16 lanes, then the
// four row results through readlane.  Every lane returns the wave maximum.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));  // row_mirror
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// Max-merge a per-thread amax into a device slot: at most one atomic per
// workgroup, and none when the slot already holds a value at least as large
// (the slot only grows, so skipping is exact).  Atomics on one address are
// serialised in L2; without the check thousands of short workgroups queue on
// them.  `red` is LDS scratch of at least (blockDim.x / 64) words.  All
// threads of the block must call it.
__device__ __forceinline__ void block_amax_merge(uint32_t v, float* slot, uint32_t* red) {
    v = wave_max_u32(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t m = 0;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) m = max(m, red[w]);
        unsigned int* s = reinterpret_cast<unsigned int*>(slot);
        if (m != 0u && m > __hip_atomic_load(s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(s, m);
    }
}

// Load 16 consecutive elements (16-byte aligned) as fp32.
template <int DT>
__device__ __forceinline__ void load16(const void* base, int64_t idx, float v[16]) {
    if constexpr (DT == kF32) {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + idx);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 u = p[j];
            v[4 * j + 0] = __uint_as_float(u.x); v[4 * j + 1] = __uint_as_float(u.y);
            v[4 * j + 2] = __uint_as_float(u.z); v[4 * j + 3] = __uint_as_float(u.w);
        }
    } else {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint4 u = p[j];
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[8 * j + 2 * h + 0] = __uint_as_float(w[h] << 16);
                v[8 * j + 2 * h + 1] = __uint_as_float(w[h] & 0xFFFF0000u);
            }
        }
    }
}

// Encode 16 fp32 values times `s` into 16 codes.
template <int FMT>
__device__ __forceinline__ uint4 scale_enc16(const float v[16], float s) {
    uint4 r;
    r.x = enc4<FMT>(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
    r.y = enc4<FMT>(v[4] * s, v[5] * s, v[6] * s, v[7] * s);
    r.z = enc4<FMT>(v[8] * s, v[9] * s, v[10] * s, v[11] * s);
    r.w = enc4<FMT>(v[12] * s, v[13] * s, v[14] * s, v[15] * s);
    return r;
}

// exp(a) that keeps subnormal results: the hardware exponential flushes them,
// so far-negative arguments are shifted by 64 ln 2 and the result is scaled
// back exactly with ldexp (which rounds into the subnormal range).
__device__ __forceinline__ float exp_sub(float a) {
    return a < -80.0f ? ldexpf(__expf(a + 44.361419555836500f), -64) : __expf(a);
}

// Phi(-|z|), the lower tail of the standard normal CDF, as erfc(|z|/sqrt 2)/2
// with the Chebyshev-fitted complementary error function of Press et al.,
// Numerical Recipes (erfcc): erfc(x) = t exp(-x^2 + P(t)), t = 1 / (1 + x/2),
// P a degree-9 polynomial; fractional error below 1.2e-7 for every x >= 0.
// One reciprocal, one exponential and nine FMAs, against several times that
// for the library erfcf; the tail keeps its relative precision.
__device__ __forceinline__ float normal_lower_tail(float z) {
    const float x = fabsf(z) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, x, 1.0f));
    float p = 0.17087277f;
    p = fmaf(p, t, -0.82215223f);
    p = fmaf(p, t, 1.48851587f);
    p = fmaf(p, t, -1.13520398f);
    p = fmaf(p, t, 0.27886807f);
    p = fmaf(p, t, -0.18628806f);
    p = fmaf(p, t, 0.09678418f);
    p = fmaf(p, t, 0.37409196f);
    p = fmaf(p, t, 1.00002368f);
    p = fmaf(p, t, -1.26551223f);
    return 0.5f * t * exp_sub(fmaf(-x, x, p));
}

// gelu(z) = z * Phi(z) (exact erf form), fp32.
__device__ __forceinline__ float gelu_f32(float z) {
    const float lt = normal_lower_tail(z);
    return z * (z < 0.0f ? lt : 1.0f - lt);
}

// gelu'(z) = Phi(z) + z * phi(z), fp32.
__device__ __forceinline__ float gelu_grad_f32(float z) {
    const float lt = normal_lower_tail(z);
    const float cdf = z < 0.0f ? lt : 1.0f - lt;
    const float pdf = exp_sub(-0.5f * z * z) * 0.39894228040143268f;
    return cdf + z * pdf;
}
#endif  // __HIPCC__

}  // namespace fp8lin
