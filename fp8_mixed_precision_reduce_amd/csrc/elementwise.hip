// HBM-bound elementwise kernels: amax, fused amax+cast, dequant, and the
// batched delayed-scaling update.
//
// Pages (titles in include/fp8lin.h): [TE-KR] "Scaling factor" strategy and
// "FP8 자동변환(Autocasting)" (amax, cast and factor in one step), [TE-RU]
// section 3 (scale before rounding, inverse scale after the GEMM), [PT-VI]
// training script (one history/scale update per step after backward).
//
// Layout: flat tensors, 16-byte aligned.  A thread owns 16 consecutive
// elements per iteration (one 16-byte FP8 store; 32 or 64 bytes of input), a
// grid-stride loop covers the tensor with two chunks in flight per thread, and
// the element tail (n % 16) is handled one element per thread.  amax is an
// unsigned max over |x| bit patterns: DPP within the wave, LDS across waves,
// one atomic per workgroup.
#include "common.h"

namespace fp8lin {
namespace {

constexpr int kThreads = 256;

int grid_for(int64_t chunks) {
    // Enough workgroups to cover every CU several times, not more than the chunks need.
    const int64_t want = (chunks + 2 * kThreads - 1) / (2 * kThreads);
    const int64_t cap = 256 * 8;
    return (int)(want < 1 ? 1 : (want > cap ? cap : want));
}

template <int DT>
__device__ __forceinline__ float load1(const void* x, int64_t i) {
    if constexpr (DT == kF32) return static_cast<const float*>(x)[i];
    return bf16_to_f32(static_cast<const uint16_t*>(x)[i]);
}

template <int DT>
__global__ void __launch_bounds__(kThreads) k_amax(const void* __restrict__ x, int64_t n, float* slot) {
    __shared__ uint32_t red[kThreads / 64];
    const int64_t chunks = n >> 4;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    uint32_t m = 0;
    int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; c + stride < chunks; c += 2 * stride) {
        float a[16], b[16];
        load16<DT>(x, c << 4, a);
        load16<DT>(x, (c + stride) << 4, b);
#pragma unroll
        for (int j = 0; j < 16; ++j) m = max(m, max(abs_bits(a[j]), abs_bits(b[j])));
    }
    if (c < chunks) {
        float a[16];
        load16<DT>(x, c << 4, a);
#pragma unroll
        for (int j = 0; j < 16; ++j) m = max(m, abs_bits(a[j]));
    }
    for (int64_t i = (chunks << 4) + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
        m = max(m, abs_bits(load1<DT>(x, i)));
    block_amax_merge(m, slot, red);
}

template <int DT, int FMT>
__global__ void __launch_bounds__(kThreads)
k_cast(const void* __restrict__ x, int64_t n, const float* __restrict__ scale_p, uint8_t* __restrict__ q,
       float* slot) {
    __shared__ uint32_t red[kThreads / 64];
    const float s = *scale_p;
    const int64_t chunks = n >> 4;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    uint32_t m = 0;
    int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; c + stride < chunks; c += 2 * stride) {
        float a[16], b[16];
        load16<DT>(x, c << 4, a);
        load16<DT>(x, (c + stride) << 4, b);
#pragma unroll
        for (int j = 0; j < 16; ++j) m = max(m, max(abs_bits(a[j]), abs_bits(b[j])));
        reinterpret_cast<uint4*>(q)[c] = scale_enc16<FMT>(a, s);
        reinterpret_cast<uint4*>(q)[c + stride] = scale_enc16<FMT>(b, s);
    }
    if (c < chunks) {
        float a[16];
        load16<DT>(x, c << 4, a);
#pragma unroll
        for (int j = 0; j < 16; ++j) m = max(m, abs_bits(a[j]));
        reinterpret_cast<uint4*>(q)[c] = scale_enc16<FMT>(a, s);
    }
    for (int64_t i = (chunks << 4) + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
        const float v = load1<DT>(x, i);
        m = max(m, abs_bits(v));
        q[i] = (uint8_t)(enc4<FMT>(v * s, 0.0f, 0.0f, 0.0f) & 0xFFu);
    }
    if (slot) block_amax_merge(m, slot, red);
}

template <int FMT, int OUT>
__global__ void __launch_bounds__(kThreads)
k_dequant(const uint8_t* __restrict__ q, int64_t n, const float* __restrict__ sinv_p, void* __restrict__ out) {
    const float si = *sinv_p;
    const int64_t chunks = n >> 4;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    auto emit = [&](int64_t c, uint4 w) {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        float v[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) dec4<FMT>(ws[j], v + 4 * j);
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = v[j] * si;
        if constexpr (OUT == kF32) {
            uint4* o = reinterpret_cast<uint4*>(static_cast<float*>(out) + (c << 4));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[j] = make_uint4(__float_as_uint(v[4 * j]), __float_as_uint(v[4 * j + 1]),
                                  __float_as_uint(v[4 * j + 2]), __float_as_uint(v[4 * j + 3]));
        } else {
            uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + (c << 4));
#pragma unroll
            for (int j = 0; j < 2; ++j)
                o[j] = make_uint4(pack_bf16x2(v[8 * j], v[8 * j + 1]), pack_bf16x2(v[8 * j + 2], v[8 * j + 3]),
                                  pack_bf16x2(v[8 * j + 4], v[8 * j + 5]), pack_bf16x2(v[8 * j + 6], v[8 * j + 7]));
        }
    };
    int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; c + stride < chunks; c += 2 * stride) {
        const uint4 w0 = reinterpret_cast<const uint4*>(q)[c];
        const uint4 w1 = reinterpret_cast<const uint4*>(q)[c + stride];
        emit(c, w0);
        emit(c + stride, w1);
    }
    if (c < chunks) emit(c, reinterpret_cast<const uint4*>(q)[c]);
    for (int64_t i = (chunks << 4) + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
        float v[4];
        dec4<FMT>((uint32_t)q[i], v);
        const float r = v[0] * si;
        if constexpr (OUT == kF32) static_cast<float*>(out)[i] = r;
        else static_cast<uint16_t*>(out)[i] = (uint16_t)(pack_bf16x2(r, 0.0f) & 0xFFFFu);
    }
}

// Per-tensor format bits travel as kernel arguments (bit t set = E5M2).
constexpr int kMaxTensors = 4096;
struct FmtBits { uint32_t w[kMaxTensors / 32]; };

// One workgroup per tensor: max over the finite history entries, the scale
// rule, then the roll h[i] <- h[i-1], h[0] <- 0 done top-down in chunks of
// 256 so every read of a chunk precedes the writes that could clobber it.
__global__ void __launch_bounds__(kThreads)
k_scale_update(float* __restrict__ hist, float* __restrict__ scale, float* __restrict__ sinv,
               FmtBits fmts, int32_t L, int32_t margin) {
    __shared__ float red[kThreads / 64];
    const int t = blockIdx.x;
    float* h = hist + (int64_t)t * L;
    float m = -INFINITY;
    for (int i = threadIdx.x; i < L; i += kThreads) {
        const float v = h[i];
        if (isfinite(v)) m = fmaxf(m, v);
    }
    // wave then block max (floats; -inf marks "no finite entry")
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float a = red[0];
        for (int w = 1; w < kThreads / 64; ++w) a = fmaxf(a, red[w]);
        if (a > 0.0f) {
            const bool e5 = (fmts.w[t >> 5] >> (t & 31)) & 1u;
            const float fmax = e5 ? 57344.0f : 448.0f;
            float s = __fdiv_rn(fmax, a);
            s = ldexpf(s, -margin);
            if (isinf(s)) s = 3.402823466e+38f;
            if (s > 0.0f) {
                scale[t] = s;
                sinv[t] = __fdiv_rn(1.0f, s);
            }
        }
    }
    __syncthreads();
    for (int base = ((L - 1) / kThreads) * kThreads; base >= 0; base -= kThreads) {
        const int i = base + threadIdx.x;
        float prev = 0.0f;
        if (i < L && i > 0) prev = h[i - 1];
        __syncthreads();
        if (i < L) h[i] = prev;
        __syncthreads();
    }
}

__global__ void k_copy_scalars(const float* a, const float* b, float* dst) {
    if (threadIdx.x == 0) {
        dst[0] = *a;
        dst[1] = *b;
    }
}

// Fill with zeros (a kernel rather than a memset so the work can sit in a
// captured HIP graph).
__global__ void __launch_bounds__(kThreads) k_zero_f32(float* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
        p[i] = 0.0f;
}

}  // namespace

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const int64_t want = (n + kThreads - 1) / kThreads;
    const int g = (int)(want > 4096 ? 4096 : want);
    timing_before(kKindOther, s);
    hipLaunchKernelGGL(k_zero_f32, dim3(g), dim3(kThreads), 0, s, p, n);
    timing_after(s);
    return hipGetLastError();
}

hipError_t launch_amax(const void* x, int dtype, int64_t n, float* slot, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const int g = grid_for((n + 15) >> 4);
    timing_before(kKindAmax, s);
    if (dtype == kF32) hipLaunchKernelGGL(k_amax<kF32>, dim3(g), dim3(kThreads), 0, s, x, n, slot);
    else hipLaunchKernelGGL(k_amax<kBF16>, dim3(g), dim3(kThreads), 0, s, x, n, slot);
    timing_after(s);
    return hipGetLastError();
}

hipError_t launch_cast(const void* x, int dtype, int64_t n, int fmt, const float* scale, uint8_t* q,
                       float* slot, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const int g = grid_for((n + 15) >> 4);
    timing_before(kKindCast, s);
    if (dtype == kF32 && fmt == kE4M3)
        hipLaunchKernelGGL((k_cast<kF32, kE4M3>), dim3(g), dim3(kThreads), 0, s, x, n, scale, q, slot);
    else if (dtype == kF32)
        hipLaunchKernelGGL((k_cast<kF32, kE5M2>), dim3(g), dim3(kThreads), 0, s, x, n, scale, q, slot);
    else if (fmt == kE4M3)
        hipLaunchKernelGGL((k_cast<kBF16, kE4M3>), dim3(g), dim3(kThreads), 0, s, x, n, scale, q, slot);
    else
        hipLaunchKernelGGL((k_cast<kBF16, kE5M2>), dim3(g), dim3(kThreads), 0, s, x, n, scale, q, slot);
    timing_after(s);
    return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* q, int fmt, int64_t n, const float* sinv, void* out, int out_dtype,
                          hipStream_t s) {
    if (n == 0) return hipSuccess;
    const int g = grid_for((n + 15) >> 4);
    timing_before(kKindDequant, s);
    if (fmt == kE4M3 && out_dtype == kF32)
        hipLaunchKernelGGL((k_dequant<kE4M3, kF32>), dim3(g), dim3(kThreads), 0, s, q, n, sinv, out);
    else if (fmt == kE4M3)
        hipLaunchKernelGGL((k_dequant<kE4M3, kBF16>), dim3(g), dim3(kThreads), 0, s, q, n, sinv, out);
    else if (out_dtype == kF32)
        hipLaunchKernelGGL((k_dequant<kE5M2, kF32>), dim3(g), dim3(kThreads), 0, s, q, n, sinv, out);
    else
        hipLaunchKernelGGL((k_dequant<kE5M2, kBF16>), dim3(g), dim3(kThreads), 0, s, q, n, sinv, out);
    timing_after(s);
    return hipGetLastError();
}

hipError_t launch_scale_update(float* hist, float* scale, float* sinv, const uint8_t* fmts, int32_t n,
                               int32_t L, int32_t margin, hipStream_t s) {
    FmtBits bits = {};
    for (int32_t t = 0; t < n; ++t)
        if (fmts[t] == kE5M2) bits.w[t >> 5] |= 1u << (t & 31);
    timing_before(kKindScaleUpdate, s);
    hipLaunchKernelGGL(k_scale_update, dim3(n), dim3(kThreads), 0, s, hist, scale, sinv, bits, L, margin);
    timing_after(s);
    return hipGetLastError();
}

hipError_t launch_copy_scalars(const float* a, const float* b, float* dst2, hipStream_t s) {
    timing_before(kKindOther, s);
    hipLaunchKernelGGL(k_copy_scalars, dim3(1), dim3(64), 0, s, a, b, dst2);
    timing_after(s);
    return hipGetLastError();
}

}  // namespace fp8lin
