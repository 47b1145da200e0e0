// HBM-bound elementwise kernels: amax, fused amax+cast, dequant, and the
// batched delayed-scaling update.
//
// Pages (titles in include/fp8lin.h): [TE-KR] "Scaling factor" strategy and
// "FP8 자동변환(Autocasting)" (amax, cast and factor in one step), [TE-RU]
// section 3 (scale before rounding, inverse scale after the GEMM), [PT-VI]
// training script (one history/scale update per step after backward).
//
// Layout: flat tensors, 16-byte aligned.  A lane owns one 16-byte vector per
// step (8 bf16 or 4 fp32 inputs; for dequant the codes of one 16-byte output
// vector), the 64 lanes of a wave own 64 consecutive vectors so every memory
// instruction covers one contiguous KiB, four steps are in flight per lane,
// and waves stride over the tensor; the element tail that does not fill a
// vector is handled one element per thread.  amax is an unsigned max over |x|
// bit patterns: DPP within the wave, LDS across waves, one atomic per
// workgroup.
#include <atomic>

#include "common.h"

namespace fp8lin {
namespace {

constexpr int kThreads = 256;

template <int DT>
__device__ __forceinline__ float load1(const void* x, int64_t i) {
    if constexpr (DT == kF32) return static_cast<const float*>(x)[i];
    return bf16_to_f32(static_cast<const uint16_t*>(x)[i]);
}

// Streaming layout: a lane owns one 16-byte vector of the input per step and
// the 64 lanes of a wave own 64 consecutive vectors (1 KiB), so every load and
// store instruction covers a contiguous range; kU steps are in flight.
constexpr int kU = 4;

template <int DT> struct InVec { static constexpr int elems = DT == kF32 ? 4 : 8; };  // elements per 16 B

// Largest |x| bit pattern among the elements of one 16-byte vector.
template <int DT>
__device__ __forceinline__ uint32_t absmax_vec(uint4 w) {
    if constexpr (DT == kF32) {
        return max(max(w.x & 0x7FFFFFFFu, w.y & 0x7FFFFFFFu), max(w.z & 0x7FFFFFFFu, w.w & 0x7FFFFFFFu));
    } else {
        const uint32_t hi = max(max(w.x & 0x7FFF0000u, w.y & 0x7FFF0000u), max(w.z & 0x7FFF0000u, w.w & 0x7FFF0000u));
        const uint32_t lo = max(max((w.x << 16) & 0x7FFF0000u, (w.y << 16) & 0x7FFF0000u),
                                max((w.z << 16) & 0x7FFF0000u, (w.w << 16) & 0x7FFF0000u));
        return max(hi, lo);
    }
}

// The elements of one 16-byte vector as fp32.
template <int DT>
__device__ __forceinline__ void unpack_vec(uint4 w, float v[InVec<DT>::elems]) {
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

int grid_vec(int64_t nvec) {
    const int64_t per_wg = (int64_t)(kThreads / 64) * 64 * kU;
    const int64_t want = (nvec + per_wg - 1) / per_wg;
    const int64_t cap = 256 * 8;
    return (int)(want < 1 ? 1 : (want > cap ? cap : want));
}

template <int DT>
__global__ void __launch_bounds__(kThreads) k_amax(const void* __restrict__ x, int64_t n, float* slot) {
    __shared__ uint32_t red[kThreads / 64];
    constexpr int E = InVec<DT>::elems;
    const uint4* p = static_cast<const uint4*>(x);
    const int64_t nvec = n / E;
    const int lane = threadIdx.x & 63;
    uint32_t m = 0;
    for (int64_t b = wave_id() * (64 * kU); b < nvec; b += wave_count() * (64 * kU)) {
        uint4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = b + 64 * u + lane;
            v[u] = i < nvec ? p[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) m = max(m, absmax_vec<DT>(v[u]));
    }
    for (int64_t i = nvec * E + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
        m = max(m, abs_bits(load1<DT>(x, i)));
    block_amax_merge(m, slot, red);
}

// Codes of the E elements of one vector, written with one store (4 or 8 bytes).
template <int DT, int FMT>
__device__ __forceinline__ void cast_vec(uint4 w, float s, uint8_t* q, int64_t i, uint32_t& m, bool count,
                                         uint32_t& nsat) {
    constexpr int E = InVec<DT>::elems;
    float v[E];
    unpack_vec<DT>(w, v);
    m = max(m, absmax_vec<DT>(w));
    if (count) nsat += sat_count<FMT, E>(v, s);
    if constexpr (E == 4) {
        reinterpret_cast<uint32_t*>(q)[i] = enc4<FMT>(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
    } else {
        reinterpret_cast<uint2*>(q)[i] = make_uint2(enc4<FMT>(v[0] * s, v[1] * s, v[2] * s, v[3] * s),
                                                    enc4<FMT>(v[4] * s, v[5] * s, v[6] * s, v[7] * s));
    }
}

template <int DT, int FMT>
__global__ void __launch_bounds__(kThreads)
k_cast(const void* __restrict__ x, int64_t n, const float* __restrict__ scale_p, uint8_t* __restrict__ q,
       float* slot, SinvSnap snap, uint32_t* sat) {
    __shared__ uint32_t red[kThreads / 64];
    take_snapshot(snap);
    const bool count = sat != nullptr;
    uint32_t nsat = 0;
    constexpr int E = InVec<DT>::elems;
    const float s = *scale_p;
    const uint4* p = static_cast<const uint4*>(x);
    const int64_t nvec = n / E;
    const int lane = threadIdx.x & 63;
    uint32_t m = 0;
    for (int64_t b = wave_id() * (64 * kU); b < nvec; b += wave_count() * (64 * kU)) {
        uint4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = b + 64 * u + lane;
            v[u] = i < nvec ? p[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = b + 64 * u + lane;
            if (i < nvec) cast_vec<DT, FMT>(v[u], s, q, i, m, count, nsat);
        }
    }
    for (int64_t i = nvec * E + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
        const float v = load1<DT>(x, i);
        m = max(m, abs_bits(v));
        q[i] = (uint8_t)(enc4<FMT>(v * s, 0.0f, 0.0f, 0.0f) & 0xFFu);
        if (count) nsat += sat_count<FMT, 1>(&v, s);
    }
    if (slot) block_amax_merge(m, slot, red);
    if (count) wave_count_add(nsat, sat);
}

// Dequant: a lane decodes the codes of one 16-byte output vector per step (8
// codes to bf16, 4 codes to fp32).
template <int FMT, int OUT>
__global__ void __launch_bounds__(kThreads)
k_dequant(const uint8_t* __restrict__ q, int64_t n, const float* __restrict__ sinv_p, void* __restrict__ out) {
    constexpr int E = OUT == kF32 ? 4 : 8;
    const float si = *sinv_p;
    const int64_t nvec = n / E;
    const int lane = threadIdx.x & 63;
    uint4* o = static_cast<uint4*>(out);
    for (int64_t b = wave_id() * (64 * kU); b < nvec; b += wave_count() * (64 * kU)) {
        uint2 w[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = b + 64 * u + lane;
            if constexpr (E == 8) w[u] = i < nvec ? reinterpret_cast<const uint2*>(q)[i] : make_uint2(0, 0);
            else w[u] = make_uint2(i < nvec ? reinterpret_cast<const uint32_t*>(q)[i] : 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = b + 64 * u + lane;
            if (i >= nvec) continue;
            float v[8];
            dec4<FMT>(w[u].x, v);
            if constexpr (E == 8) dec4<FMT>(w[u].y, v + 4);
#pragma unroll
            for (int j = 0; j < E; ++j) v[j] = v[j] * si;
            if constexpr (E == 4)
                store_nt(o + i, make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                           __float_as_uint(v[3])));
            else
                store_nt(o + i, make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                                           pack_bf16x2(v[6], v[7])));
        }
    }
    for (int64_t i = nvec * E + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
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

// One workgroup per tensor (the scale rule and the roll: scale_update_block).
__global__ void __launch_bounds__(kThreads)
k_scale_update(float* __restrict__ hist, float* __restrict__ scale, float* __restrict__ sinv,
               FmtBits fmts, int32_t L, int32_t margin) {
    __shared__ float red[kThreads / 64];
    const int t = blockIdx.x;
    const bool e5 = (fmts.w[t >> 5] >> (t & 31)) & 1u;
    scale_update_block<false>(hist + (int64_t)t * L, scale + t, sinv + t, e5 ? 57344.0f : 448.0f, L, margin, red);
}

// Just-in-time scaling: the scale of tensor t from its current amax alone
// (slot 0 of its history, `stride` floats apart), a non-finite amax keeping
// the old scale; the history is not rolled.
__global__ void __launch_bounds__(kThreads)
k_scale_from_current(const float* __restrict__ hist, int64_t stride, float* __restrict__ scale,
                     float* __restrict__ sinv, FmtBits fmts, int32_t n, int32_t margin) {
    const int t = blockIdx.x * kThreads + threadIdx.x;
    if (t >= n) return;
    const float a = hist[(int64_t)t * stride];
    const bool e5 = (fmts.w[t >> 5] >> (t & 31)) & 1u;
    const float s = isfinite(a) ? scale_rule(a, e5 ? 57344.0f : 448.0f, margin) : 0.0f;
    if (s > 0.0f) {
        scale[t] = s;
        sinv[t] = __fdiv_rn(1.0f, s);
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

// Shader-clock sample (a measurement aid, not a step of the method): one
// wave reads the shader-clock counter and the constant 100 MHz counter,
// sleeps until `ticks` of the latter have passed (at most 2^22 sleeps of 512
// cycles), reads both again and writes {clock0, clock1, ref0, ref1}.
// Launched on a second stream beside running kernels it gives their clock.
__global__ void __launch_bounds__(64) k_clock_sample(unsigned long long* out, unsigned long long ticks) {
    const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    unsigned long long r = r0;
    for (int i = 0; i < (1 << 22) && r - r0 < ticks; ++i) {
        __builtin_amdgcn_s_sleep(8);
        r = __builtin_amdgcn_s_memrealtime();
    }
    const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        out[0] = c0;
        out[1] = c1;
        out[2] = r0;
        out[3] = r1;
    }
}

// Streaming reference kernels (measurement aids, not steps of the method):
// the same layout and grid as the elementwise kernels above, without their
// arithmetic.  Read: every 16-byte vector of src is loaded and folded into an
// xor per workgroup, written to dst[blockIdx.x] (one word).  Copy: dst = src,
// with plain or non-temporal stores (the latter as the dequant kernel uses).
__global__ void __launch_bounds__(kThreads) k_stream_read(const uint4* __restrict__ p, int64_t nvec,
                                                         uint32_t* __restrict__ dst) {
    __shared__ uint32_t red[kThreads / 64];
    const int lane = threadIdx.x & 63;
    uint32_t x = 0;
    for (int64_t b = wave_id() * (64 * kU); b < nvec; b += wave_count() * (64 * kU)) {
        uint4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = b + 64 * u + lane;
            v[u] = i < nvec ? p[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off);
    if (lane == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kThreads / 64; ++w) x ^= red[w];
        dst[blockIdx.x] = x;
    }
}

// TWICE: each vector is also written nvec vectors further on (one read, two
// writes: the read:write ratio of the dual-format cast and of the dequant).
template <bool NT, bool TWICE = false>
__global__ void __launch_bounds__(kThreads) k_stream_copy(const uint4* __restrict__ p, int64_t nvec,
                                                         uint4* __restrict__ q) {
    const int lane = threadIdx.x & 63;
    for (int64_t b = wave_id() * (64 * kU); b < nvec; b += wave_count() * (64 * kU)) {
        uint4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = b + 64 * u + lane;
            v[u] = i < nvec ? p[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = b + 64 * u + lane;
            if (i < nvec) {
                if constexpr (NT) store_nt(q + i, v[u]);
                else q[i] = v[u];
                if constexpr (TWICE) {
                    if constexpr (NT) store_nt(q + nvec + i, v[u]);
                    else q[nvec + i] = v[u];
                }
            }
        }
    }
}

hipError_t launch_stream_probe(const void* src, void* dst, int64_t bytes, int mode, hipStream_t s) {
    const int64_t nvec = bytes / 16;
    if (nvec == 0) return hipSuccess;
    const int g = grid_vec(nvec);
    timing_before(kKindStream, s);
    if (mode == 0)
        hipLaunchKernelGGL(k_stream_read, dim3(g), dim3(kThreads), 0, s, static_cast<const uint4*>(src), nvec,
                           static_cast<uint32_t*>(dst));
    else if (mode == 1)
        hipLaunchKernelGGL(k_stream_copy<false>, dim3(g), dim3(kThreads), 0, s, static_cast<const uint4*>(src), nvec,
                           static_cast<uint4*>(dst));
    else if (mode == 2)
        hipLaunchKernelGGL(k_stream_copy<true>, dim3(g), dim3(kThreads), 0, s, static_cast<const uint4*>(src), nvec,
                           static_cast<uint4*>(dst));
    else if (mode == 3)
        hipLaunchKernelGGL((k_stream_copy<false, true>), dim3(g), dim3(kThreads), 0, s, static_cast<const uint4*>(src),
                           nvec, static_cast<uint4*>(dst));
    else
        hipLaunchKernelGGL((k_stream_copy<true, true>), dim3(g), dim3(kThreads), 0, s, static_cast<const uint4*>(src),
                           nvec, static_cast<uint4*>(dst));
    timing_after(s);
    return hipGetLastError();
}

// Compute units of the current device (cached per device; callers on several
// host threads may race to fill an entry, with the same value).
int cu_count() {
    static std::atomic<int> cached[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

hipError_t launch_clock_sample(unsigned long long* out, int64_t ticks, hipStream_t s) {
    hipLaunchKernelGGL(k_clock_sample, dim3(1), dim3(64), 0, s, out, (unsigned long long)ticks);
    return hipGetLastError();
}

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
    const int g = grid_vec(n / (dtype == kF32 ? 4 : 8));
    timing_before(kKindAmax, s);
    if (dtype == kF32) hipLaunchKernelGGL(k_amax<kF32>, dim3(g), dim3(kThreads), 0, s, x, n, slot);
    else hipLaunchKernelGGL(k_amax<kBF16>, dim3(g), dim3(kThreads), 0, s, x, n, slot);
    timing_after(s);
    return hipGetLastError();
}

hipError_t launch_cast(const void* x, int dtype, int64_t n, int fmt, const float* scale, uint8_t* q,
                       float* slot, hipStream_t s, SinvSnap snap, SatCounts sat) {
    if (n == 0) return hipSuccess;
    const int g = grid_vec(n / (dtype == kF32 ? 4 : 8));
    timing_before(kKindCast, s);
    if (dtype == kF32 && fmt == kE4M3)
        hipLaunchKernelGGL((k_cast<kF32, kE4M3>), dim3(g), dim3(kThreads), 0, s, x, n, scale, q, slot, snap, sat.a);
    else if (dtype == kF32)
        hipLaunchKernelGGL((k_cast<kF32, kE5M2>), dim3(g), dim3(kThreads), 0, s, x, n, scale, q, slot, snap, sat.a);
    else if (fmt == kE4M3)
        hipLaunchKernelGGL((k_cast<kBF16, kE4M3>), dim3(g), dim3(kThreads), 0, s, x, n, scale, q, slot, snap, sat.a);
    else
        hipLaunchKernelGGL((k_cast<kBF16, kE5M2>), dim3(g), dim3(kThreads), 0, s, x, n, scale, q, slot, snap, sat.a);
    timing_after(s);
    return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* q, int fmt, int64_t n, const float* sinv, void* out, int out_dtype,
                          hipStream_t s) {
    if (n == 0) return hipSuccess;
    const int g = grid_vec(n / (out_dtype == kF32 ? 4 : 8));
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

hipError_t launch_scale_from_current(const float* hist, int64_t stride, float* scale, float* sinv,
                                     const uint8_t* fmts, int32_t n, int32_t margin, hipStream_t s) {
    FmtBits bits{};
    for (int32_t t = 0; t < n; ++t)
        if (fmts[t] == kE5M2) bits.w[t >> 5] |= 1u << (t & 31);
    timing_before(kKindScaleUpdate, s);
    hipLaunchKernelGGL(k_scale_from_current, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, s, hist, stride,
                       scale, sinv, bits, n, margin);
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
