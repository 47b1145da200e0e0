// Loss scaling and the fp32 master-weight update around the FP8 layers.
//
// Pages (titles in include/fp8lin.h): [MP-KR] "Mixed-Precision Training
// Iteration" (scale the loss by S, back-propagate, multiply the weight
// gradients by 1/S, update the fp32 master weights) and the dynamic loss-scale
// procedure on the same page (on Inf/NaN: lower S and skip the update; after N
// clean iterations raise S).  [MP-KR] "FP32 Master Copy of Weights".
//
// The whole state lives on the device (float[4]: S, clean iterations,
// found_inf of the last step, S the last step's gradients carry), so a step
// never waits for the host: the update kernel reads the step's gradient amaxes
// and the SGD kernels read found_inf and S themselves.
#include "common.h"

namespace fp8lin {
namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(64)
k_loss_scale_update(const float* __restrict__ amaxes, int32_t n, int64_t stride, float* __restrict__ state,
                    int32_t interval, float backoff, float growth) {
    int found = 0;
    for (int32_t i = threadIdx.x; i < n; i += 64)
        if (!isfinite(amaxes[(int64_t)i * stride])) found = 1;
    found = __any(found);
    if (threadIdx.x == 0) {
        const float s = state[0];
        state[3] = s;
        state[2] = found ? 1.0f : 0.0f;
        if (found) {
            state[0] = s * backoff;
            state[1] = 0.0f;
        } else {
            const float clean = state[1] + 1.0f;
            if (clean >= (float)interval) {
                state[0] = s * growth;
                state[1] = 0.0f;
            } else {
                state[1] = clean;
            }
        }
    }
}

// Streaming layout as in the elementwise kernels: a lane owns one 16-byte
// vector per step, a wave 64 consecutive vectors, kU steps in flight.
constexpr int kU = 4;

// w <- w - lr * (g * (1/S)), three roundings, skipped when found_inf.
__global__ void __launch_bounds__(kThreads)
k_sgd(float* __restrict__ w, const float* __restrict__ g, int64_t n, float lr, const float* __restrict__ state) {
    if (state[2] != 0.0f) return;
    const float inv = __fdiv_rn(1.0f, state[3]);
    const int64_t n4 = n >> 2;
    float4* w4 = reinterpret_cast<float4*>(w);
    const float4* g4 = reinterpret_cast<const float4*>(g);
    const int lane = threadIdx.x & 63;
    for (int64_t b = wave_id() * (64 * kU); b < n4; b += wave_count() * (64 * kU)) {
        float4 wv[kU], gv[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = b + 64 * u + lane;
            if (i < n4) {
                wv[u] = w4[i];
                gv[u] = g4[i];
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = b + 64 * u + lane;
            if (i < n4) {
                float4 r = wv[u];
                r.x = r.x - lr * (gv[u].x * inv);
                r.y = r.y - lr * (gv[u].y * inv);
                r.z = r.z - lr * (gv[u].z * inv);
                r.w = r.w - lr * (gv[u].w * inv);
                w4[i] = r;
            }
        }
    }
    for (int64_t i = (n4 << 2) + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
        w[i] = w[i] - lr * (g[i] * inv);
}

// out = round(x * S), elementwise, in x's element type.
template <int DT>
__global__ void __launch_bounds__(kThreads)
k_scale_by(const void* __restrict__ x, int64_t n, const float* __restrict__ state, void* __restrict__ out) {
    constexpr int E = DT == kF32 ? 4 : 8;          // elements per 16-byte vector
    const float s = state[0];
    const int64_t nv = n / E;
    const uint4* xv = static_cast<const uint4*>(x);
    uint4* ov = static_cast<uint4*>(out);
    const int lane = threadIdx.x & 63;
    for (int64_t b = wave_id() * (64 * kU); b < nv; b += wave_count() * (64 * kU)) {
        uint4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = b + 64 * u + lane;
            v[u] = i < nv ? xv[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = b + 64 * u + lane;
            if (i >= nv) continue;
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            uint32_t o[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                if constexpr (DT == kF32) o[h] = __float_as_uint(__uint_as_float(w[h]) * s);
                else o[h] = pack_bf16x2(__uint_as_float(w[h] << 16) * s, __uint_as_float(w[h] & 0xFFFF0000u) * s);
            }
            ov[i] = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
    for (int64_t i = nv * E + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
        if constexpr (DT == kF32) {
            static_cast<float*>(out)[i] = static_cast<const float*>(x)[i] * s;
        } else {
            const float v = bf16_to_f32(static_cast<const uint16_t*>(x)[i]) * s;
            static_cast<uint16_t*>(out)[i] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
        }
    }
}

// Workgroups for `nvec` 16-byte vectors: one step of kU vectors per lane, at
// most 8 workgroups per CU.
int grid_of(int64_t nvec) {
    const int64_t per_wg = (int64_t)kThreads * kU;
    const int64_t want = (nvec + per_wg - 1) / per_wg;
    return (int)(want < 1 ? 1 : (want > 256 * 8 ? 256 * 8 : want));
}

}  // namespace

hipError_t launch_loss_scale_update(const float* amaxes, int32_t n, int64_t stride, float* state,
                                    int32_t interval, float backoff, float growth, hipStream_t s) {
    timing_before(kKindOther, s);
    hipLaunchKernelGGL(k_loss_scale_update, dim3(1), dim3(64), 0, s, amaxes, n, stride, state, interval, backoff,
                       growth);
    timing_after(s);
    return hipGetLastError();
}

hipError_t launch_sgd(float* w, const float* g, int64_t n, float lr, const float* state, hipStream_t s) {
    if (n == 0) return hipSuccess;
    timing_before(kKindSgd, s);
    hipLaunchKernelGGL(k_sgd, dim3(grid_of(n >> 2)), dim3(kThreads), 0, s, w, g, n, lr, state);
    timing_after(s);
    return hipGetLastError();
}

hipError_t launch_scale_by(const void* x, int dtype, int64_t n, const float* state, void* out, hipStream_t s) {
    if (n == 0) return hipSuccess;
    timing_before(kKindOther, s);
    if (dtype == kF32)
        hipLaunchKernelGGL(k_scale_by<kF32>, dim3(grid_of(n >> 2)), dim3(kThreads), 0, s, x, n, state, out);
    else
        hipLaunchKernelGGL(k_scale_by<kBF16>, dim3(grid_of(n >> 3)), dim3(kThreads), 0, s, x, n, state, out);
    timing_after(s);
    return hipGetLastError();
}

}  // namespace fp8lin
