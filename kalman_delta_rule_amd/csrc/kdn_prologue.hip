// kdn_prologue.hip -- the gates of the end-to-end network from their
// pre-activations, gfx950.
//
// KDN reading notes, method part §8: alpha = sigmoid(a), omega = softplus(w)
// (per channel for Diagonal, per token for Isotropic) and
// r = r_min + softplus(rho).  An elementwise, HBM-bound pass: each thread
// turns 8 consecutive pre-activations (16 bytes of bf16 or 32 of fp32) into
// 8 fp32 gates, and the forward then reads the gates as usual.
// The activations are the shared gate_sigmoid / gate_softplus, so that
// these gates equal, bit for bit, the ones the bf16 forward forms itself
// when it reads the pre-activations directly.
#include "kdn_common.h"
#include "kdn_internal.h"
#include "kdn_ops.h"

namespace kdn {

template <int ACT>
__device__ __forceinline__ float gate_act(float x, float add)
{
    if constexpr (ACT == 0)
        return gate_sigmoid(x);
    else
        return gate_softplus(x, add);
}

template <typename IO, int ACT>
__global__ __launch_bounds__(256) void kdn_gate_prologue_kernel(const IO* __restrict__ x,
                                                                float* __restrict__ y, size_t n,
                                                                float add)
{
    const size_t i0 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i0 + 8 <= n) {
        float v[8];
        if constexpr (sizeof(IO) == 2) {
            const uint4 raw = *reinterpret_cast<const uint4*>(x + i0);
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[2 * j] = __builtin_bit_cast(float, w[j] << 16);
                v[2 * j + 1] = __builtin_bit_cast(float, w[j] & 0xFFFF0000u);
            }
        } else {
            const float4 a = *reinterpret_cast<const float4*>(x + i0);
            const float4 b = *reinterpret_cast<const float4*>(x + i0 + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        }
        float4 o0, o1;
        o0.x = gate_act<ACT>(v[0], add); o0.y = gate_act<ACT>(v[1], add);
        o0.z = gate_act<ACT>(v[2], add); o0.w = gate_act<ACT>(v[3], add);
        o1.x = gate_act<ACT>(v[4], add); o1.y = gate_act<ACT>(v[5], add);
        o1.z = gate_act<ACT>(v[6], add); o1.w = gate_act<ACT>(v[7], add);
        *reinterpret_cast<float4*>(y + i0) = o0;
        *reinterpret_cast<float4*>(y + i0 + 4) = o1;
    } else {
        for (size_t i = i0; i < n; ++i)
            y[i] = gate_act<ACT>(to_f32(x[i]), add);
    }
}

template <typename IO, int ACT>
static hipError_t launch_act(const void* x, float* y, size_t n, float add, hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    const size_t threads = (n + 7) / 8;
    hipLaunchKernelGGL((kdn_gate_prologue_kernel<IO, ACT>), dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, stream, reinterpret_cast<const IO*>(x), y, n, add);
    return hipGetLastError();
}

hipError_t launch_gate_prologue(const PrologueArgs& a, int io_dtype, hipStream_t stream)
{
    const bool bf = io_dtype == 1;
    hipError_t e = bf ? launch_act<bf16, 0>(a.a_pre, a.alpha, a.n_alpha, 0.f, stream)
                      : launch_act<float, 0>(a.a_pre, a.alpha, a.n_alpha, 0.f, stream);
    if (e != hipSuccess)
        return e;
    e = bf ? launch_act<bf16, 1>(a.w_pre, a.omega, a.n_omega, 0.f, stream)
           : launch_act<float, 1>(a.w_pre, a.omega, a.n_omega, 0.f, stream);
    if (e != hipSuccess)
        return e;
    return bf ? launch_act<bf16, 1>(a.r_pre, a.r, a.n_r, a.r_min, stream)
              : launch_act<float, 1>(a.r_pre, a.r, a.n_r, a.r_min, stream);
}

}  // namespace kdn

namespace kdn {

// The gradients of the gates become the gradients of their pre-activations,
// in place: da *= alpha (1 - alpha), dw *= sigmoid(w), dr *= sigmoid(rho)
// (d softplus(x)/dx = sigmoid(x)).
template <typename IO, int ACT>
__global__ __launch_bounds__(256) void kdn_gate_epilogue_kernel(const float* __restrict__ gate,
                                                                const IO* __restrict__ pre,
                                                                float* __restrict__ g, size_t n)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    if constexpr (ACT == 0) {
        const float al = gate[i];
        g[i] *= al * (1.f - al);
    } else {
        g[i] *= gate_act<0>(to_f32(pre[i]), 0.f);
    }
}

template <typename IO, int ACT>
static hipError_t launch_epi(const float* gate, const void* pre, float* g, size_t n,
                             hipStream_t stream)
{
    if (n == 0 || !g)
        return hipSuccess;
    hipLaunchKernelGGL((kdn_gate_epilogue_kernel<IO, ACT>), dim3((unsigned)((n + 255) / 256)),
                       dim3(256), 0, stream, gate, reinterpret_cast<const IO*>(pre), g, n);
    return hipGetLastError();
}

hipError_t launch_gate_epilogue(const PrologueArgs& p, float* da, float* dw, float* dr,
                                int io_dtype, hipStream_t stream)
{
    const bool bf = io_dtype == 1;
    hipError_t e = bf ? launch_epi<bf16, 0>(p.alpha, nullptr, da, p.n_alpha, stream)
                      : launch_epi<float, 0>(p.alpha, nullptr, da, p.n_alpha, stream);
    if (e != hipSuccess)
        return e;
    e = bf ? launch_epi<bf16, 1>(nullptr, p.w_pre, dw, p.n_omega, stream)
           : launch_epi<float, 1>(nullptr, p.w_pre, dw, p.n_omega, stream);
    if (e != hipSuccess)
        return e;
    return bf ? launch_epi<bf16, 1>(nullptr, p.r_pre, dr, p.n_r, stream)
              : launch_epi<float, 1>(nullptr, p.r_pre, dr, p.n_r, stream);
}

}  // namespace kdn
