// kdn_step.hip -- single-token KDN decode step, gfx950.
//
// One workgroup per (batch, head).  The fp32 state S (dk x dv) is read once
// into registers (float4 per lane along the value dimension, so every load
// and store is a coalesced 16-byte access), updated, and written once:
//   gain   (KDN reading notes, method part §4-§5 / §7):
//          p^ = alpha^2 p + omega, z = sum p^ k^2, kappa = p^ k / (r + z),
//          p <- p^ / (1 + (mu/r) k^2 p^)      [Isotropic: scalar b]
//   memory (§2 Eq. (12)-(17) specialised to D = diag(alpha)):
//          delta_j = v_j - sum_i alpha_i S_ij k_i
//          S_ij   <- alpha_i S_ij + kappa_i delta_j
//          o_j     = sum_i S_ij q_i            (after the write)
// The two reductions over i run as partial sums per row group followed by a
// small LDS reduction.  The step is HBM-bound (about 1 flop per byte).
#include "kdn_common.h"
#include "kdn_internal.h"

namespace kdn {

constexpr int STEP_THREADS = 256;

template <typename IO, int DK, int DV, bool ISO>
__global__ __launch_bounds__(STEP_THREADS) void kdn_step_kernel(StepArgs a)
{
    constexpr int LPR = DV / 4;                 // lanes per state row
    constexpr int RG = STEP_THREADS / LPR;      // row groups
    constexpr int RPT = DK / RG;                // rows per thread
    static_assert(RPT >= 1 && DK % RG == 0, "shape");
    static_assert(DK <= STEP_THREADS, "one gain lane per channel");

    __shared__ float s_alpha[DK], s_kap[DK], s_ak[DK], s_q[DK];
    __shared__ __align__(16) float s_red[RG][DV];
    __shared__ __align__(16) float s_delta[DV];
    __shared__ float s_wsum[2][STEP_THREADS / 64];

    const int bh = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rg = tid / LPR, cl = tid % LPR;
    const IO* qg = reinterpret_cast<const IO*>(a.q) + (size_t)bh * DK;
    const IO* kg = reinterpret_cast<const IO*>(a.k) + (size_t)bh * DK;
    const IO* vg = reinterpret_cast<const IO*>(a.v) + (size_t)bh * DV;
    IO* og = reinterpret_cast<IO*>(a.o) + (size_t)bh * DV;
    float* S = a.S + (size_t)bh * DK * DV;

    // issue the state loads first: RPT float4 per lane
    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = *reinterpret_cast<const f32x4*>(S + (size_t)(rg + RG * m) * DV + 4 * cl);

    const float rt = a.r[bh];
    const float mu = a.mu_h ? a.mu_h[bh % a.H] : a.mu;
    // read the head's scalar variance before any lane overwrites it
    const float bvar = ISO ? a.var[bh] : 0.f;
    // ---- gain (lanes = key channels)
    float al = 0.f, kv = 0.f, ph = 0.f, x0 = 0.f, x1 = 0.f;
    if (tid < DK) {
        al = a.alpha[(size_t)bh * DK + tid];
        kv = to_f32(kg[tid]);
        s_q[tid] = to_f32(qg[tid]);
        if (!ISO) {
            ph = al * al * a.var[(size_t)bh * DK + tid] + a.omega[(size_t)bh * DK + tid];
            x0 = ph * kv * kv;  // z partial
        } else {
            x0 = al * al;       // sum alpha^2
            x1 = kv * kv;       // |k|^2
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        x0 += __shfl_xor(x0, m);
        x1 += __shfl_xor(x1, m);
    }
    if (lane == 0) {
        s_wsum[0][wave] = x0;
        s_wsum[1][wave] = x1;
    }
    __syncthreads();
    float sum0 = 0.f, sum1 = 0.f;
#pragma unroll
    for (int w = 0; w < STEP_THREADS / 64; ++w) {
        sum0 += s_wsum[0][w];
        sum1 += s_wsum[1][w];
    }
    if (tid < DK) {
        float kap;
        if (!ISO) {
            const float z = sum0;
            const float dz = rcp(rt + z);
            kap = ph * kv * dz;
            if (a.beta && tid == 0)
                a.beta[bh] = z * dz;
            const float u = (mu / rt) * kv * kv;
            a.var[(size_t)bh * DK + tid] = ph * rcp(1.f + u * ph);
        } else {
            const float am = sum0 * (1.f / DK), n = sum1;
            const float bh_ = am * bvar + a.omega[bh];
            const float beta = bh_ * rcp(rt + bh_ * n);
            kap = beta * kv;
            if (tid == 0) {
                if (a.beta)
                    a.beta[bh] = beta * n;  // z / (r + z) with z = b^ |k|^2
                const float u = mu * n * rcp((float)DK * rt);
                a.var[bh] = bh_ * rcp(1.f + u * bh_);
            }
        }
        s_alpha[tid] = al;
        s_kap[tid] = kap;
        s_ak[tid] = al * kv;
    }
    __syncthreads();

    // ---- innovation delta_j = v_j - sum_i alpha_i k_i S_ij
    f32x4 part = zero4();
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        part += s_ak[rg + RG * m] * s[m];
    *reinterpret_cast<f32x4*>(&s_red[rg][4 * cl]) = part;
    __syncthreads();
    if (tid < DV) {
        float acc = 0.f;
#pragma unroll
        for (int g = 0; g < RG; ++g)
            acc += s_red[g][tid];
        s_delta[tid] = to_f32(vg[tid]) - acc;
    }
    __syncthreads();

    // ---- write and read-after-write
    const f32x4 dl = *reinterpret_cast<const f32x4*>(&s_delta[4 * cl]);
    part = zero4();
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + RG * m;
        s[m] = s_alpha[i] * s[m] + s_kap[i] * dl;
        part += s_q[i] * s[m];
        *reinterpret_cast<f32x4*>(S + (size_t)i * DV + 4 * cl) = s[m];
    }
    *reinterpret_cast<f32x4*>(&s_red[rg][4 * cl]) = part;
    __syncthreads();
    if (tid < DV) {
        float acc = 0.f;
#pragma unroll
        for (int g = 0; g < RG; ++g)
            acc += s_red[g][tid];
        og[tid] = from_f32<IO>(acc);
    }
}

template <typename IO, int DK, int DV, bool ISO>
static hipError_t launch_step_one(const StepArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL((kdn_step_kernel<IO, DK, DV, ISO>), dim3(a.B * a.H), dim3(STEP_THREADS), 0,
                       stream, a);
    return hipGetLastError();
}

template <typename IO, bool ISO>
static hipError_t dispatch_dims(const StepArgs& a, hipStream_t stream)
{
    if (a.dk == 128 && a.dv == 128)
        return launch_step_one<IO, 128, 128, ISO>(a, stream);
    if (a.dk == 128 && a.dv == 64)
        return launch_step_one<IO, 128, 64, ISO>(a, stream);
    if (a.dk == 64 && a.dv == 128)
        return launch_step_one<IO, 64, 128, ISO>(a, stream);
    if (a.dk == 64 && a.dv == 64)
        return launch_step_one<IO, 64, 64, ISO>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_step(const StepArgs& a, bool iso, int io_dtype, hipStream_t stream)
{
    if (io_dtype == 1)
        return iso ? dispatch_dims<bf16, true>(a, stream) : dispatch_dims<bf16, false>(a, stream);
    return iso ? dispatch_dims<float, true>(a, stream) : dispatch_dims<float, false>(a, stream);
}

}  // namespace kdn
