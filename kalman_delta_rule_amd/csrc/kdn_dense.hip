// kdn_dense.hip -- exact dense-covariance Kalman memory for small d_k, gfx950.
//
// The exact filter of the KDN reading notes, method part §2 (Eq. (12)-(17)),
// with the Diagonal KDN's own gates as its transition and process noise,
// D_t = diag(alpha_t) and Omega_t = diag(omega_t), so that Diagonal KDN is
// this filter's mean-field projection (method part §4):
//   S^ = D S,   P^ = D P D + Omega,   delta = v - S^^T k,
//   z = k^T P^ k,   kappa = P^ k / (r + z),
//   S = S^ + kappa delta^T,   P = (I - kappa k^T) P^ = P^ - kappa u^T (u = P^ k),
//   o = S^T q (read after the write),   beta_eff = z / (r + z).
// The covariance is d_k x d_k per head and its update is a serial Riccati
// step, so this is an ablation and cross-check tool for small d_k, not a
// throughput path.  One 256-thread workgroup per (batch, head) keeps P and S
// in LDS for the whole sequence; every token is five barrier-separated
// phases (inputs, prediction, u and delta, update, readout).
#include "kdn_common.h"
#include "kdn_internal.h"
#include "kdn_ops.h"

namespace kdn {

constexpr int DENSE_THREADS = 256;

template <typename IO, int DK, int DV>
__global__ __launch_bounds__(DENSE_THREADS) void kdn_dense_kernel(DenseArgs a)
{
    constexpr int TPR = DENSE_THREADS / DK;  // threads per row of P (u = P^ k)
    constexpr int TPC = DENSE_THREADS / DV;  // threads per column of S (delta, o)
    static_assert(TPR >= 1 && TPR <= 64 && DK % TPR == 0, "row split");
    static_assert(TPC >= 1 && TPC <= 64 && DK % TPC == 0, "column split");

    __shared__ float sP[DK][DK + 1];
    __shared__ float sS[DK][DV + 1];
    __shared__ float sk[DK], sq[DK], sa[DK], sw[DK], su[DK];
    __shared__ float sv[DV], sd[DV];

    const int bh = blockIdx.x;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x;
    const int T = a.T, H = a.H;

    // initial state: S0 (or zeros) and P0 (or the identity)
    for (int idx = tid; idx < DK * DV; idx += DENSE_THREADS) {
        const int i = idx / DV, j = idx % DV;
        sS[i][j] = a.S0 ? a.S0[(size_t)bh * DK * DV + idx] : 0.f;
    }
    for (int idx = tid; idx < DK * DK; idx += DENSE_THREADS) {
        const int i = idx / DK, j = idx % DK;
        sP[i][j] = a.P0 ? a.P0[(size_t)bh * DK * DK + idx] : (i == j ? 1.f : 0.f);
    }

    const IO* qg = reinterpret_cast<const IO*>(a.q);
    const IO* kg = reinterpret_cast<const IO*>(a.k);
    const IO* vg = reinterpret_cast<const IO*>(a.v);
    IO* og = reinterpret_cast<IO*>(a.o);
    const int row = tid / TPR, rpart = tid % TPR;  // u = P^ k: row, slice
    const int col = tid / TPC, cpart = tid % TPC;  // delta / o: column, slice

    for (int t = 0; t < T; ++t) {
        const size_t tok = ((size_t)b * T + t) * H + h;
        // (1) this token's inputs
        if (tid < DK) {
            sk[tid] = to_f32(kg[tok * DK + tid]);
            sq[tid] = to_f32(qg[tok * DK + tid]);
            sa[tid] = a.alpha[tok * DK + tid];
            sw[tid] = a.omega[tok * DK + tid];
        }
        if (tid < DV)
            sv[tid] = to_f32(vg[tok * DV + tid]);
        const float rt = a.r[tok];
        __syncthreads();

        // (2) prediction: P^ = D P D + Omega,  S^ = D S
        for (int idx = tid; idx < DK * DK; idx += DENSE_THREADS) {
            const int i = idx / DK, j = idx % DK;
            sP[i][j] = sa[i] * sa[j] * sP[i][j] + (i == j ? sw[i] : 0.f);
        }
        for (int idx = tid; idx < DK * DV; idx += DENSE_THREADS) {
            const int i = idx / DV, j = idx % DV;
            sS[i][j] *= sa[i];
        }
        __syncthreads();

        // (3) u = P^ k and delta = v - S^^T k, partial sums then a lane reduction
        {
            float x = 0.f;
#pragma unroll
            for (int jj = 0; jj < DK / TPR; ++jj) {
                const int j = rpart * (DK / TPR) + jj;
                x = fmaf(sP[row][j], sk[j], x);
            }
#pragma unroll
            for (int off = TPR / 2; off >= 1; off >>= 1)
                x += __shfl_xor(x, off);
            if (rpart == 0)
                su[row] = x;
            float y = 0.f;
#pragma unroll
            for (int ii = 0; ii < DK / TPC; ++ii) {
                const int i = cpart * (DK / TPC) + ii;
                y = fmaf(sS[i][col], sk[i], y);
            }
#pragma unroll
            for (int off = TPC / 2; off >= 1; off >>= 1)
                y += __shfl_xor(y, off);
            if (cpart == 0)
                sd[col] = sv[col] - y;
        }
        __syncthreads();

        // (4) z = k^T u (every thread), then the rank-one updates
        float z = 0.f;
#pragma unroll 8
        for (int i = 0; i < DK; ++i)
            z = fmaf(sk[i], su[i], z);
        const float dinv = 1.f / (rt + z);
        if (a.beta && tid == 0)
            a.beta[tok] = z * dinv;
        for (int idx = tid; idx < DK * DV; idx += DENSE_THREADS) {
            const int i = idx / DV, j = idx % DV;
            sS[i][j] = fmaf(su[i] * dinv, sd[j], sS[i][j]);
        }
        for (int idx = tid; idx < DK * DK; idx += DENSE_THREADS) {
            const int i = idx / DK, j = idx % DK;
            sP[i][j] = fmaf(-su[i] * dinv, su[j], sP[i][j]);
        }
        __syncthreads();

        // (5) readout after the write: o = S^T q
        {
            float y = 0.f;
#pragma unroll
            for (int ii = 0; ii < DK / TPC; ++ii) {
                const int i = cpart * (DK / TPC) + ii;
                y = fmaf(sS[i][col], sq[i], y);
            }
#pragma unroll
            for (int off = TPC / 2; off >= 1; off >>= 1)
                y += __shfl_xor(y, off);
            if (cpart == 0)
                og[tok * DV + col] = from_f32<IO>(y);
        }
        __syncthreads();
    }

    for (int idx = tid; idx < DK * DV; idx += DENSE_THREADS) {
        const int i = idx / DV, j = idx % DV;
        a.S_T[(size_t)bh * DK * DV + idx] = sS[i][j];
    }
    for (int idx = tid; idx < DK * DK; idx += DENSE_THREADS) {
        const int i = idx / DK, j = idx % DK;
        a.P_T[(size_t)bh * DK * DK + idx] = sP[i][j];
    }
}

template <typename IO, int DK, int DV>
static hipError_t launch_dense_one(const DenseArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL((kdn_dense_kernel<IO, DK, DV>), dim3(a.B * a.H), dim3(DENSE_THREADS), 0,
                       stream, a);
    return hipGetLastError();
}

template <typename IO, int DK>
static hipError_t dense_dv(const DenseArgs& a, hipStream_t stream)
{
    switch (a.dv) {
    case 16: return launch_dense_one<IO, DK, 16>(a, stream);
    case 32: return launch_dense_one<IO, DK, 32>(a, stream);
    case 64: return launch_dense_one<IO, DK, 64>(a, stream);
    case 128: return launch_dense_one<IO, DK, 128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename IO>
static hipError_t dense_dk(const DenseArgs& a, hipStream_t stream)
{
    switch (a.dk) {
    case 16: return dense_dv<IO, 16>(a, stream);
    case 32: return dense_dv<IO, 32>(a, stream);
    case 64: return dense_dv<IO, 64>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dense_fwd(const DenseArgs& a, int io_dtype, hipStream_t stream)
{
    return io_dtype == 1 ? dense_dk<bf16>(a, stream) : dense_dk<float>(a, stream);
}

}  // namespace kdn
