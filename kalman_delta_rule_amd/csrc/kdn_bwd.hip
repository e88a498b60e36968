// kdn_bwd.hip -- backward pass of Diagonal and Isotropic KDN, gfx950.
//
// The KDN reading notes train the mixer with the scanned recurrence (method
// part §8) but print no gradient formulas.  This is the reverse-mode
// derivative of the token recurrence of method part §2, §4-§5 (Diagonal) and
// §7 (Isotropic):
//   p^ = alpha^2 p + omega,  kap = p^ k / (r + z),  z = sum p^ k^2
//   (Isotropic: b^ = mean(alpha^2) b + omega, kap = b^ k / (r + b^ |k|^2)),
//   S^ = diag(alpha) S,  delta = v - S^^T k,  S = S^ + kap delta^T,  o = S^T q,
//   p = p^ / (1 + (mu/r) k^2 p^)   (Isotropic: b = b^/(1 + mu |k|^2 b^/(dk r))).
// Adjoints, with G = dL/dS_t carried backwards:
//   G += q do^T, dq = S do;  kapbar = G delta, delbar = G^T kap = dv;
//   S^bar = G - k delbar^T, dk -= S^ delbar, dalpha += rowsum(S^bar (.) S_{t-1}),
//   G <- diag(alpha) S^bar; then the variance recurrence's adjoint per channel.
//
// Three kernels, all fp32 arithmetic whatever the io type:
//   A  gain forward, one wave per (b,h): recomputes kap_t, p_{t-1} and
//      r + z_t (Isotropic: beta_t, b_{t-1}, mean alpha^2, |k|^2) for every token.
//   B  memory backward, one 256-thread workgroup per (b,h) and 16-column
//      block of the value dimension (the columns of S evolve independently
//      given the gain).  A forward pass stores S every 16 tokens; then for
//      each 16-token chunk, last first, the chunk's 17 states are recomputed
//      into registers and walked backwards.  dv is complete per column and
//      written here; the four row vectors that sum over all columns (dq, kapbar,
//      dk and dalpha of the memory) are written as per-block partials.
//   C  gain backward, one wave per (b,h): sums the partials and runs the
//      variance recurrence's adjoint backwards, writing dq, dk, dalpha,
//      domega, dr and the initial variance's and information scale's gradients.
// Each thread of B owns one row of S (one key channel) and 8 (d_k = 128) or 4
// (d_k = 64) columns, so row reductions stay in a lane pair or quad and the
// column reductions (delta, delbar) cross the workgroup through LDS once per
// token.
#include "kdn_common.h"
#include "kdn_internal.h"

namespace kdn {

constexpr int BWD_L = 16;    // tokens per recompute chunk (checkpoint spacing)
constexpr int BWD_COLS = 16; // value columns per memory workgroup

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        x += __shfl_xor(x, off);
    return x;
}

// ---------------------------------------------------------------------------
// A: gain forward
// ---------------------------------------------------------------------------
template <typename IO, bool ISO, int CPL>
__global__ __launch_bounds__(64) void kdn_bwd_gain_fwd_kernel(BwdArgs a)
{
    constexpr int DK = 64 * CPL;
    const int bh = blockIdx.x, H = a.H, T = a.T;
    const int b = bh / H, h = bh % H, lane = threadIdx.x;
    const float mu = a.mu_h ? a.mu_h[h] : a.mu;
    const IO* kg = reinterpret_cast<const IO*>(a.k);
    if constexpr (!ISO) {
        float p[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            p[c] = a.var0 ? a.var0[(size_t)bh * DK + lane + 64 * c] : (a.c0 ? a.c0[h] : 1.f);
        for (int t = 0; t < T; ++t) {
            const size_t tok = ((size_t)b * T + t) * H + h;
            const float rt = a.r[tok];
            float ph[CPL], kk[CPL], zp = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const size_t e = tok * DK + lane + 64 * c;
                const float al = a.alpha[e];
                kk[c] = to_f32(kg[e]);
                ph[c] = al * al * p[c] + a.omega[e];
                zp += ph[c] * kk[c] * kk[c];
            }
            const float d = rt + wave_sum(zp);
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const size_t e = tok * DK + lane + 64 * c;
                a.kap[e] = ph[c] * kk[c] / d;
                a.pprev[e] = p[c];
                p[c] = ph[c] / (1.f + (mu / rt) * kk[c] * kk[c] * ph[c]);
            }
            if (lane == 0)
                a.dd[tok] = d;
        }
    } else {
        float bv = a.var0 ? a.var0[bh] : (a.c0 ? a.c0[h] : 1.f);
        for (int t = 0; t < T; ++t) {
            const size_t tok = ((size_t)b * T + t) * H + h;
            const float rt = a.r[tok];
            float sa = 0.f, sn = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const size_t e = tok * DK + lane + 64 * c;
                const float al = a.alpha[e], kk = to_f32(kg[e]);
                sa += al * al;
                sn += kk * kk;
            }
            const float am = wave_sum(sa) / (float)DK, n = wave_sum(sn);
            const float bhat = am * bv + a.omega[tok];
            const float beta = bhat / (rt + bhat * n);
            if (lane == 0) {
                float4 g = {beta, bv, am, n};
                *reinterpret_cast<float4*>(a.gsc + tok * 4) = g;
            }
            bv = bhat / (1.f + mu * n / ((float)DK * rt) * bhat);
        }
    }
}

// ---------------------------------------------------------------------------
// B: memory backward
// ---------------------------------------------------------------------------
template <typename IO, bool ISO, int DK>
__global__ __launch_bounds__(256) void kdn_bwd_mem_kernel(BwdArgs a)
{
    constexpr int TPR = 256 / DK;        // threads per row of S
    constexpr int CPT = BWD_COLS / TPR;  // columns per thread
    constexpr int L = BWD_L;
    __shared__ float red[2][4][BWD_COLS];
    __shared__ float dbuf[L][BWD_COLS];

    const int blk = blockIdx.x, nblk = gridDim.x, bh = blockIdx.y;
    const int H = a.H, T = a.T, dv = a.dv;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = tid / TPR, cp = tid % TPR;
    const int cb = cp * CPT;                // first column of this thread in the block
    const int col0 = blk * BWD_COLS + cb;   // ... in the value dimension
    const int nch = (T + L - 1) / L;
    const size_t ntok = (size_t)a.B * T * H;
    const IO* qg = reinterpret_cast<const IO*>(a.q);
    const IO* kg = reinterpret_cast<const IO*>(a.k);
    const IO* vg = reinterpret_cast<const IO*>(a.v);
    const IO* dog = reinterpret_cast<const IO*>(a.go);
    IO* dvg = reinterpret_cast<IO*>(a.gv);
    float* ck = a.ckpt + ((size_t)bh * nblk + blk) * nch * (DK * BWD_COLS) + row * BWD_COLS + cb;

    int slot = 0;
    // sum over all rows of the block, per column; every thread gets the sums
    // of its CPT columns.  One barrier; the two LDS slots alternate so the
    // next call's writes never meet this call's reads.
    auto col_sum = [&](float (&x)[CPT]) {
#pragma unroll
        for (int off = TPR; off < 64; off <<= 1)
#pragma unroll
            for (int j = 0; j < CPT; ++j)
                x[j] += __shfl_xor(x[j], off);
        if (lane < TPR)
#pragma unroll
            for (int j = 0; j < CPT; ++j)
                red[slot][wave][cb + j] = x[j];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < CPT; ++j)
            x[j] = red[slot][0][cb + j] + red[slot][1][cb + j] + red[slot][2][cb + j] +
                   red[slot][3][cb + j];
        slot ^= 1;
    };
    auto row_sum = [&](float x) {
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1)
            x += __shfl_xor(x, off);
        return x;
    };
    auto gain = [&](size_t tok, float kk) {
        if constexpr (ISO)
            return a.gsc[tok * 4] * kk;
        else
            return a.kap[tok * DK + row];
    };

    // forward pass: the state at every chunk start
    float s[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
        s[j] = a.S0 ? a.S0[((size_t)bh * DK + row) * dv + col0 + j] : 0.f;
    for (int t = 0; t < T; ++t) {
        if ((t & (L - 1)) == 0)
#pragma unroll
            for (int j = 0; j < CPT; ++j)
                ck[(size_t)(t / L) * (DK * BWD_COLS) + j] = s[j];
        const size_t tok = ((size_t)b * T + t) * H + h;
        const float al = a.alpha[tok * DK + row], kk = to_f32(kg[tok * DK + row]);
        const float kap = gain(tok, kk);
        float x[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            s[j] *= al;
            x[j] = s[j] * kk;
        }
        col_sum(x);
#pragma unroll
        for (int j = 0; j < CPT; ++j)
            s[j] += kap * (to_f32(vg[tok * dv + col0 + j]) - x[j]);
    }
    __threadfence_block();  // this thread's checkpoint stores before its loads below

    // reverse pass
    float g[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
        g[j] = a.gS_T ? a.gS_T[((size_t)bh * DK + row) * dv + col0 + j] : 0.f;
    for (int c = nch - 1; c >= 0; --c) {
        const int t0 = c * L, len = min(L, T - t0);
        float st[L + 1][CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j)
            st[0][j] = ck[(size_t)c * (DK * BWD_COLS) + j];
        // recompute the chunk's states and innovations
#pragma unroll
        for (int tau = 0; tau < L; ++tau) {
            if (tau < len) {
                const size_t tok = ((size_t)b * T + t0 + tau) * H + h;
                const float al = a.alpha[tok * DK + row], kk = to_f32(kg[tok * DK + row]);
                const float kap = gain(tok, kk);
                float x[CPT];
#pragma unroll
                for (int j = 0; j < CPT; ++j)
                    x[j] = al * st[tau][j] * kk;
                col_sum(x);
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    const float del = to_f32(vg[tok * dv + col0 + j]) - x[j];
                    dbuf[tau][cb + j] = del;  // every row stores the same value
                    st[tau + 1][j] = al * st[tau][j] + kap * del;
                }
            }
        }
        // walk the chunk backwards
#pragma unroll
        for (int tau = L - 1; tau >= 0; --tau) {
            if (tau < len) {
                const size_t tok = ((size_t)b * T + t0 + tau) * H + h;
                const size_t e = tok * DK + row;
                const float al = a.alpha[e], kk = to_f32(kg[e]), qq = to_f32(qg[e]);
                const float kap = gain(tok, kk);
                float dov[CPT], y[CPT];
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    dov[j] = to_f32(dog[tok * dv + col0 + j]);
                    g[j] = fmaf(qq, dov[j], g[j]);               // readout o = S^T q
                    sq = fmaf(st[tau + 1][j], dov[j], sq);      // dq = S do
                    sk = fmaf(g[j], dbuf[tau][cb + j], sk);     // kapbar = G delta
                    y[j] = g[j] * kap;
                }
                col_sum(y);                                     // delbar = G^T kap
                if (row == 0)
#pragma unroll
                    for (int j = 0; j < CPT; ++j)
                        dvg[tok * dv + col0 + j] = from_f32<IO>(y[j]);
                float skm = 0.f, sam = 0.f;
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    const float shb = fmaf(-kk, y[j], g[j]);    // S^bar = G - k delbar^T
                    skm = fmaf(st[tau][j], y[j], skm);
                    sam = fmaf(shb, st[tau][j], sam);
                    g[j] = al * shb;                            // adjoint of S_{t-1}
                }
                sq = row_sum(sq);
                sk = row_sum(sk);
                skm = row_sum(skm);
                sam = row_sum(sam);
                if (cp == 0) {
                    float* pp = a.part + ((size_t)blk * ntok + tok) * DK + row;
                    const size_t kstride = (size_t)nblk * ntok * DK;
                    pp[0] = sq;
                    pp[kstride] = sk;
                    pp[2 * kstride] = -al * skm;
                    pp[3 * kstride] = sam;
                }
            }
        }
    }
    if (a.gS0)
#pragma unroll
        for (int j = 0; j < CPT; ++j)
            a.gS0[((size_t)bh * DK + row) * dv + col0 + j] = g[j];
}

// ---------------------------------------------------------------------------
// C: gain backward
// ---------------------------------------------------------------------------
template <typename IO, bool ISO, int CPL>
__global__ __launch_bounds__(64) void kdn_bwd_gain_rev_kernel(BwdArgs a, int nblk)
{
    constexpr int DK = 64 * CPL;
    const int bh = blockIdx.x, H = a.H, T = a.T;
    const int b = bh / H, h = bh % H, lane = threadIdx.x;
    const float mu = a.mu_h ? a.mu_h[h] : a.mu;
    const size_t ntok = (size_t)a.B * T * H, kstride = (size_t)nblk * ntok * DK;
    const IO* kg = reinterpret_cast<const IO*>(a.k);
    IO* dqg = reinterpret_cast<IO*>(a.gq);
    IO* dkg = reinterpret_cast<IO*>(a.gk);

    float pbar[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        pbar[c] = 0.f;
    float bbar = 0.f, mub = 0.f;
    if constexpr (!ISO) {
        if (a.gvar_T)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                pbar[c] = a.gvar_T[(size_t)bh * DK + lane + 64 * c];
    } else {
        bbar = a.gvar_T ? a.gvar_T[bh] : 0.f;
    }

    for (int t = T - 1; t >= 0; --t) {
        const size_t tok = ((size_t)b * T + t) * H + h;
        const float rt = a.r[tok];
        float kb[CPL], kmb[CPL], amb[CPL], kk[CPL], al[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const size_t e = tok * DK + lane + 64 * c;
            float qs = 0.f, ks = 0.f, km = 0.f, am = 0.f;
            for (int bl = 0; bl < nblk; ++bl) {
                const float* pp = a.part + ((size_t)bl * ntok + tok) * DK + lane + 64 * c;
                qs += pp[0];
                ks += pp[kstride];
                km += pp[2 * kstride];
                am += pp[3 * kstride];
            }
            dqg[e] = from_f32<IO>(qs);
            kb[c] = ks;
            kmb[c] = km;
            amb[c] = am;
            kk[c] = to_f32(kg[e]);
            al[c] = a.alpha[e];
        }
        if constexpr (!ISO) {
            const float d = a.dd[tok];
            float ph[CPL], pp[CPL], kap[CPL], u[CPL], phb[CPL], ub[CPL];
            float s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const size_t e = tok * DK + lane + 64 * c;
                pp[c] = a.pprev[e];
                ph[c] = al[c] * al[c] * pp[c] + a.omega[e];
                kap[c] = ph[c] * kk[c] / d;
                u[c] = (mu / rt) * kk[c] * kk[c];
                const float den = 1.f + u[c] * ph[c];
                phb[c] = pbar[c] / (den * den);
                ub[c] = -pbar[c] * ph[c] * ph[c] / (den * den);
                s1 += kb[c] * kap[c];
                s2 += ub[c] * u[c];
                s3 += ub[c] * kk[c] * kk[c];
            }
            const float dbar = -wave_sum(s1) / d;
            const float rbar = dbar - wave_sum(s2) / rt;
            mub += s3 / rt;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const size_t e = tok * DK + lane + 64 * c;
                phb[c] += kb[c] * kk[c] / d + dbar * kk[c] * kk[c];
                const float kbar = kmb[c] + 2.f * ub[c] * (mu / rt) * kk[c] +
                                   kb[c] * ph[c] / d + 2.f * dbar * ph[c] * kk[c];
                dkg[e] = from_f32<IO>(kbar);
                a.galpha[e] = amb[c] + 2.f * phb[c] * al[c] * pp[c];
                a.gomega[e] = phb[c];
                pbar[c] = phb[c] * al[c] * al[c];
            }
            if (lane == 0)
                a.gr[tok] = rbar;
        } else {
            const float4 gs = *reinterpret_cast<const float4*>(a.gsc + tok * 4);
            const float beta = gs.x, bprev = gs.y, am = gs.z, n = gs.w;
            const float bhat = am * bprev + a.omega[tok];
            const float e = rt + bhat * n;
            const float u = mu * n / ((float)DK * rt);
            const float den = 1.f + u * bhat;
            float bhb = bbar / (den * den);
            const float ub = -bbar * bhat * bhat / (den * den);
            float nb = ub * mu / ((float)DK * rt);
            float rbar = -ub * u / rt;
            mub += ub * n / ((float)DK * rt);
            float sb = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                sb += kb[c] * kk[c];
            const float betab = wave_sum(sb);
            bhb += betab * rt / (e * e);
            rbar -= betab * bhat / (e * e);
            nb -= betab * bhat * bhat / (e * e);
            const float abar = bhb * bprev;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const size_t ei = tok * DK + lane + 64 * c;
                dkg[ei] = from_f32<IO>(kmb[c] + beta * kb[c] + 2.f * nb * kk[c]);
                a.galpha[ei] = amb[c] + 2.f * abar * al[c] / (float)DK;
            }
            if (lane == 0) {
                a.gomega[tok] = bhb;
                a.gr[tok] = rbar;
            }
            bbar = bhb * am;
        }
    }
    if constexpr (!ISO) {
        if (a.gvar0)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                a.gvar0[(size_t)bh * DK + lane + 64 * c] = pbar[c];
        mub = wave_sum(mub);
    } else {
        if (a.gvar0 && lane == 0)
            a.gvar0[bh] = bbar;
    }
    if (a.gmu && lane == 0)
        a.gmu[bh] = mub;
}

// ---------------------------------------------------------------------------
// workspace and launch
// ---------------------------------------------------------------------------
static size_t round64(size_t n) { return (n + 63) & ~(size_t)63; }

size_t bwd_workspace_floats(bool iso, int B, int T, int H, int dk, int dv)
{
    const size_t ntok = (size_t)B * T * H, bh = (size_t)B * H;
    const size_t nch = ((size_t)T + BWD_L - 1) / BWD_L, nblk = (size_t)dv / BWD_COLS;
    size_t n = 0;
    if (iso)
        n += round64(ntok * 4);
    else
        n += 2 * round64(ntok * dk) + round64(ntok);
    n += round64(bh * nch * dk * dv);        // checkpoints
    n += round64(4 * nblk * ntok * dk);      // partials
    return n;
}

void bwd_carve_workspace(BwdArgs& a, bool iso, float* ws)
{
    const size_t ntok = (size_t)a.B * a.T * a.H, bh = (size_t)a.B * a.H;
    const size_t nch = ((size_t)a.T + BWD_L - 1) / BWD_L, nblk = (size_t)a.dv / BWD_COLS;
    float* p = ws;
    a.kap = a.pprev = a.dd = a.gsc = nullptr;
    if (iso) {
        a.gsc = p;
        p += round64(ntok * 4);
    } else {
        a.kap = p;
        p += round64(ntok * a.dk);
        a.pprev = p;
        p += round64(ntok * a.dk);
        a.dd = p;
        p += round64(ntok);
    }
    a.ckpt = p;
    p += round64(bh * nch * a.dk * a.dv);
    a.part = p;
}

template <typename IO, bool ISO, int DK>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream)
{
    constexpr int CPL = DK / 64;
    const int bh = a.B * a.H, nblk = a.dv / BWD_COLS;
    if (a.T > 0) {
        hipLaunchKernelGGL((kdn_bwd_gain_fwd_kernel<IO, ISO, CPL>), dim3(bh), dim3(64), 0, stream,
                           a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((kdn_bwd_mem_kernel<IO, ISO, DK>), dim3(nblk, bh), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((kdn_bwd_gain_rev_kernel<IO, ISO, CPL>), dim3(bh), dim3(64), 0, stream, a,
                       nblk);
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, bool iso, int io_dtype, hipStream_t stream)
{
    const bool bf = io_dtype == 1;
    if (a.dk == 128) {
        if (iso)
            return bf ? launch_bwd_t<bf16, true, 128>(a, stream) : launch_bwd_t<float, true, 128>(a, stream);
        return bf ? launch_bwd_t<bf16, false, 128>(a, stream) : launch_bwd_t<float, false, 128>(a, stream);
    }
    if (iso)
        return bf ? launch_bwd_t<bf16, true, 64>(a, stream) : launch_bwd_t<float, true, 64>(a, stream);
    return bf ? launch_bwd_t<bf16, false, 64>(a, stream) : launch_bwd_t<float, false, 64>(a, stream);
}

}  // namespace kdn
