// kdn_seqpar.hip -- the bf16 forward split over the sequence for grids that
// leave most compute units idle (few heads, long sequences), gfx950.
//
// The state recurrence is affine in the state: over a span of tokens,
// S_out = M S_in + N, where M (d_k x d_k) depends on the keys and gains only
// and N is the output from a zero state (KDN reading notes, method part §2
// and §6: the chunked form composes exactly these maps).  The variance
// recurrence does not depend on the state, so its value at every span start
// comes from the Moebius gain scan (method part §6).  With T split into S
// segments, a [B, T, H] tensor read as [B*S, T/S, H] makes the segments
// independent problems for the walk kernel:
//   1. gain scan: the variance entering every 64-token chunk;
//   2. state-only walk from a zero state: N of every segment (no q read, no
//      o written);
//   3. state-only walk with v = 0 (not read) from S_in = I: M of every segment
//      (d_k = d_v).  (A walk from I on the real v gives M + N, but recovering
//      M by subtracting N loses M's precision where N dominates, as without
//      decay.)
//   4. combine per head: S_in(s+1) = M(s) S_in(s) + N(s), from the caller's S0;
//   5. full walk from S_in(s): the outputs o (and beta_eff).
// Three walks over S times as many workgroups, two of them reading only the
// keys and gates (and v for N).  The final state is the combine's last S_out,
// the final variance the gain scan's.  All three walks start each segment
// from the same variance, so they apply the same gains.
//
// The backward's memory part splits the same way.  Its reverse pass carries
// the state adjoint dS back through the tokens, and that map is affine too:
// the adjoint entering a segment from its right, X(s+1), reaches the
// segment's start as M(s)^T X(s+1) (the transpose of the forward map above),
// and the segment's own outputs add B(s), the adjoint at its start from a
// zero X(s+1).  So after the gain scan:
//   1-3. the state walks and the combine above give every segment's entry state;
//   4. the chunked backward in its adjoint-only mode, from a zero incoming
//      adjoint, gives B(s) (no forward pass, no per-token output);
//   5. a combine from the last segment, X(S) = dS_T, X(s) = M(s)^T X(s+1) + B(s),
//      gives each segment's incoming adjoint X(s+1) and dS0 = X(0);
//   6. the chunked backward over the segments as batch rows, from their
//      entry states and incoming adjoints, writes every per-token gradient.
#include "kdn_common.h"
#include "kdn_internal.h"
#include "kdn_ops.h"

namespace kdn {

static size_t r64(size_t n) { return (n + 63) & ~(size_t)63; }

__global__ __launch_bounds__(256) void sp_identity_kernel(float* I, size_t n, int D)
{
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx < n) {
        const int i = (int)((idx / D) % D), j = (int)(idx % D);
        I[idx] = i == j ? 1.f : 0.f;
    }
}

// p_in[(b S + s) H + h][i] = variance entering token s T / S of (b, h)
__global__ __launch_bounds__(256) void sp_gather_var_kernel(const float* carry, float* pin, int B,
                                                            int H, int S, int width, int nchunks,
                                                            int seg_chunks)
{
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)B * S * H * width)
        return;
    const int i = (int)(idx % width);
    const size_t m = idx / width;
    const int h = (int)(m % H);
    const int bsi = (int)(m / H), b = bsi / S, s = bsi % S;
    pin[idx] = carry[(((size_t)b * H + h) * nchunks + (size_t)s * seg_chunks) * width + i];
}

// S_in(0) = S0 (or 0), S_in(s+1) = M(s) S_in(s) + N(s), S_T = S_in(S).  The
// columns of the state are independent, so one workgroup owns a 16-column
// block of one (b, h).  Its state block and the segment's whole M sit in LDS;
// thread t owns column t % 16 of D / 16 consecutive rows, and the M rows are
// read four entries at a time (16 lanes share an address: a broadcast).
template <int D>
__global__ __launch_bounds__(256) void sp_combine_kernel(const float* S0, const float* Mg,
                                                         const float* Ng, float* Sin, float* S_T,
                                                         int H, int S)
{
    constexpr int CB = 16, R = D / 16, NBLK = D / CB;
    __shared__ __align__(16) float sS[D][CB];
    __shared__ __align__(16) float sM[D][D];
    const int bh = blockIdx.x / NBLK, c0 = (blockIdx.x % NBLK) * CB;
    const int b = bh / H, h = bh % H, t = threadIdx.x;
    const int j = t % CB, r0 = (t / CB) * R;
    const size_t DD = (size_t)D * D;
    for (int e = t; e < D * CB; e += 256)
        sS[e / CB][e % CB] = S0 ? S0[(size_t)bh * DD + (size_t)(e / CB) * D + c0 + e % CB] : 0.f;
    for (int s = 0; s < S; ++s) {
        const size_t seg = ((size_t)(b * S + s) * H + h) * DD;
        __syncthreads();
        for (int e = t; e < D * CB; e += 256)
            Sin[seg + (size_t)(e / CB) * D + c0 + e % CB] = sS[e / CB][e % CB];
        for (int e = 4 * t; e < D * D; e += 1024)
            *reinterpret_cast<float4*>(&sM[e / D][e % D]) =
                *reinterpret_cast<const float4*>(Mg + seg + e);
        __syncthreads();
        float acc[R];
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
            acc[rr] = Ng[seg + (size_t)(r0 + rr) * D + c0 + j];
        for (int k = 0; k < D; k += 4) {
            const float s0 = sS[k][j], s1 = sS[k + 1][j], s2 = sS[k + 2][j], s3 = sS[k + 3][j];
#pragma unroll
            for (int rr = 0; rr < R; ++rr) {
                const float4 m = *reinterpret_cast<const float4*>(&sM[r0 + rr][k]);
                acc[rr] = fmaf(m.x, s0, acc[rr]);
                acc[rr] = fmaf(m.y, s1, acc[rr]);
                acc[rr] = fmaf(m.z, s2, acc[rr]);
                acc[rr] = fmaf(m.w, s3, acc[rr]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
            sS[r0 + rr][j] = acc[rr];
    }
    __syncthreads();
    if (S_T)
        for (int e = t; e < D * CB; e += 256)
            S_T[(size_t)bh * DD + (size_t)(e / CB) * D + c0 + e % CB] = sS[e / CB][e % CB];
}

// The backward's combine, from the last segment: X(S) = dS_T (or 0),
// X(s) = M(s)^T X(s+1) + B(s); Xin(s) = X(s+1) is the adjoint entering
// segment s from its right, and dS0 = X(0).  Layout and work split as in
// sp_combine_kernel; row r of M^T X is column r of M against X, R
// consecutive entries of one M row per thread (two 16-byte reads).
template <int D>
__global__ __launch_bounds__(256) void sp_combine_adj_kernel(const float* dS_T, const float* Mg,
                                                             const float* Bg, float* Xin,
                                                             float* dS0, int H, int S)
{
    constexpr int CB = 16, R = D / 16, NBLK = D / CB;
    static_assert(R % 4 == 0, "rows per thread in 16-byte pieces");
    __shared__ __align__(16) float sS[D][CB];
    __shared__ __align__(16) float sM[D][D];
    const int bh = blockIdx.x / NBLK, c0 = (blockIdx.x % NBLK) * CB;
    const int b = bh / H, h = bh % H, t = threadIdx.x;
    const int j = t % CB, r0 = (t / CB) * R;
    const size_t DD = (size_t)D * D;
    for (int e = t; e < D * CB; e += 256)
        sS[e / CB][e % CB] = dS_T ? dS_T[(size_t)bh * DD + (size_t)(e / CB) * D + c0 + e % CB] : 0.f;
    for (int s = S - 1; s >= 0; --s) {
        const size_t seg = ((size_t)(b * S + s) * H + h) * DD;
        __syncthreads();
        for (int e = t; e < D * CB; e += 256)
            Xin[seg + (size_t)(e / CB) * D + c0 + e % CB] = sS[e / CB][e % CB];
        for (int e = 4 * t; e < D * D; e += 1024)
            *reinterpret_cast<float4*>(&sM[e / D][e % D]) =
                *reinterpret_cast<const float4*>(Mg + seg + e);
        __syncthreads();
        float acc[R];
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
            acc[rr] = Bg[seg + (size_t)(r0 + rr) * D + c0 + j];
        for (int k = 0; k < D; ++k) {
            const float x = sS[k][j];
#pragma unroll
            for (int q = 0; q < R; q += 4) {
                const float4 m = *reinterpret_cast<const float4*>(&sM[k][r0 + q]);
                acc[q] = fmaf(m.x, x, acc[q]);
                acc[q + 1] = fmaf(m.y, x, acc[q + 1]);
                acc[q + 2] = fmaf(m.z, x, acc[q + 2]);
                acc[q + 3] = fmaf(m.w, x, acc[q + 3]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
            sS[r0 + rr][j] = acc[rr];
    }
    __syncthreads();
    if (dS0)
        for (int e = t; e < D * CB; e += 256)
            dS0[(size_t)bh * DD + (size_t)(e / CB) * D + c0 + e % CB] = sS[e / CB][e % CB];
}

hipError_t launch_seqpar_fwd(const FwdArgs& a, bool iso, int S, float* ws, hipStream_t stream)
{
    const int B = a.B, T = a.T, H = a.H, DK = a.dk, DV = a.dv;
    const size_t bs = (size_t)B * S, width = iso ? 1 : (size_t)DK;
    const size_t st = bs * H * (size_t)DK * DV;
    const int nchunks = (T + 63) / 64, seg_chunks = (T / S) / 64;
    float* p = ws;
    float* gscan = p;
    p += r64(gain_workspace_floats(iso, B, T, H, DK));
    float* pin = p;
    p += r64(bs * H * width);
    float* vscr = p;
    p += r64(bs * H * width);
    float* Nb = p;
    p += r64(st);
    float* Mb = p;
    p += r64(st);
    float* Sin = p;
    p += r64(st);
    float* Ib = p;

    // 1. the variance entering every chunk (and the final variance)
    GainArgs g{a.k, a.alpha, a.omega, a.r, a.var0, nullptr, a.var_T, gscan,
               gscan + (size_t)B * H * 4 * width * nchunks, B, T, H, DK, a.mu};
    g.mu_h = a.mu_h;
    g.c0 = a.c0;
    hipError_t e = launch_gain_scan(g, iso, 1, stream);
    if (e != hipSuccess)
        return e;
    const size_t npin = bs * H * width;
    hipLaunchKernelGGL(sp_gather_var_kernel, dim3((unsigned)((npin + 255) / 256)), dim3(256), 0,
                       stream, (const float*)(gscan + (size_t)B * H * 4 * width * nchunks), pin, B,
                       H, S, (int)width, nchunks, seg_chunks);
    hipLaunchKernelGGL(sp_identity_kernel, dim3((unsigned)((st + 255) / 256)), dim3(256), 0, stream,
                       Ib, st, DK);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    // segments as batch rows
    FwdArgs w = a;
    w.B = (int)bs;
    w.T = T / S;
    w.var0 = pin;
    w.c0 = nullptr;
    w.var_T = vscr;
    w.beta = nullptr;
    // 2. N: from a zero state, the state only
    FwdArgs wn = w;
    wn.S0 = nullptr;
    wn.S_T = Nb;
    wn.state_only = 1;
    if ((e = launch_walk_fwd(wn, iso, stream)) != hipSuccess)
        return e;
    // 3. M: v = 0 from the identity, the state only
    FwdArgs wm = w;
    wm.S0 = Ib;
    wm.S_T = Mb;
    wm.state_only = 2;
    if ((e = launch_walk_fwd(wm, iso, stream)) != hipSuccess)
        return e;
    // 4. every segment's entry state and the final state
    if (DK == 128)
        hipLaunchKernelGGL(sp_combine_kernel<128>, dim3(B * H * (128 / 16)), dim3(256), 0, stream,
                           a.S0, Mb, Nb, Sin, a.S_T, H, S);
    else
        hipLaunchKernelGGL(sp_combine_kernel<64>, dim3(B * H * (64 / 16)), dim3(256), 0, stream,
                           a.S0, Mb, Nb, Sin, a.S_T, H, S);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    // 5. the outputs, from each segment's entry state
    FwdArgs wo = w;
    wo.S0 = Sin;
    wo.S_T = Nb;  // the segments' end states, not needed again
    wo.beta = a.beta;
    return launch_walk_fwd(wo, iso, stream);
}

hipError_t launch_seqpar_bwd_mem(const BwdArgs& a, bool iso, hipStream_t stream)
{
    const int B = a.B, T = a.T, H = a.H, D = a.dk, S = a.nseg;
    if (S < 2 || a.dv != D || T % (64 * S) != 0 || (D != 64 && D != 128) || !a.segws)
        return hipErrorInvalidValue;
    const size_t bs = (size_t)B * S, width = iso ? 1 : (size_t)D;
    const size_t st = bs * H * (size_t)D * D;
    const int nchunks = (T + 63) / 64, seg_chunks = (T / S) / 64;
    float* p = a.segws;
    float* pin = p;
    p += r64(bs * H * width);
    float* vscr = p;
    p += r64(bs * H * width);
    float* Nb = p;
    p += r64(st);
    float* Mb = p;
    p += r64(st);
    float* Sin = p;
    p += r64(st);
    float* Ib = p;
    p += r64(st);
    float* Bb = p;
    p += r64(st);
    float* Xin = p;

    // the variance entering every segment, from the gain scan's carries
    const size_t npin = bs * H * width;
    hipLaunchKernelGGL(sp_gather_var_kernel, dim3((unsigned)((npin + 255) / 256)), dim3(256), 0,
                       stream, (const float*)(a.gscan + (size_t)B * H * 4 * width * nchunks), pin,
                       B, H, S, (int)width, nchunks, seg_chunks);
    hipLaunchKernelGGL(sp_identity_kernel, dim3((unsigned)((st + 255) / 256)), dim3(256), 0, stream,
                       Ib, st, D);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    // 1-3. every segment's entry state: the state walks (split-bf16 products
    // for Diagonal, as the forward's default) and the combine
    FwdArgs w{};
    w.q = a.q;
    w.k = a.k;
    w.v = a.v;
    w.alpha = a.alpha;
    w.omega = a.omega;
    w.r = a.r;
    w.var0 = pin;
    w.var_T = vscr;
    w.B = (int)bs;
    w.T = T / S;
    w.H = H;
    w.dk = D;
    w.dv = D;
    w.mu = a.mu;
    w.mu_h = a.mu_h;
    w.split = !iso;
    FwdArgs wn = w;
    wn.S_T = Nb;
    wn.state_only = 1;
    if ((e = launch_walk_fwd(wn, iso, stream)) != hipSuccess)
        return e;
    FwdArgs wm = w;
    wm.S0 = Ib;
    wm.S_T = Mb;
    wm.state_only = 2;
    if ((e = launch_walk_fwd(wm, iso, stream)) != hipSuccess)
        return e;
    if (D == 128)
        hipLaunchKernelGGL(sp_combine_kernel<128>, dim3(B * H * (128 / 16)), dim3(256), 0, stream,
                           a.S0, Mb, Nb, Sin, (float*)nullptr, H, S);
    else
        hipLaunchKernelGGL(sp_combine_kernel<64>, dim3(B * H * (64 / 16)), dim3(256), 0, stream,
                           a.S0, Mb, Nb, Sin, (float*)nullptr, H, S);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    // segments as batch rows
    BwdArgs v = a;
    v.B = (int)bs;
    v.T = T / S;
    v.nseg = 0;
    v.segws = nullptr;
    // 4. each segment's own adjoint at its start
    BwdArgs va = v;
    va.S0 = nullptr;
    va.gS_T = nullptr;
    va.gS0 = Bb;
    if ((e = launch_bwd_chunk_mem(va, iso, 1, true, stream)) != hipSuccess)
        return e;
    // 5. the adjoint entering every segment, and dS0
    if (D == 128)
        hipLaunchKernelGGL(sp_combine_adj_kernel<128>, dim3(B * H * (128 / 16)), dim3(256), 0,
                           stream, a.gS_T, Mb, Bb, Xin, a.gS0, H, S);
    else
        hipLaunchKernelGGL(sp_combine_adj_kernel<64>, dim3(B * H * (64 / 16)), dim3(256), 0,
                           stream, a.gS_T, Mb, Bb, Xin, a.gS0, H, S);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    // 6. the per-token gradients, every segment from its entry state and
    // incoming adjoint; the chunk-start states from a state-only walk of the
    // segments from their entry states
    FwdArgs wc = w;
    wc.S0 = Sin;
    wc.S_T = Nb;  // not needed again
    wc.state_only = 1;
    wc.ckpt = a.ckpt;
    if ((e = launch_walk_fwd(wc, iso, stream)) != hipSuccess)
        return e;
    BwdArgs vf = v;
    vf.S0 = Sin;
    vf.gS_T = Xin;
    vf.gS0 = nullptr;
    vf.ckpt_given = true;
    return launch_bwd_chunk_mem(vf, iso, 1, false, stream);
}

}  // namespace kdn
