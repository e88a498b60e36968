// kdn_gain.hip -- the KDN gain scan on its own (variance recurrence + Kalman
// gain, no memory), gfx950.
//
// The per-channel variance recurrence of Diagonal KDN is a fractional-linear
// (Moebius) map of p_{t-1}; in homogeneous coordinates one token is
//   M_t = [[alpha^2, omega], [u alpha^2, 1 + u omega]],  u = (mu / r_t) k^2
// (KDN reading notes, method part §6, Eq. (32)-(39)); Isotropic KDN has the
// same form for its scalar with alpha^2 -> mean_i alpha_i^2 and
// u = mu |k|^2 / (d_k r_t) (§7, Eq. (40), Appendix C).  Composition is
// associative but not commutative, so prefixes are taken in token order by
// left multiplication.  Following the chunked schedule the notes describe for
// Appendix D (chunk summaries, an exclusive carry across chunks, replay inside
// each chunk):
//   pass 1  summary of every 64-token chunk: Diagonal composes its channel's
//           64 maps serially in one lane (lanes = channels, coalesced loads);
//           Isotropic scans the chunk's 64 maps across the lanes of one
//           wavefront with DPP.
//   pass 2  carry: one lane per (batch, head, channel) and eight runs of
//           chunks per lane's channel: each run's maps are composed, the runs
//           before a run are applied to the initial variance, then each run
//           applies its chunk summaries to the variance in chunk order (a 2x2
//           map of a scalar per chunk), giving every chunk's entry variance
//           and the final variance.
//   pass 3  (only when kappa is requested) replay each chunk from its entry
//           variance: p^_t, z_t = sum_i p^_t,i k_t,i^2, kappa = p^ k/(r + z);
//           Diagonal takes its chunk in four 16-token pieces, so that its LDS
//           tile of p^ k^2 stays small and more workgroups share a compute unit.
// Summaries are stored chunk-major, [B H][chunk][width][4] (one 16-byte map per
// channel), so that pass 1 writes whole rows and pass 2 reads them with lanes
// on adjacent channels.
// Every combine rescales by 1/max|entry| (entries are non-negative), which
// keeps the ratios and avoids fp32 overflow.
#include "kdn_common.h"

#include <algorithm>
#include <mutex>
#include "kdn_internal.h"
#include "kdn_ops.h"

namespace kdn {

__device__ __forceinline__ float mu_of(const GainArgs& a, int h) { return a.mu_h ? a.mu_h[h] : a.mu; }

constexpr int GC = GAIN_CHUNK;  // tokens per gain chunk

__device__ __forceinline__ Mob mob_mul_raw(const Mob& later, const Mob& earlier)
{
    return Mob{later.m00 * earlier.m00 + later.m01 * earlier.m10,
               later.m00 * earlier.m01 + later.m01 * earlier.m11,
               later.m10 * earlier.m00 + later.m11 * earlier.m10,
               later.m10 * earlier.m01 + later.m11 * earlier.m11};
}

__device__ __forceinline__ Mob mob_normalize(const Mob& r)
{
    const float s = rcp(fmaxf(fmaxf(r.m00, r.m01), fmaxf(r.m10, r.m11)));
    return Mob{r.m00 * s, r.m01 * s, r.m10 * s, r.m11 * s};
}

// Per-token isotropic factor inputs for the 64 tokens of a chunk, computed by
// a 256-thread block: 4 threads per token reduce alpha^2 and k^2 over the key
// channels.  Results land in sa[t] (mean alpha^2) and sn[t] (|k|^2).
template <typename IO, int DK>
__device__ __forceinline__ void iso_token_reductions(const GainArgs& a, int bh, int t0,
                                                     int n_valid, float* sa, float* sn)
{
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x;
    constexpr int TPT = 4, CPT = DK / TPT;
    const int t = tid / TPT, part = tid % TPT;
    const IO* kg = reinterpret_cast<const IO*>(a.k);
    float xa = 0.f, xn = 0.f;
    if (t < n_valid) {
        const size_t off = (((size_t)b * a.T + t0 + t) * a.H + h) * DK + part * CPT;
#pragma unroll
        for (int c = 0; c < CPT; c += 4) {
            const f32x4 al = *reinterpret_cast<const f32x4*>(a.alpha + off + c);
            xa += al[0] * al[0] + al[1] * al[1] + al[2] * al[2] + al[3] * al[3];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float kv = to_f32(kg[off + c + e]);
                xn += kv * kv;
            }
        }
    }
    xa += __shfl_xor(xa, 1);
    xn += __shfl_xor(xn, 1);
    xa += __shfl_xor(xa, 2);
    xn += __shfl_xor(xn, 2);
    if (part == 0) {
        sa[t] = (t < n_valid) ? xa * (1.f / DK) : 1.f;
        sn[t] = xn;
    }
}

// ---------------------------------------------------------------- pass 1
template <typename IO, int DK>
__global__ __launch_bounds__(DK) void gain_summary_diag(GainArgs a, int nchunks)
{
    const int bh = blockIdx.x / nchunks, c = blockIdx.x % nchunks;
    const int b = bh / a.H, h = bh % a.H, i = threadIdx.x;
    const int t0 = c * GC, n_valid = min(GC, a.T - t0);
    const IO* kg = reinterpret_cast<const IO*>(a.k);
    Mob P = mob_identity();
    // eight tokens' gates are loaded before the product chain that consumes them
    constexpr int PF = 8;
    for (int tb = 0; tb < n_valid; tb += PF) {
        float al[PF], w[PF], kv[PF], rt[PF];
#pragma unroll
        for (int e = 0; e < PF; ++e) {
            const size_t tok = ((size_t)b * a.T + t0 + min(tb + e, n_valid - 1)) * a.H + h;
            al[e] = a.alpha[tok * DK + i];
            w[e] = a.omega[tok * DK + i];
            kv[e] = to_f32(kg[tok * DK + i]);
            rt[e] = a.r[tok];
        }
#pragma unroll
        for (int e = 0; e < PF; ++e) {
            const int t = tb + e;
            if (t < n_valid) {
                const float u = (mu_of(a, h) / rt[e]) * kv[e] * kv[e];
                const float a2 = al[e] * al[e];
                P = mob_mul_raw(Mob{a2, w[e], u * a2, 1.f + u * w[e]}, P);
                if ((t & 3) == 3)
                    P = mob_normalize(P);
            }
        }
    }
    P = mob_normalize(P);
    *reinterpret_cast<float4*>(a.summ + (((size_t)bh * nchunks + c) * DK + i) * 4) =
        float4{P.m00, P.m01, P.m10, P.m11};
}

template <typename IO, int DK>
__global__ __launch_bounds__(256) void gain_summary_iso(GainArgs a, int nchunks)
{
    __shared__ float sa[GC], sn[GC];
    const int bh = blockIdx.x / nchunks, c = blockIdx.x % nchunks;
    const int b = bh / a.H, h = bh % a.H;
    const int t0 = c * GC, n_valid = min(GC, a.T - t0);
    iso_token_reductions<IO, DK>(a, bh, t0, n_valid, sa, sn);
    __syncthreads();
    if (threadIdx.x < 64) {
        const int t = threadIdx.x;
        Mob m = mob_identity();
        if (t < n_valid) {
            const size_t tok = ((size_t)b * a.T + t0 + t) * a.H + h;
            const float u = mu_of(a, h) * sn[t] / ((float)DK * a.r[tok]);
            const float w = a.omega[tok];
            m = Mob{sa[t], w, u * sa[t], 1.f + u * w};
        }
        const Mob incl = mob_wave_scan_inclusive(m);
        if (t == 63)
            *reinterpret_cast<float4*>(a.summ + ((size_t)bh * nchunks + c) * 4) =
                float4{incl.m00, incl.m01, incl.m10, incl.m11};
    }
}

// ---------------------------------------------------------------- pass 2
// One lane per (bh, channel), 64 channels per wavefront, up to CARRY_WAVES
// wavefronts per workgroup (one per 64 chunks: blockDim.x / 64 of them), each
// over its own contiguous run of chunks: every
// wave composes its run's maps into one (normalised products, later on the
// left), the waves exchange those through LDS so that wave w applies the runs
// before its own to the initial variance, then each wave walks its run again,
// p entering chunk c, then p <- (m00 p + m01) / (m10 p + m11) with chunk c's
// summary.  Two serial passes over nchunks / waves maps instead of one over
// nchunks; maps are read PF chunks ahead through a register ring.
constexpr int CARRY_WAVES = 8;
__global__ __launch_bounds__(64 * CARRY_WAVES) void gain_carry(GainArgs a, int width, int nchunks)
{
    __shared__ float4 run_map[CARRY_WAVES][64];
    const int groups = (width + 63) / 64;
    const int bh = blockIdx.x / groups, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int i = (blockIdx.x % groups) * 64 + lane;
    const bool live = i < width;
    const int nwave = blockDim.x >> 6;
    const int per = (nchunks + nwave - 1) / nwave;
    const int c_begin = min(nchunks, wv * per), c_end = min(nchunks, c_begin + per);
    const int ic = live ? i : 0;  // lanes past the last channel read channel 0 and store nothing
    const float4* s = reinterpret_cast<const float4*>(a.summ) + (size_t)bh * nchunks * width + ic;
    constexpr int PF = 24;
    float4 ring[PF];
    // chunk indices clamped into the run (an empty run reads nothing)
    auto load = [&](int c) { return s[(size_t)min(c, c_end - 1) * width]; };
    auto prime = [&]() {
        if (c_begin < c_end) {
#pragma unroll
            for (int e = 0; e < PF; ++e)
                ring[e] = load(c_begin + e);
        }
    };
    // 1. this run's composed map (the last wave's is not needed)
    Mob run = mob_identity();
    const int c_comp_end = wv + 1 < nwave ? c_end : c_begin;
    if (c_begin < c_comp_end)
        prime();
    for (int c0 = c_begin; c0 < c_comp_end; c0 += PF) {
#pragma unroll
        for (int e = 0; e < PF; ++e) {
            const int c = c0 + e;
            const float4 m = ring[e];
            ring[e] = load(c + PF);
            if (c < c_comp_end) {
                run = mob_mul_raw(Mob{m.x, m.y, m.z, m.w}, run);
                if ((e & 3) == 3)
                    run = mob_normalize(run);
            }
        }
    }
    run = mob_normalize(run);
    run_map[wv][lane] = float4{run.m00, run.m01, run.m10, run.m11};
    __syncthreads();
    // 2. the variance entering this run
    float p = live ? (a.var0 ? a.var0[(size_t)bh * width + i] : (a.c0 ? a.c0[bh % a.H] : 1.f)) : 1.f;
    for (int w2 = 0; w2 < wv; ++w2) {
        const float4 m = run_map[w2][lane];
        p = mob_apply(Mob{m.x, m.y, m.z, m.w}, p);
    }
    // 3. every chunk's entry variance
    float* out = a.carry + (size_t)bh * nchunks * width + ic;
    prime();
    for (int c0 = c_begin; c0 < c_end; c0 += PF) {
#pragma unroll
        for (int e = 0; e < PF; ++e) {
            const int c = c0 + e;
            const float4 m = ring[e];
            ring[e] = load(c + PF);
            if (c < c_end) {
                if (live)
                    out[(size_t)c * width] = p;
                p = mob_apply(Mob{m.x, m.y, m.z, m.w}, p);
            }
        }
    }
    // the last run ends with the final variance (the first wave when there
    // are no chunks at all)
    const int last = nchunks > 0 ? (nchunks - 1) / per : 0;
    if (live && wv == last && a.var_T)
        a.var_T[(size_t)bh * width + i] = p;
}

// ---------------------------------------------------------------- pass 3
template <typename IO, int DK>
__global__ __launch_bounds__(DK) void gain_replay_diag(GainArgs a, int nchunks)
{
    // The chunk in NQ pieces of HT tokens (a small LDS tile, so that more
    // workgroups fit on a compute unit): s_w[t][i] = p^_t,i k_t,i^2 (rows
    // padded to keep 16-byte reads aligned); z_t is the sum of row t, taken
    // by NP lanes per token
    constexpr int NQ = 4, HT = GC / NQ, LDW = DK + 4, NP = DK / HT, CPP = DK / NP;
    static_assert(NP * HT == DK, "one lane per (part, token) in the reduction");
    __shared__ __align__(16) float s_w[HT][LDW];
    __shared__ float s_zp[NP][HT];
    const int bh = blockIdx.x / nchunks, c = blockIdx.x % nchunks;
    const int b = bh / a.H, h = bh % a.H, i = threadIdx.x;
    const int t0 = c * GC, n_valid = min(GC, a.T - t0);
    const IO* kg = reinterpret_cast<const IO*>(a.k);
    float p = a.carry[((size_t)bh * nchunks + c) * DK + i];
    // eight tokens' gates are loaded before the chain (and the pprev stores,
    // which the compiler cannot move loads across) consume them
    constexpr int PF = 8;
#pragma unroll
    for (int hf = 0; hf < NQ; ++hf) {
        float num[HT];  // p^_t k_t of this lane's channel (kappa's numerator)
#pragma unroll
        for (int tb = 0; tb < HT; tb += PF) {
            float al8[PF], w8[PF], kv8[PF], r8[PF];
#pragma unroll
            for (int e = 0; e < PF; ++e) {
                const int t = hf * HT + tb + e;
                const size_t tok = ((size_t)b * a.T + t0 + min(t, n_valid - 1)) * a.H + h;
                al8[e] = a.alpha[tok * DK + i];
                w8[e] = a.omega[tok * DK + i];
                kv8[e] = to_f32(kg[tok * DK + i]);
                r8[e] = a.r[tok];
            }
#pragma unroll
            for (int e = 0; e < PF; ++e) {
                const int tl = tb + e, t = hf * HT + tl;
                float ph = 0.f, kv = 0.f;
                if (t < n_valid) {
                    const size_t tok = ((size_t)b * a.T + t0 + t) * a.H + h;
                    kv = kv8[e];
                    ph = al8[e] * al8[e] * p + w8[e];
                    const float u = (mu_of(a, h) / r8[e]) * kv * kv;
                    if (a.pprev)
                        a.pprev[tok * DK + i] = p;
                    p = ph * rcp(1.f + u * ph);
                }
                num[tl] = ph * kv;
                s_w[tl][i] = num[tl] * kv;
            }
        }
        __syncthreads();
        {
            // lane (part, t): channels CPP part .. CPP part + CPP - 1 of token t
            const int t = i % HT, part = i / HT;
            {
                const float* row = &s_w[t][CPP * part];
                float z = 0.f;
#pragma unroll
                for (int j = 0; j < CPP; j += 4) {
                    const float4 w4 = *reinterpret_cast<const float4*>(row + j);
                    z += (w4.x + w4.y) + (w4.z + w4.w);
                }
                s_zp[part][t] = z;
            }
        }
        __syncthreads();
#pragma unroll
        for (int tl = 0; tl < HT; ++tl) {
            const int t = hf * HT + tl;
            if (t < n_valid) {
                const size_t tok = ((size_t)b * a.T + t0 + t) * a.H + h;
                float z = s_zp[0][tl];
#pragma unroll
                for (int q = 1; q < NP; ++q)
                    z += s_zp[q][tl];
                a.kappa[tok * DK + i] = num[tl] * rcp(a.r[tok] + z);
                if (a.dd && i == 0)
                    a.dd[tok] = a.r[tok] + z;
            }
        }
    }
}

template <typename IO, int DK>
__global__ __launch_bounds__(256) void gain_replay_iso(GainArgs a, int nchunks)
{
    __shared__ float sa[GC], sn[GC], sbeta[GC];
    const int bh = blockIdx.x / nchunks, c = blockIdx.x % nchunks;
    const int b = bh / a.H, h = bh % a.H;
    const int t0 = c * GC, n_valid = min(GC, a.T - t0);
    iso_token_reductions<IO, DK>(a, bh, t0, n_valid, sa, sn);
    __syncthreads();
    if (threadIdx.x < 64) {
        const int t = threadIdx.x;
        Mob m = mob_identity();
        float r = 1.f, w = 0.f;
        if (t < n_valid) {
            const size_t tok = ((size_t)b * a.T + t0 + t) * a.H + h;
            r = a.r[tok];
            w = a.omega[tok];
            const float u = mu_of(a, h) * sn[t] / ((float)DK * r);
            m = Mob{sa[t], w, u * sa[t], 1.f + u * w};
        }
        const Mob excl = mob_wave_shift_right(mob_wave_scan_inclusive(m));
        const float bprev = mob_apply(excl, a.carry[(size_t)bh * nchunks + c]);
        const float bhat = sa[t] * bprev + w;
        sbeta[t] = bhat * rcp(r + bhat * sn[t]);
        if (a.gsc && t < n_valid) {
            const size_t tok = ((size_t)b * a.T + t0 + t) * a.H + h;
            *reinterpret_cast<float4*>(a.gsc + tok * 4) = float4{sbeta[t], bprev, sa[t], sn[t]};
        }
    }
    __syncthreads();
    const IO* kg = reinterpret_cast<const IO*>(a.k);
    for (int e = threadIdx.x; a.kappa && e < n_valid * DK; e += 256) {
        const int t = e / DK, i = e % DK;
        const size_t idx = (((size_t)b * a.T + t0 + t) * a.H + h) * DK + i;
        a.kappa[idx] = sbeta[t] * to_f32(kg[idx]);
    }
}

// Scratch of the allocation-free gain scan (kdn_gain_scan_static): one copy
// per device, resident from the module's load until the process ends.  Host
// code reaches it only through the device address hipGetSymbolAddress returns
// (looked up once per device); the array's own name is a host-side stand-in.
static __device__ __align__(256) float scratch[GAIN_STATIC_FLOATS];

hipError_t gain_static_scratch(float** ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static float* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        addr[dev] = static_cast<float*>(p);
    }
    *ptr = addr[dev];
    return hipSuccess;
}

template <typename IO, int DK>
static hipError_t launch_gain_t(const GainArgs& a0, bool iso, hipStream_t stream)
{
    GainArgs a = a0;
    const int nchunks = (a.T + GC - 1) / GC;
    const int BH = a.B * a.H;
    const int width = iso ? 1 : DK;
    if (nchunks > 0) {
        if (iso)
            hipLaunchKernelGGL((gain_summary_iso<IO, DK>), dim3(BH * nchunks), dim3(256), 0,
                               stream, a, nchunks);
        else
            hipLaunchKernelGGL((gain_summary_diag<IO, DK>), dim3(BH * nchunks), dim3(DK), 0,
                               stream, a, nchunks);
    }
    const int carry_waves = std::min(CARRY_WAVES, std::max(1, nchunks / 64));
    hipLaunchKernelGGL(gain_carry, dim3(BH * ((width + 63) / 64)), dim3(64 * carry_waves), 0,
                       stream, a, width, nchunks);
    if ((a.kappa || a.gsc) && nchunks > 0) {
        if (iso)
            hipLaunchKernelGGL((gain_replay_iso<IO, DK>), dim3(BH * nchunks), dim3(256), 0,
                               stream, a, nchunks);
        else
            hipLaunchKernelGGL((gain_replay_diag<IO, DK>), dim3(BH * nchunks), dim3(DK), 0,
                               stream, a, nchunks);
    }
    return hipGetLastError();
}

hipError_t launch_gain_scan(const GainArgs& a, bool iso, int io_dtype, hipStream_t stream)
{
    if (io_dtype == 1)
        return a.dk == 128 ? launch_gain_t<bf16, 128>(a, iso, stream)
                           : launch_gain_t<bf16, 64>(a, iso, stream);
    return a.dk == 128 ? launch_gain_t<float, 128>(a, iso, stream)
                       : launch_gain_t<float, 64>(a, iso, stream);
}

}  // namespace kdn
