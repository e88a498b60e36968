// kdn_chunk.hip -- chunkwise KDN forward ("walk" regime), gfx950.
//
// One workgroup owns one (batch, head, value tile of DVT columns) and walks
// the sequence in chunks of C = 64 tokens.  The memory state S (dk x DVT,
// fp32) lives in MFMA accumulators for the whole sequence (held transposed,
// S^T[j][i]); the variance state lives in registers of the gain lanes.  Per
// chunk:
//
//  A  gain + operands (KDN reading notes, method part §4-§7):
//     Diagonal: one lane per key channel runs the per-channel recurrence
//       p^_t = alpha_t^2 p_{t-1} + omega_t,  p_t = p^_t / (1 + (mu/r_t) k_t^2 p^_t)
//     serially over the chunk, carrying p across chunks (the chunk carry of
//     Appendix D, held in a register).
//     Isotropic: per-token reductions a_t = mean alpha^2, n_t = |k_t|^2, then
//     one wavefront scans the scalar 2x2 Moebius maps of the chunk with DPP
//     (§6 Eq. (32)-(39), §7), carrying b across chunks.
//     Both write, with G_t = prod_{s<=t} alpha_s (cumulative decay from the
//     chunk start; decay ratios are G_t / G_s):
//       Kb  = k (.) G      (read keys, decayed)
//       Ktp = p^ (.) k / G (write keys without the 1/(r+z) factor)
//       Qb  = q (.) G
//  B  L' = Kb Ktp^T (its diagonal is z_t = sum_i p^ k^2), Aqk = tril(Qb Ktp^T)
//     (inclusive diagonal: the read sees this token's write), and per wave
//     R = V - Kb S, O = Qb S.
//  C  inverses of the 16x16 diagonal blocks of M = diag(r + z) + tril(L', -1).
//  D  blocked forward substitution M Delta' = R (Delta' = Delta / (r + z)),
//     O += Aqk Delta', S <- diag(G_C) (S + Ktp^T Delta').
//
// The chunk form is the affine memory scan S_t = (I - kappa_t k_t^T) D_t
// S_{t-1} + kappa_t v_t^T of §6 in compact-WY form (Appendix D, summarised in
// the notes), with the gain's 1/(r+z) folded into the triangular system; it
// equals the token recurrence exactly in exact arithmetic.  Ragged tails are
// padded with identity tokens (k = q = v = 0, alpha = 1, omega = 0, r = 1),
// which leave state and variances unchanged.
#include "kdn_common.h"
#include "kdn_internal.h"

namespace kdn {

constexpr int C = 64;  // tokens per chunk

template <typename IO, int DK, int DVT>
struct ChunkSmem {
    static constexpr int PADE = 16 / sizeof(IO);  // 16-byte row padding
    static constexpr int LD_K = DK + PADE;        // rows of Kb/Ktp/Qb/ShT
    static constexpr int LD_T = C + PADE;         // rows of KtpT/DeltaT/Aqk
    static constexpr int LD_V = DVT + PADE;
    static constexpr int LD_L = C + 4;            // fp32 L'
    static constexpr int LD_B = 16 + PADE;        // 16-wide blocks
    IO Kb[C * LD_K];
    IO Ktp[C * LD_K];
    IO Qb[C * LD_K];
    IO KtpT[DK * LD_T];
    IO ShT[DVT * LD_K];
    IO V[C * LD_V];
    IO Aqk[C * LD_T];
    IO Tii[4 * 16 * LD_B];
    IO DeltaT[DVT * LD_T];
    IO RhsT[DVT * LD_B];
    float Lp[C * LD_L];
    float gC[DK];
    float rr[2][C];    // r_t of this / next chunk
    float murt[2][C];  // mu / r_t
    // isotropic scan inputs / outputs
    float iso_a[C], iso_n[C], iso_w[C], iso_bh[C];
};

template <typename IO, int DK, int DVT, bool ISO>
__global__ __launch_bounds__(64 * (DVT / 16)) void kdn_chunk_fwd_kernel(FwdArgs a)
{
    constexpr int NW = DVT / 16;
    constexpr int NT = NW * 64;
    using SM = ChunkSmem<IO, DK, DVT>;
    static_assert(sizeof(SM) <= 160 * 1024, "LDS budget");
    static_assert(DK <= NT, "one gain lane per key channel");
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SM& sm = *reinterpret_cast<SM*>(smem_raw);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int g4 = lane >> 4, c16 = lane & 15;

    // XCD-aware tile order: workgroups are dispatched round-robin over the 8
    // XCDs, so consecutive logical tiles (the value tiles of one head, which
    // read the same keys and gates) are placed on the same XCD / L2.
    const int ntiles = a.dv / DVT;
    const int nblk = gridDim.x;
    int L = blockIdx.x;
    if ((nblk & 7) == 0)
        L = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    const int bh = L / ntiles, tile = L % ntiles;
    const int b = bh / a.H, h = bh % a.H;
    const int j0 = tile * DVT;
    const int T = a.T, H = a.H, dv = a.dv;
    const IO* __restrict__ qg = reinterpret_cast<const IO*>(a.q);
    const IO* __restrict__ kg = reinterpret_cast<const IO*>(a.k);
    const IO* __restrict__ vg = reinterpret_cast<const IO*>(a.v);
    IO* __restrict__ og = reinterpret_cast<IO*>(a.o);
    const size_t tok_stride_k = (size_t)H * DK;  // elements between tokens
    const size_t tok_stride_v = (size_t)H * dv;
    const size_t base_k = ((size_t)b * T * H + h) * DK;
    const size_t base_v = ((size_t)b * T * H + h) * dv;
    const size_t base_r = (size_t)b * T * H + h;

    // ---- state: S^T tile in accumulators, S^T[j][i], j = 16*wave + 4*g4 + r,
    // i = 16*n + c16
    f32x4 Sacc[DK / 16];
    {
        const float* S0 = a.S0 ? a.S0 + (size_t)bh * DK * dv : nullptr;
#pragma unroll
        for (int n = 0; n < DK / 16; ++n) {
            if (S0) {
                const int i = 16 * n + c16;
                Sacc[n] = *reinterpret_cast<const f32x4*>(S0 + (size_t)i * dv + j0 + 16 * wave +
                                                          4 * g4);
            } else {
                Sacc[n] = zero4();
            }
        }
    }
    // variance carry: Diagonal -> one channel per gain lane; Isotropic -> the
    // head's scalar, held by every lane of wave 0
    float pvar = 1.f;
    if (!ISO) {
        if (tid < DK && a.var0)
            pvar = a.var0[(size_t)bh * DK + tid];
    } else {
        if (a.var0)
            pvar = a.var0[bh];
    }
    const float mu = a.mu;

    auto load_r = [&](int chunk, int buf) {
        if (tid < C) {
            const int t = chunk * C + tid;
            const float rt = (t < T) ? a.r[base_r + (size_t)t * H] : 1.f;
            sm.rr[buf][tid] = rt;
            sm.murt[buf][tid] = mu / rt;
        }
    };

    const int nchunks = (T + C - 1) / C;
    if (nchunks > 0)
        load_r(0, 0);
    // S^ for the first chunk (bf16 / fp32 copy of S^T for the MFMA operands)
#pragma unroll
    for (int n = 0; n < DK / 16; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            sm.ShT[(16 * wave + 4 * g4 + r) * SM::LD_K + 16 * n + c16] = from_f32<IO>(Sacc[n][r]);
    __syncthreads();

    for (int ch = 0; ch < nchunks; ++ch) {
        const int t0 = ch * C;
        const int n_valid = min(C, T - t0);
        const int buf = ch & 1;

        // ================= A: gain and decayed operands =================
        if (ISO) {
            // A0: per-token reductions over the key channels
            constexpr int TPT = NT / C;     // threads per token
            constexpr int CPT = DK / TPT;   // channels per thread
            const int t = tid / TPT, part = tid % TPT;
            float sa = 0.f, sn = 0.f;
            if (t < n_valid) {
                const size_t off = base_k + (size_t)(t0 + t) * tok_stride_k + part * CPT;
#pragma unroll
                for (int c = 0; c < CPT; c += 4) {
                    const f32x4 al = *reinterpret_cast<const f32x4*>(a.alpha + off + c);
                    sa += al[0] * al[0] + al[1] * al[1] + al[2] * al[2] + al[3] * al[3];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float kv = to_f32(kg[off + c + e]);
                        sn += kv * kv;
                    }
                }
            }
#pragma unroll
            for (int m = 1; m < TPT; m <<= 1) {
                sa += __shfl_xor(sa, m);
                sn += __shfl_xor(sn, m);
            }
            if (part == 0) {
                sm.iso_a[t] = (t < n_valid) ? sa * (1.f / DK) : 1.f;
                sm.iso_n[t] = sn;
                sm.iso_w[t] = (t < n_valid) ? a.omega[base_r + (size_t)(t0 + t) * H] : 0.f;
            }
            __syncthreads();
            // A1: wavefront Moebius scan over the chunk's tokens (wave 0)
            if (wave == 0) {
                const int t = lane;
                const float at = sm.iso_a[t], nt = sm.iso_n[t], wt = sm.iso_w[t];
                const float ut = sm.murt[buf][t] * nt * (1.f / DK);
                Mob m{at, wt, ut * at, 1.f + ut * wt};
                const Mob incl = mob_wave_scan_inclusive(m);
                const Mob excl = mob_wave_shift_right(incl);
                const float bprev = mob_apply(excl, pvar);
                sm.iso_bh[t] = at * bprev + wt;
                // carry: the whole chunk applied to the entry variance
                const Mob last = Mob{__shfl(incl.m00, 63), __shfl(incl.m01, 63),
                                     __shfl(incl.m10, 63), __shfl(incl.m11, 63)};
                pvar = mob_apply(last, pvar);
            }
            __syncthreads();
        }

        if (tid < DK) {
            // one lane per key channel, serially over the chunk
            const int i = tid;
            float g = 1.f;
            const size_t off0 = base_k + (size_t)t0 * tok_stride_k + i;
#pragma unroll 8
            for (int t = 0; t < C; ++t) {
                float al = 1.f, wt = 0.f, kv = 0.f, qv = 0.f;
                if (t < n_valid) {
                    const size_t off = off0 + (size_t)t * tok_stride_k;
                    al = a.alpha[off];
                    if (!ISO)
                        wt = a.omega[off];
                    kv = to_f32(kg[off]);
                    qv = to_f32(qg[off]);
                }
                float ph;
                if (!ISO) {
                    ph = al * al * pvar + wt;
                    const float u = sm.murt[buf][t] * kv * kv;
                    pvar = ph * rcp(1.f + u * ph);
                } else {
                    ph = sm.iso_bh[t];
                }
                g *= al;
                const float ig = rcp(g);
                const float kt = ph * kv * ig;
                sm.Kb[t * SM::LD_K + i] = from_f32<IO>(kv * g);
                sm.Ktp[t * SM::LD_K + i] = from_f32<IO>(kt);
                sm.KtpT[i * SM::LD_T + t] = from_f32<IO>(kt);
                sm.Qb[t * SM::LD_K + i] = from_f32<IO>(qv * g);
            }
            sm.gC[i] = g;
        } else {
            // value tile of this chunk (rows padded with zeros)
            constexpr int VEC = 16 / sizeof(IO);
            constexpr int PER_ROW = DVT / VEC;
            for (int e = tid - DK; e < C * PER_ROW; e += NT - DK) {
                const int t = e / PER_ROW, c = (e % PER_ROW) * VEC;
                f32x4 raw = zero4();
                if (t < n_valid)
                    raw = *reinterpret_cast<const f32x4*>(vg + base_v +
                                                          (size_t)(t0 + t) * tok_stride_v + j0 + c);
                *reinterpret_cast<f32x4*>(&sm.V[t * SM::LD_V + c]) = raw;
            }
        }
        __syncthreads();

        // ================= B: chunk contractions =================
        {
            // shared lower-triangular tiles of L' (fp32) and Aqk (masked)
            constexpr int NJOB = 2 * 10;
            for (int job = wave; job < NJOB; job += NW) {
                const int which = job / 10, idx = job % 10;
                int mt = 0, nt2 = idx;
                while (nt2 > mt) {
                    nt2 -= mt + 1;
                    ++mt;
                }
                f32x4 acc = zero4();
                const IO* Arow = (which == 0 ? sm.Kb : sm.Qb) + 16 * mt * SM::LD_K;
                mma_nt(acc, Arow, SM::LD_K, sm.Ktp + 16 * nt2 * SM::LD_K, SM::LD_K, DK, lane);
                const int s = 16 * nt2 + c16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * mt + 4 * g4 + r;
                    if (which == 0)
                        sm.Lp[t * SM::LD_L + s] = acc[r];
                    else
                        sm.Aqk[t * SM::LD_T + s] = from_f32<IO>(s <= t ? acc[r] : 0.f);
                }
            }
        }
        // per wave: R = V - Kb S and O = Qb S for this wave's 16 columns
        f32x4 Racc[4], Oacc[4];
        {
            const IO* Sw = sm.ShT + 16 * wave * SM::LD_K;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 kr = zero4(), qo = zero4();
                mma_nt(kr, sm.Kb + 16 * mt * SM::LD_K, SM::LD_K, Sw, SM::LD_K, DK, lane);
                mma_nt(qo, sm.Qb + 16 * mt * SM::LD_K, SM::LD_K, Sw, SM::LD_K, DK, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * mt + 4 * g4 + r;
                    Racc[mt][r] = to_f32(sm.V[t * SM::LD_V + 16 * wave + c16]) - kr[r];
                }
                Oacc[mt] = qo;
            }
        }
        __syncthreads();

        // ================= C: inverses of the diagonal blocks =================
        if (wave == 0) {
            const int blk = g4, cc = c16;
            const float* M = sm.Lp + 16 * blk * SM::LD_L + 16 * blk;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = (r == cc) ? 1.f : 0.f;
#pragma unroll
                for (int c = 0; c < r; ++c)
                    s -= M[r * SM::LD_L + c] * x[c];
                const float diag = sm.rr[buf][16 * blk + r] + M[r * SM::LD_L + r];
                x[r] = s * rcp(diag);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sm.Tii[(blk * 16 + r) * SM::LD_B + cc] = from_f32<IO>(x[r]);
        }
        __syncthreads();

        // ================= D: triangular solve, output, state =================
        {
            IO* DeltaW = sm.DeltaT + 16 * wave * SM::LD_T;  // this wave's rows
            IO* RhsW = sm.RhsT + 16 * wave * SM::LD_B;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                f32x4 acc = zero4();
                for (int kb = 0; kb < blk; ++kb)
                    mma_nt_f32a(acc, sm.Lp + 16 * blk * SM::LD_L + 16 * kb, SM::LD_L,
                                DeltaW + 16 * kb, SM::LD_T, 16, lane);
                f32x4 rhs = Racc[blk] - acc;
                store4(RhsW + c16 * SM::LD_B + 4 * g4, rhs);
                wave_lds_sync();
                f32x4 d = zero4();
                mma_nt(d, sm.Tii + 16 * blk * SM::LD_B, SM::LD_B, RhsW, SM::LD_B, 16, lane);
                store4(DeltaW + c16 * SM::LD_T + 16 * blk + 4 * g4, d);
                wave_lds_sync();
            }
            // O += Aqk Delta'
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                mma_nt(Oacc[mt], sm.Aqk + 16 * mt * SM::LD_T, SM::LD_T, DeltaW, SM::LD_T,
                       16 * (mt + 1), lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * mt + 4 * g4 + r;
                    if (t < n_valid)
                        og[base_v + (size_t)(t0 + t) * tok_stride_v + j0 + 16 * wave + c16] =
                            from_f32<IO>(Oacc[mt][r]);
                }
            }
            // S <- diag(G_C) (S + Ktp^T Delta')   (held as S^T)
#pragma unroll
            for (int n = 0; n < DK / 16; ++n) {
                mma_nt(Sacc[n], DeltaW, SM::LD_T, sm.KtpT + 16 * n * SM::LD_T, SM::LD_T, C, lane);
                const float gc = sm.gC[16 * n + c16];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    Sacc[n][r] *= gc;
                    sm.ShT[(16 * wave + 4 * g4 + r) * SM::LD_K + 16 * n + c16] =
                        from_f32<IO>(Sacc[n][r]);
                }
            }
        }
        if (ch + 1 < nchunks)
            load_r(ch + 1, buf ^ 1);
        __syncthreads();
    }

    // ---- final state and variances
    float* ST = a.S_T + (size_t)bh * DK * dv;
#pragma unroll
    for (int n = 0; n < DK / 16; ++n) {
        const int i = 16 * n + c16;
        *reinterpret_cast<f32x4*>(ST + (size_t)i * dv + j0 + 16 * wave + 4 * g4) = Sacc[n];
    }
    if (tile == 0) {
        if (!ISO) {
            if (tid < DK)
                a.var_T[(size_t)bh * DK + tid] = pvar;
        } else if (tid == 0) {
            a.var_T[bh] = pvar;
        }
    }
}

template <typename IO, int DK, int DVT, bool ISO>
static hipError_t launch_one(const FwdArgs& a, hipStream_t stream)
{
    using SM = ChunkSmem<IO, DK, DVT>;
    auto kern = kdn_chunk_fwd_kernel<IO, DK, DVT, ISO>;
    const size_t smem = sizeof(SM);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess)
        return e;
    const int nblk = a.B * a.H * (a.dv / DVT);
    hipLaunchKernelGGL(kern, dim3(nblk), dim3(64 * (DVT / 16)), smem, stream, a);
    return hipGetLastError();
}

int chunk_fwd_value_tile(int io_dtype, int dk)
{
    (void)dk;
    return io_dtype == 1 ? 64 : 32;
}

hipError_t launch_chunk_fwd(const FwdArgs& a, bool iso, int io_dtype, hipStream_t stream)
{
    if (io_dtype == 1) {
        if (a.dk == 128)
            return iso ? launch_one<bf16, 128, 64, true>(a, stream)
                       : launch_one<bf16, 128, 64, false>(a, stream);
        return iso ? launch_one<bf16, 64, 64, true>(a, stream)
                   : launch_one<bf16, 64, 64, false>(a, stream);
    }
    return iso ? launch_one<float, 64, 32, true>(a, stream)
               : launch_one<float, 64, 32, false>(a, stream);
}

}  // namespace kdn
