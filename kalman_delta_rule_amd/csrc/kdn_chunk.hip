// kdn_chunk.hip -- chunkwise KDN forward ("walk" regime), gfx950.
//
// One workgroup owns one (batch, head, value tile of DVT columns) and walks
// the sequence in chunks of C = 32 tokens.  The memory state S (dk x DVT,
// fp32) stays in MFMA accumulators for the whole sequence (held transposed,
// S^T[j][i]); the variance state stays in registers.
//
// Method (KDN reading notes, method part):
//   gain   §4-§5 (Diagonal):  p^_t = alpha_t^2 p_{t-1} + omega_t,
//            p_t = p^_t / (1 + (mu / r_t) k_t^2 p^_t)
//          §7 (Isotropic): a_t = mean alpha^2, b^_t = a_t b_{t-1} + omega_t,
//            b_t = b^_t / (1 + mu |k_t|^2 b^_t / (d_k r_t)), as a wavefront
//            scan of 2x2 Moebius maps (§6 Eq. (32)-(39)).
//   memory §6: S_t = (I - kappa_t k_t^T) D_t S_{t-1} + kappa_t v_t^T,
//          kappa_t = p^_t (.) k_t / (r_t + z_t),  z_t = sum_i p^_t,i k_t,i^2,
//          o_t = S_t^T q_t (read after the write).
// Chunk form (compact WY, Appendix D as summarised in the notes), with
// G_t = prod_{s<=t} alpha_s the cumulative decay from the chunk start:
//   Kb = k (.) G,  Ktp = p^ (.) k / G,  Qb = q (.) G
//   L' = Kb Ktp^T  (diagonal = z_t),  Aqk = tril(Qb Ktp^T) (inclusive)
//   (diag(r + z) + tril(L', -1)) Delta' = V - Kb S        [Delta' = Delta/(r+z)]
//   O = Qb S + Aqk Delta',   S <- diag(G_C) (S + Ktp^T Delta')
// equal to the token recurrence in exact arithmetic.  Ragged tails are padded
// with identity tokens (k = q = v = 0, alpha = 1, omega = 0, r = 1).
//
// Workgroup schedule (warp-specialised, two barriers per chunk):
//   waves [0, NMM)      "memory" waves: each owns 16 value columns and runs
//                        the MFMA part of chunk c (L', Aqk, diagonal-block
//                        inverses recomputed per wave, R, O, triangular solve,
//                        state update) with wave-private LDS only;
//   waves NMM..NMM+3    "gain" waves, during the same segment: the serial
//                        variance / decay recurrence of chunk c+1 (one lane per
//                        key channel, or the isotropic DPP scan), and the
//                        loader for v and r of later chunks.  Their raw inputs
//                        sit in a rolling register buffer refilled one chunk
//                        ahead, so global latency overlaps a whole segment.
//   barrier (LDS only: in-flight global prefetches are not waited for)
//   all waves           elementwise build of Kb, Ktp, Ktp^T, Qb for chunk c+1
//   barrier
#include "kdn_common.h"
#include "kdn_internal.h"

namespace kdn {

constexpr int CH = 32;  // tokens per chunk

// Raw storage of one IO value in a 32-bit register (no conversion at load
// time, so the load is only waited for where the value is used).
__device__ __forceinline__ float raw_bits(float x) { return x; }
__device__ __forceinline__ float raw_bits(bf16 x)
{
    return __builtin_bit_cast(float, (uint32_t)__builtin_bit_cast(uint16_t, x));
}
template <typename IO>
__device__ __forceinline__ float from_raw_bits(float r);
template <>
__device__ __forceinline__ float from_raw_bits<float>(float r)
{
    return r;
}
template <>
__device__ __forceinline__ float from_raw_bits<bf16>(float r)
{
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, r) << 16);
}

template <typename IO>
struct VecOf;
template <>
struct VecOf<bf16> {
    using type = bf16x8;
};
template <>
struct VecOf<float> {
    using type = f32x4;
};

__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename IO, int DK, int DVT, bool ISO>
struct ChunkSmem {
    static constexpr int C = CH;
    static constexpr int NB = C / 16;
    static constexpr int NMM = DVT >= 64 ? DVT / 32 : DVT / 16;  // memory waves
    static constexpr int NJ = DVT / 16 / NMM;              // 16-column tiles per memory wave
    static constexpr int PADE = 16 / sizeof(IO);
    static constexpr int LD_K = DK + PADE;  // Kb, Ktp, Qb, ShT rows
    static constexpr int LD_T = C + PADE;   // KtpT, Aqk, Delta rows
    static constexpr int LD_V = DVT + PADE;
    static constexpr int LD_L = C + 4;      // fp32 L'
    static constexpr int LD_B = 16 + PADE;  // 16-wide blocks
    static constexpr int LD_G = DK + 4;     // fp32 gain staging rows
    static constexpr int LD_D = 16 + 4;     // fp32 transposed diagonal blocks
    struct MemWave {
        alignas(16) float LdT[NB * 16 * LD_D];  // diagonal blocks of L', transposed
        alignas(16) IO Loff[C * LD_T];          // L' below the diagonal blocks
        alignas(16) IO Aqk[C * LD_T];
        alignas(16) IO Tii[NB * 16 * LD_B];
        alignas(16) IO Delta[NJ * 16 * LD_T];
        alignas(16) IO Rhs[NJ * 16 * LD_B];
    };
    // gain staging [t][i], rewritten in place chunk after chunk:
    //   A  : alpha (fp32)  -> cumulative decay G
    //   W  : omega (fp32, Diagonal only)
    //   Kst: raw k (io dtype)
    alignas(16) float A[C * LD_G];
    alignas(16) float W[ISO ? 4 : C * LD_G];
    alignas(16) IO Kst[C * LD_K];
    alignas(16) float bhat[C];  // isotropic predicted variance
    alignas(16) IO Kb[C * LD_K];
    alignas(16) IO Qb[C * LD_K];
    // write keys are produced by the gain lanes while the memory waves still
    // read the previous chunk's: two buffers, indexed by chunk parity
    alignas(16) IO Ktp[2][C * LD_K];
    alignas(16) IO KtpT[2][DK * LD_T];
    alignas(16) IO ShT[DVT * LD_K];
    alignas(16) IO V[2][C * LD_V];
    alignas(16) float gC[DK];
    alignas(16) float rr[4][C];    // r_t ring
    alignas(16) float murt[4][C];  // mu / r_t ring
    alignas(16) float wring[4][C]; // isotropic omega_t ring
    MemWave mw[NMM];
};

// memory waves + 6 gain / loader waves
#define KDN_CHUNK_THREADS(DVT) (64 * (((DVT) >= 64 ? (DVT) / 32 : (DVT) / 16) + 6))

template <typename IO, int DK, int DVT, bool ISO>
__global__ __launch_bounds__(KDN_CHUNK_THREADS(DVT)) void kdn_chunk_fwd_kernel(FwdArgs a)
{
    constexpr int C = CH;
    constexpr int NB = C / 16;
    using SM0 = ChunkSmem<IO, DK, DVT, ISO>;
    constexpr int NMM = SM0::NMM;
    constexpr int NJ = SM0::NJ;
    constexpr int NW = NMM + 6;
    constexpr int NT = NW * 64;
    constexpr int NCH = DK / 64;         // waves for one lane per key channel
    constexpr int VE = 16 / sizeof(IO);  // IO elements per 16-byte vector
    constexpr int NV4 = VE / 4;          // fp32 16-byte vectors per unit
    using VecIO = typename VecOf<IO>::type;
    using SM = ChunkSmem<IO, DK, DVT, ISO>;
    static_assert(sizeof(SM) <= 160 * 1024, "LDS budget");
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SM& sm = *reinterpret_cast<SM*>(smem_raw);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int g4 = lane >> 4, c16 = lane & 15;

    // XCD-aware tile order: blocks are dispatched round-robin over the 8
    // XCDs, so consecutive logical tiles (the value tiles of one head, which
    // read the same keys and gates) land on the same XCD / L2.
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
    const size_t ts_k = (size_t)H * DK;  // elements between consecutive tokens
    const size_t ts_v = (size_t)H * dv;
    const size_t base_k = ((size_t)b * T * H + h) * DK;
    const size_t base_v = ((size_t)b * T * H + h) * dv;
    const size_t base_r = (size_t)b * T * H + h;
    const float mu = a.mu;
    const int nchunks = (T + C - 1) / C;
    auto n_valid = [&](int cc) { return min(C, T - cc * C); };

    // ---- roles
    const bool is_mm = wave < NMM;
    const int gw = wave - NMM;
    const bool is_chain = !ISO && !is_mm && gw < NCH;
    const bool is_scan = ISO && !is_mm && gw == 0;
    const bool is_loader = !is_mm && gw == 5;
    const int ch_i = (gw * 64 + lane) & (DK - 1);  // chain lane's key channel
    if (is_chain || is_scan)
        __builtin_amdgcn_s_setprio(2);  // the serial recurrence is the critical path

    // ------------------------------------------------------------ units
    // Every gain-side thread owns UPT units of (token t, VE consecutive key
    // channels); consecutive lanes cover consecutive channels of a token row,
    // so global loads are coalesced and LDS row accesses are conflict-free.
    // The memory waves take no units (their registers hold the state).
    constexpr int NTU = NT - NMM * 64;  // threads sharing the units
    const int utid = tid - NMM * 64;
    constexpr int UPR = DK / VE;        // units per token row
    constexpr int NUNITS = C * UPR;
    constexpr int UPT = (NUNITS + NTU - 1) / NTU;
    struct Stage {
        f32x4 al[NV4], om[NV4];
        f32x4 kn;  // raw 16 bytes of k
    };
    Stage st[UPT];
    f32x4 kcur[UPT], qcur[UPT];  // raw k, q of the chunk whose operands are built next

    // global -> registers: gates and k of chunk cs (staged later), q of chunk cq
    auto issue_loads = [&](int cs, int cq) {
        const int nvs = (cs < nchunks) ? n_valid(cs) : 0;
        const int nvq = (cq < nchunks) ? n_valid(cq) : 0;
        const size_t sbase = base_k + (size_t)(cs * C) * ts_k;  // uniform
        const size_t qbase = base_k + (size_t)(cq * C) * ts_k;
#pragma unroll
        for (int m = 0; m < UPT; ++m) {
            const int u = utid + NTU * m;
            const int t = u / UPR, i0 = (u % UPR) * VE;
            const uint32_t off = (uint32_t)(t * ts_k + i0);
            const bool uval = u < NUNITS;
#pragma unroll
            for (int e = 0; e < NV4; ++e) {
                st[m].al[e] = f32x4{1.f, 1.f, 1.f, 1.f};
                st[m].om[e] = zero4();
            }
            st[m].kn = zero4();
            qcur[m] = zero4();
            if (uval && t < nvs) {
#pragma unroll
                for (int e = 0; e < NV4; ++e) {
                    st[m].al[e] = *reinterpret_cast<const f32x4*>(a.alpha + sbase + off + 4 * e);
                    if (!ISO)
                        st[m].om[e] =
                            *reinterpret_cast<const f32x4*>(a.omega + sbase + off + 4 * e);
                }
                st[m].kn = *reinterpret_cast<const f32x4*>(kg + sbase + off);
            }
            if (uval && t < nvq)
                qcur[m] = *reinterpret_cast<const f32x4*>(qg + qbase + off);
        }
    };
    // registers -> LDS staging of chunk cs (identity tokens past the end)
    auto stage_store = [&](int cs) {
        if (cs >= nchunks)
            return;
#pragma unroll
        for (int m = 0; m < UPT; ++m) {
            const int u = utid + NTU * m;
            if (u < NUNITS) {
                const int t = u / UPR, i0 = (u % UPR) * VE;
#pragma unroll
                for (int e = 0; e < NV4; ++e) {
                    *reinterpret_cast<f32x4*>(&sm.A[t * SM::LD_G + i0 + 4 * e]) = st[m].al[e];
                    if (!ISO)
                        *reinterpret_cast<f32x4*>(&sm.W[t * SM::LD_G + i0 + 4 * e]) =
                            st[m].om[e];
                }
                *reinterpret_cast<f32x4*>(&sm.Kst[t * SM::LD_K + i0]) = st[m].kn;
            }
        }
    };
    // segment 2 (every wave): decayed read keys / queries of chunk cn, then
    // stage chunk cn + 1 into the slots just read (same thread, same addresses)
    auto elementwise = [&](int cn) {
        if (cn < nchunks) {
#pragma unroll
            for (int m = 0; m < UPT; ++m) {
                const int u = utid + NTU * m;
                if (u < NUNITS) {
                    const int t = u / UPR, i0 = (u % UPR) * VE;
                    const VecIO kv = __builtin_bit_cast(VecIO, kcur[m]);
                    const VecIO qv = __builtin_bit_cast(VecIO, qcur[m]);
                    VecIO kb, qb;
#pragma unroll
                    for (int e = 0; e < VE; ++e) {
                        const float G = sm.A[t * SM::LD_G + i0 + e];
                        kb[e] = from_f32<IO>(to_f32(kv[e]) * G);
                        qb[e] = from_f32<IO>(to_f32(qv[e]) * G);
                        if (t == C - 1)
                            sm.gC[i0 + e] = G;
                    }
                    *reinterpret_cast<VecIO*>(&sm.Kb[t * SM::LD_K + i0]) = kb;
                    *reinterpret_cast<VecIO*>(&sm.Qb[t * SM::LD_K + i0]) = qb;
                }
            }
        }
        stage_store(cn + 1);
#pragma unroll
        for (int m = 0; m < UPT; ++m)
            kcur[m] = st[m].kn;
    };

    // ------------------------------------------------------------ loader
    constexpr int PIECES_ROW = DVT / VE;
    constexpr int NPL = C * PIECES_ROW / 64;  // 16-byte v pieces per loader lane
    f32x4 vreg[NPL];
    float rreg = 1.f, wreg = 0.f;
    auto loader_load = [&](int cv, int cr) {
        const int nvv = (cv < nchunks) ? n_valid(cv) : 0;
        const IO* vc = vg + base_v + (size_t)(cv * C) * ts_v;  // uniform
#pragma unroll
        for (int m = 0; m < NPL; ++m) {
            const int p = lane + 64 * m;
            const int t = p / PIECES_ROW, sg = p % PIECES_ROW;
            vreg[m] = zero4();
            if (t < nvv)
                vreg[m] = *reinterpret_cast<const f32x4*>(vc + (uint32_t)(t * ts_v + j0 + sg * VE));
        }
        const int t = cr * C + lane;
        const bool ok = lane < C && t < T;
        rreg = ok ? a.r[base_r + (size_t)t * H] : 1.f;
        if (ISO)
            wreg = ok ? a.omega[base_r + (size_t)t * H] : 0.f;
    };

    // ------------------------------------------------------------ prologue
    if (!is_mm) {
        issue_loads(0, 0);
        stage_store(0);
#pragma unroll
        for (int m = 0; m < UPT; ++m)
            kcur[m] = st[m].kn;
        // staging loads are always issued one whole segment before their use:
        // gates / k of chunk c+2 and q of chunk c+1 leave at the end of
        // iteration c-1 and are consumed in the elementwise step of iteration c
        issue_loads(1, 0);
    }
    if (is_loader) {
        if (lane < C) {
            const bool ok = lane < T;
            const float rt = ok ? a.r[base_r + (size_t)lane * H] : 1.f;
            sm.rr[0][lane] = rt;
            sm.murt[0][lane] = mu / rt;
            if (ISO)
                sm.wring[0][lane] = ok ? a.omega[base_r + (size_t)lane * H] : 0.f;
        }
        loader_load(0, 1);
    }

    // Every role runs the same sequence of barriers: one after the prologue,
    // then two per iteration c = -1 .. nchunks-1 (s_barrier counts arrivals,
    // so the roles stay in lockstep while their register live ranges stay
    // apart).  In iteration c the gain side works on chunk c+1 and stages
    // chunk c+2 while the memory waves multiply chunk c.
    if (is_mm) {
        // ================= memory waves =================
        // wave owns NJ tiles of 16 value columns: local columns jw + 16 jt + ...
        const int jw = wave * 16 * NJ;
        f32x4 Sacc[NJ][DK / 16];
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
            for (int n = 0; n < DK / 16; ++n)
                Sacc[jt][n] = zero4();
        // accumulator layout: Sacc[jt][n][r] = S[i = 16 n + 4 g4 + r][j = jw + 16 jt + c16]
        if (a.S0) {
            const float* S0 = a.S0 + (size_t)bh * DK * dv + j0 + jw + c16;
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
                for (int n = 0; n < DK / 16; ++n)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Sacc[jt][n][r] = S0[(size_t)(16 * n + 4 * g4 + r) * dv + 16 * jt];
        }
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
            for (int n = 0; n < DK / 16; ++n)
                store4(&sm.ShT[(jw + 16 * jt + c16) * SM::LD_K + 16 * n + 4 * g4], Sacc[jt][n]);
        lds_barrier();
        auto& P = sm.mw[wave];
        {
            lds_barrier();
            lds_barrier();
        }
        for (int c = 0; c < nchunks; ++c) {
            {
                const int nv = n_valid(c);
                const size_t obase = base_v + (size_t)(c * C) * ts_v;  // uniform
                const IO* Vb = sm.V[c & 1];
                const IO* Ktpb = sm.Ktp[c & 1];
                const IO* KtpTb = sm.KtpT[c & 1];
                // Front contractions of the chunk, fused: every K-step loads the
                // Kb / Qb row fragments once and uses them for
                //   L'  = Kb Ktp^T (lower tiles),  Aqk = Qb Ktp^T (lower tiles),
                //   KS  = Kb S,                    O   = Qb S   (this wave's columns)
                using FR = Frag<IO>;
                f32x4 accL[NB][NB], accA[NB][NB], accR[NJ][NB], accO[NJ][NB];
#pragma unroll
                for (int mt = 0; mt < NB; ++mt) {
#pragma unroll
                    for (int nt = 0; nt < NB; ++nt) {
                        accL[mt][nt] = zero4();
                        accA[mt][nt] = zero4();
                    }
#pragma unroll
                    for (int jt = 0; jt < NJ; ++jt) {
                        accR[jt][mt] = zero4();
                        accO[jt][mt] = zero4();
                    }
                }
#pragma unroll
                for (int k0 = 0; k0 < DK; k0 += FR::KSTEP) {
                    typename FR::type aK[NB], aQ[NB], bT[NB], bS[NJ];
#pragma unroll
                    for (int mt = 0; mt < NB; ++mt) {
                        aK[mt] = FR::load(sm.Kb + 16 * mt * SM::LD_K, SM::LD_K, k0, lane);
                        aQ[mt] = FR::load(sm.Qb + 16 * mt * SM::LD_K, SM::LD_K, k0, lane);
                        bT[mt] = FR::load(Ktpb + 16 * mt * SM::LD_K, SM::LD_K, k0, lane);
                    }
#pragma unroll
                    for (int jt = 0; jt < NJ; ++jt)
                        bS[jt] = FR::load(sm.ShT + (jw + 16 * jt) * SM::LD_K, SM::LD_K, k0, lane);
#pragma unroll
                    for (int mt = 0; mt < NB; ++mt) {
#pragma unroll
                        for (int nt = 0; nt <= mt; ++nt) {
                            FR::mma(accL[mt][nt], aK[mt], bT[nt]);
                            FR::mma(accA[mt][nt], aQ[mt], bT[nt]);
                        }
#pragma unroll
                        for (int jt = 0; jt < NJ; ++jt) {
                            FR::mma(accR[jt][mt], aK[mt], bS[jt]);
                            FR::mma(accO[jt][mt], aQ[mt], bS[jt]);
                        }
                    }
                }
#pragma unroll
                for (int mt = 0; mt < NB; ++mt) {
#pragma unroll
                    for (int nt = 0; nt <= mt; ++nt) {
                        const int s = 16 * nt + c16;
                        if (nt == mt) {
                            // diagonal block, kept in fp32 and transposed:
                            // LdT[s][t] for the column-oriented substitution
                            *reinterpret_cast<f32x4*>(
                                &P.LdT[(16 * mt + c16) * SM::LD_D + 4 * g4]) = accL[mt][nt];
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int t = 16 * mt + 4 * g4 + r;
                            if (nt < mt)
                                P.Loff[t * SM::LD_T + s] = from_f32<IO>(accL[mt][nt][r]);
                            P.Aqk[t * SM::LD_T + s] =
                                from_f32<IO>(s <= t ? accA[mt][nt][r] : 0.f);
                        }
                    }
                }
                // R = V - Kb S
#pragma unroll
                for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
                    for (int mt = 0; mt < NB; ++mt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int t = 16 * mt + 4 * g4 + r;
                            accR[jt][mt][r] =
                                to_f32(Vb[t * SM::LD_V + jw + 16 * jt + c16]) - accR[jt][mt][r];
                        }
                wave_lds_sync();
                // inverses of the diagonal blocks of diag(r + z) + tril(L', -1)
                if (g4 < NB) {
                    // column cc of the inverse of the unit-free lower-triangular
                    // block M = diag(r + z) + tril(L', -1): forward substitution
                    // by columns of M (LdT rows), every update independent
                    const int blk = g4, cc = c16;
                    const float* Mt = P.LdT + 16 * blk * SM::LD_D;  // Mt[q][r] = M[r][q]
                    const float* rrc = sm.rr[c & 3] + 16 * blk;
                    float acc[16], x[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[r] = (r == cc) ? 1.f : 0.f;
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        float col[16];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const f32x4 v = *reinterpret_cast<const f32x4*>(Mt + q * SM::LD_D + 4 * e);
                            col[4 * e] = v[0];
                            col[4 * e + 1] = v[1];
                            col[4 * e + 2] = v[2];
                            col[4 * e + 3] = v[3];
                        }
                        x[q] = acc[q] * rcp(rrc[q] + col[q]);
#pragma unroll
                        for (int r = q + 1; r < 16; ++r)
                            acc[r] -= col[r] * x[q];
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        P.Tii[(blk * 16 + r) * SM::LD_B + cc] = from_f32<IO>(x[r]);
                }
                wave_lds_sync();
#pragma unroll
                for (int jt = 0; jt < NJ; ++jt) {
                    // blocked forward substitution for Delta'
                    IO* Dj = P.Delta + 16 * jt * SM::LD_T;
                    IO* Rj = P.Rhs + 16 * jt * SM::LD_B;
#pragma unroll
                    for (int blk = 0; blk < NB; ++blk) {
                        f32x4 acc = zero4();
#pragma unroll
                        for (int kb = 0; kb < blk; ++kb)
                            mma_nt(acc, P.Loff + 16 * blk * SM::LD_T + 16 * kb, SM::LD_T,
                                   Dj + 16 * kb, SM::LD_T, 16, lane);
                        store4(Rj + c16 * SM::LD_B + 4 * g4, accR[jt][blk] - acc);
                        wave_lds_sync();
                        f32x4 d = zero4();
                        mma_nt(d, P.Tii + 16 * blk * SM::LD_B, SM::LD_B, Rj, SM::LD_B, 16, lane);
                        store4(Dj + c16 * SM::LD_T + 16 * blk + 4 * g4, d);
                        wave_lds_sync();
                    }
                    // O += Aqk Delta'  and store
#pragma unroll
                    for (int mt = 0; mt < NB; ++mt) {
                        mma_nt(accO[jt][mt], P.Aqk + 16 * mt * SM::LD_T, SM::LD_T, Dj, SM::LD_T,
                               16 * (mt + 1), lane);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int t = 16 * mt + 4 * g4 + r;
                            if (t < nv)
                                (og + obase)[(uint32_t)(t * ts_v + j0 + jw + 16 * jt + c16)] =
                                    from_f32<IO>(accO[jt][mt][r]);
                        }
                    }
                    // S <- diag(G_C) (S + Ktp^T Delta'); the bf16 copy S^T feeds
                    // the next chunk's R / O contractions
#pragma unroll
                    for (int n = 0; n < DK / 16; ++n) {
                        mma_nt(Sacc[jt][n], KtpTb + 16 * n * SM::LD_T, SM::LD_T, Dj, SM::LD_T, C,
                               lane);
                        const f32x4 gc = *reinterpret_cast<const f32x4*>(&sm.gC[16 * n + 4 * g4]);
                        Sacc[jt][n] *= gc;
                        store4(&sm.ShT[(jw + 16 * jt + c16) * SM::LD_K + 16 * n + 4 * g4],
                               Sacc[jt][n]);
                    }
                }
            }
            lds_barrier();
            lds_barrier();
        }
        float* ST = a.S_T + (size_t)bh * DK * dv + j0 + jw + c16;
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
            for (int n = 0; n < DK / 16; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    ST[(size_t)(16 * n + 4 * g4 + r) * dv + 16 * jt] = Sacc[jt][n][r];
    } else if (is_chain) {
        // ====== Diagonal: per-channel recurrence from the LDS staging ======
        // lane = key channel; writes G (in place of alpha), the write keys
        // Ktp = p^ k / G in both layouts
        float pvar = a.var0 ? a.var0[(size_t)bh * DK + ch_i] : 1.f;
        lds_barrier();
        for (int c = -1; c < nchunks; ++c) {
            const int cn = c + 1;
            if (cn < nchunks) {
                const float* mr = sm.murt[cn & 3];
                IO* Ktpb = sm.Ktp[cn & 1];
                IO* KtpTb = sm.KtpT[cn & 1];
                float g = 1.f;
#pragma unroll
                for (int t4 = 0; t4 < C; t4 += 4) {
                    f32x4 kt4;
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const int t = t4 + x;
                        const int o = t * SM::LD_G + ch_i;
                        const float al = sm.A[o];
                        const float kv = to_f32(sm.Kst[t * SM::LD_K + ch_i]);
                        const float ph = al * al * pvar + sm.W[o];
                        const float u = mr[t] * kv * kv;
                        pvar = ph * rcp(1.f + u * ph);
                        g *= al;
                        sm.A[o] = g;
                        kt4[x] = ph * kv * rcp(g);
                        Ktpb[t * SM::LD_K + ch_i] = from_f32<IO>(kt4[x]);
                    }
                    store4(&KtpTb[ch_i * SM::LD_T + t4], kt4);
                }
            }
            lds_barrier();
            elementwise(cn);
            issue_loads(c + 3, cn + 1);
            lds_barrier();
        }
        if (tile == 0)
            a.var_T[(size_t)bh * DK + ch_i] = pvar;
    } else if (is_scan) {
        // ====== Isotropic: DPP Moebius scan, then the decay chain ======
        float pvar = a.var0 ? a.var0[bh] : 1.f;
        constexpr int SH = DK / 2;   // channels per lane in the reductions
        constexpr int CPL = DK / 64; // channels per lane in the decay chain
        lds_barrier();
        for (int c = -1; c < nchunks; ++c) {
            const int cn = c + 1;
            if (cn < nchunks) {
                {
                    // per-token reductions, two lanes per token
                    const int t = lane >> 1, half = lane & 1;
                    float sa = 0.f, sn = 0.f;
                    const float* Ar = sm.A + t * SM::LD_G + half * SH;
                    const IO* Kr = sm.Kst + t * SM::LD_K + half * SH;
#pragma unroll
                    for (int e = 0; e < SH; e += 4) {
                        const f32x4 av = *reinterpret_cast<const f32x4*>(Ar + e);
                        sa += av[0] * av[0] + av[1] * av[1] + av[2] * av[2] + av[3] * av[3];
                    }
#pragma unroll
                    for (int e = 0; e < SH; e += VE) {
                        const VecIO kv = *reinterpret_cast<const VecIO*>(Kr + e);
#pragma unroll
                        for (int x = 0; x < VE; ++x) {
                            const float f = to_f32(kv[x]);
                            sn += f * f;
                        }
                    }
                    sa += __shfl_xor(sa, 1);
                    sn += __shfl_xor(sn, 1);
                    // padded tokens were staged as alpha = 1, k = 0: a = 1, u = 0
                    const float at = sa * (1.f / DK);
                    const float wt = sm.wring[cn & 3][t];
                    const float ut = sm.murt[cn & 3][t] * sn * (1.f / DK);
                    const Mob m = (lane & 1) ? Mob{at, wt, ut * at, 1.f + ut * wt} : mob_identity();
                    // odd lane 2t+1 carries token t; the even lane 2t ends with
                    // the exclusive prefix (tokens < t)
                    const Mob incl = mob_wave_scan_inclusive(m);
                    if ((lane & 1) == 0)
                        sm.bhat[t] = at * mob_apply(incl, pvar) + wt;
                    const Mob last = Mob{__shfl(incl.m00, 63), __shfl(incl.m01, 63),
                                         __shfl(incl.m10, 63), __shfl(incl.m11, 63)};
                    pvar = mob_apply(last, pvar);
                }
                wave_lds_sync();
                // decay chain and write keys Ktp = b^ k / G, CPL channels per lane
                IO* Ktpb = sm.Ktp[cn & 1];
                IO* KtpTb = sm.KtpT[cn & 1];
                float g[CPL];
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc)
                    g[cc] = 1.f;
#pragma unroll
                for (int t4 = 0; t4 < C; t4 += 4) {
                    f32x4 kt4[CPL];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const int t = t4 + x;
                        const float bht = sm.bhat[t];
#pragma unroll
                        for (int cc = 0; cc < CPL; ++cc) {
                            const int i = lane + 64 * cc;
                            const int o = t * SM::LD_G + i;
                            g[cc] *= sm.A[o];
                            sm.A[o] = g[cc];
                            const float kv = to_f32(sm.Kst[t * SM::LD_K + i]);
                            kt4[cc][x] = bht * kv * rcp(g[cc]);
                            Ktpb[t * SM::LD_K + i] = from_f32<IO>(kt4[cc][x]);
                        }
                    }
#pragma unroll
                    for (int cc = 0; cc < CPL; ++cc)
                        store4(&KtpTb[(lane + 64 * cc) * SM::LD_T + t4], kt4[cc]);
                }
            }
            lds_barrier();
            elementwise(cn);
            issue_loads(c + 3, cn + 1);
            lds_barrier();
        }
        if (tile == 0 && lane == 0)
            a.var_T[bh] = pvar;
    } else {
        // ====== loader (v tile, r, iso omega) and spare waves ======
        lds_barrier();
        for (int c = -1; c < nchunks; ++c) {
            const int cn = c + 1;
            if (is_loader) {
                // v of chunk cn -> LDS; r / omega of chunk cn + 1 -> rings;
                // then prefetch v of cn + 1 and r / omega of cn + 2
                if (cn < nchunks) {
                    IO* Vd = sm.V[cn & 1];
#pragma unroll
                    for (int m = 0; m < NPL; ++m) {
                        const int p = lane + 64 * m;
                        const int t = p / PIECES_ROW, sg = p % PIECES_ROW;
                        *reinterpret_cast<f32x4*>(&Vd[t * SM::LD_V + sg * VE]) = vreg[m];
                    }
                }
                if (cn + 1 < nchunks && lane < C) {
                    sm.rr[(cn + 1) & 3][lane] = rreg;
                    sm.murt[(cn + 1) & 3][lane] = mu / rreg;
                    if (ISO)
                        sm.wring[(cn + 1) & 3][lane] = wreg;
                }
                asm volatile("" ::: "memory");
                loader_load(cn + 1, cn + 2);
            }
            lds_barrier();
            elementwise(cn);
            issue_loads(c + 3, cn + 1);
            lds_barrier();
        }
    }
}

template <typename IO, int DK, int DVT, bool ISO>
static hipError_t launch_one(const FwdArgs& a, hipStream_t stream)
{
    using SM = ChunkSmem<IO, DK, DVT, ISO>;
    auto kern = kdn_chunk_fwd_kernel<IO, DK, DVT, ISO>;
    const size_t smem = sizeof(SM);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess)
        return e;
    const int nblk = a.B * a.H * (a.dv / DVT);
    hipLaunchKernelGGL(kern, dim3(nblk), dim3(KDN_CHUNK_THREADS(DVT)), smem, stream, a);
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
