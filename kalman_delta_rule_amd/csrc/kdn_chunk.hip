// kdn_chunk.hip -- chunkwise KDN forward, gfx950.
//
// One workgroup owns one (batch, head, tile of DVT value columns) and walks
// the sequence in chunks of C = 16 tokens.  The memory state S (dk x DVT,
// fp32) lives in MFMA accumulators for the whole sequence; the variance state
// lives in registers of the chain lanes.
//
// Method (KDN reading notes, method part):
//   gain   §4-§5 (Diagonal):  p^_t = alpha_t^2 p_{t-1} + omega_t,
//            p_t = p^_t / (1 + (mu / r_t) k_t^2 p^_t)
//          §7 (Isotropic): a_t = mean alpha^2, b^_t = a_t b_{t-1} + omega_t,
//            b_t = b^_t / (1 + mu |k_t|^2 b^_t / (d_k r_t))
//   memory §6: S_t = (I - kappa_t k_t^T) D_t S_{t-1} + kappa_t v_t^T,
//          kappa_t = p^_t (.) k_t / (r_t + z_t),  z_t = sum_i p^_t,i k_t,i^2,
//          o_t = S_t^T q_t (read after the write).
// Chunk form (compact WY, Appendix D as summarised in the notes), with
// G_t = prod_{s<=t} alpha_s the cumulative decay from the chunk start:
//   Kb = k (.) G,  Ktp = p^ (.) k / G,  Qb = q (.) G
//   L' = Kb Ktp^T  (diagonal = z_t),  Aqk = tril(Qb Ktp^T) (inclusive)
//   M  = diag(r + z) + tril(L', -1),   T = M^-1
//   Delta' = T (V - Kb S),   O = Qb S + Aqk Delta',
//   S <- diag(G_C) (S + Ktp^T Delta')
// which equals the token recurrence in exact arithmetic.  Ragged tails are
// padded with identity tokens (k = q = v = 0, alpha = 1, omega = 0, r = 1).
//
// Workgroup pipeline, one LDS barrier per step.  In step c:
//   loader wave   copies the raw inputs of chunk c+5 straight from global
//                 memory into LDS (no registers), and v of chunk c+2;
//   chain wave(s) run the serial variance / decay recurrence of chunk c+3
//                 (one lane per key channel; the isotropic variant reduces
//                 over channels per token and runs the scalar recurrence);
//   memory waves  build Kb, Qb, Ktp of chunk c+2 (elementwise), then apply
//                 chunk c to their 16 value columns on the matrix cores;
//   factor wave   forms L', Aqk and T = M^-1 of chunk c+1 (matrix cores for
//                 the products, forward substitution for the inverse).
// Every buffer is indexed by chunk number modulo its lifetime, so no stage
// waits for another inside a step.
#include "kdn_common.h"
#include "kdn_internal.h"

#include <type_traits>

namespace kdn {

constexpr int CH = 16;      // tokens per chunk
constexpr int NSTAGE = 4;   // raw-input slots: in flight (2 steps) -> chain -> elementwise
constexpr int NOPS = 3;     // operand slots: elementwise -> factor -> memory
constexpr int NRING = 8;    // per-token scalar rings
constexpr int LEAD = 5;     // steps between loading a chunk and applying it

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Direct global -> LDS copy: lane l's 16 (or 4) bytes land at dst + 16 l
// (4 l).  dst must be uniform over the wave.  Completion is tracked by vmcnt.
__device__ __forceinline__ void dma16(const void* src, void* dst)
{
    __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* dst)
{
    __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)dst, 4, 0, 0);
}

template <int N>
__device__ __forceinline__ void vm_wait()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename IO>
struct Vec16;
template <>
struct Vec16<bf16> {
    using type = bf16x8;
};
template <>
struct Vec16<float> {
    using type = f32x4;
};

// 16x16x16 contraction pieces (K = 16) by element type.  An operand fragment
// holds, for lane (g = l >> 4, c = l & 15), the values X[m = c][k] of an A
// operand, or X[k][n = c] of a B operand, for the k the lane feeds (bf16: one
// 16x16x16 MFMA, k = 4 g + e; fp32: four 16x16x4 MFMAs, value s at k = 4 s + g).
//   lds   : row-major [m or n][k] in LDS (k contiguous)
//   lds_t : row-major [k][m or n] in LDS (k strided)
//   acc   : a 16x16 accumulator X in D layout, as the B operand X or the A
//           operand X^T.  bf16 only rounds (the D layout is the bf16 operand
//           layout); fp32 goes through a wave-private [16][17] LDS scratch.
template <typename T>
struct F16;
template <>
struct F16<bf16> {
    using type = bf16x4;
    static __device__ __forceinline__ type lds(const bf16* p, int ld, int lane)
    {
        return *reinterpret_cast<const bf16x4*>(p + (lane & 15) * ld + 4 * (lane >> 4));
    }
    // transpose read (ds_read_b64_tr_b16): inside each group of 16 lanes,
    // lane j receives element j & 3 of the 8-byte row segments addressed by
    // lanes 4 e + (j >> 2), e = 0..3; addressing row 4 g + ((l >> 2) & 3),
    // columns 4 (l & 3) .. +3 therefore yields X[k = 4 g + e][c] in lane (g, c)
    static __device__ __forceinline__ type lds_t(const bf16* p, int ld, int lane)
    {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const bf16* q = p + (4 * (lane >> 4) + ((lane >> 2) & 3)) * ld + 4 * (lane & 3);
        const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)q);
        return __builtin_bit_cast(bf16x4, r);
    }
    static __device__ __forceinline__ type acc(const f32x4& x, float* scratch, int lane)
    {
        (void)scratch;
        (void)lane;
        return bf16x4{static_cast<bf16>(x[0]), static_cast<bf16>(x[1]), static_cast<bf16>(x[2]),
                      static_cast<bf16>(x[3])};
    }
    static __device__ __forceinline__ void mma(f32x4& d, const type& a, const type& b)
    {
        d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, d, 0, 0, 0);
    }
};
template <>
struct F16<float> {
    struct type {
        float v[4];
    };
    static __device__ __forceinline__ type lds(const float* p, int ld, int lane)
    {
        const float* q = p + (lane & 15) * ld + (lane >> 4);
        return type{{q[0], q[4], q[8], q[12]}};
    }
    static __device__ __forceinline__ type lds_t(const float* p, int ld, int lane)
    {
        const float* q = p + (lane >> 4) * ld + (lane & 15);
        return type{{q[0], q[4 * ld], q[8 * ld], q[12 * ld]}};
    }
    static __device__ __forceinline__ type acc(const f32x4& x, float* scratch, int lane)
    {
        const int g = lane >> 4, c = lane & 15;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            scratch[(4 * g + r) * 17 + c] = x[r];
        wave_lds_sync();
        type t;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            t.v[s] = scratch[(4 * s + g) * 17 + c];
        wave_lds_sync();
        return t;
    }
    static __device__ __forceinline__ void mma(f32x4& d, const type& a, const type& b)
    {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            d = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], d, 0, 0, 0);
    }
};

template <typename IO, int DK, int DVT, bool ISO>
struct ChunkSmem {
    static constexpr int C = CH;
    static constexpr int NMM = DVT / 16;           // memory waves
    static constexpr int NCW = ISO ? 1 : DK / 64;  // chain waves
    static constexpr int PAD = 16 / sizeof(IO);
    static constexpr int LD_K = DK + PAD;  // Kb, Qb, Ktp rows (matrix-core operands)
    static constexpr int LD_S = C + PAD;   // T, Aqk rows
    // raw inputs of one chunk as rows of tokens, unpadded (filled by direct
    // copies); the chain overwrites alpha with G and (Diagonal) omega with p^ / G
    struct Stage {
        alignas(16) float alpha[C * DK];
        alignas(16) float omega[ISO ? 4 : C * DK];
        alignas(16) IO k[C * DK];
        alignas(16) IO q[C * DK];
        alignas(16) float cS[DK];  // per-channel decay reference c (a power of two)
        int cfl[4];                // per chain wave: some c != 1 in this chunk
    };
    struct Ops {
        alignas(16) IO Kb[C * LD_K];
        alignas(16) IO Qb[C * LD_K];
        alignas(16) IO Ktp[C * LD_K];
        alignas(16) float gC[DK];
        alignas(16) float cS[DK];
        int cfl;
    };
    struct Fac {
        alignas(16) IO T[C * LD_S];
        alignas(16) IO Aqk[C * LD_S];
    };
    Stage st[NSTAGE];
    alignas(16) IO v[3][C * DVT];    // rows of DVT, 16-byte block b of row t at b ^ (t & 7)
    Ops op[NOPS];
    Fac fac[2];
    alignas(16) float Mt[C * 20];    // factor: M^T (fp32), rows padded to 20
    alignas(16) float dinv[C];       // factor: 1 / (r_t + z_t)
    alignas(16) float rr[NRING][C];  // r_t
    alignas(16) float wr[NRING][C];  // isotropic omega_t
    alignas(16) float bh[NRING][C];  // isotropic b^_t
    alignas(16) float Tf[C * 20];    // factor: diagonal blocks of T (fp32)
    // fp32 operand hops: one per memory wave (fp32 io only), then the factor's
    alignas(16) float scratch[(sizeof(IO) == 4 ? NMM : 0) + 1][16 * 17];
};

#define KDN_CHUNK_THREADS(DK, DVT, ISO) (64 * ((DVT) / 16 + ((ISO) ? 1 : (DK) / 64) + 2))

template <typename IO, int DK, int DVT, bool ISO>
__global__ __launch_bounds__(KDN_CHUNK_THREADS(DK, DVT, ISO), 1) void kdn_chunk_fwd_kernel(
    FwdArgs a)
{
    using SM = ChunkSmem<IO, DK, DVT, ISO>;
    constexpr int C = CH;
    constexpr int NMM = SM::NMM;
    constexpr int NCW = SM::NCW;
    constexpr int LD_K = SM::LD_K;
    constexpr int LD_S = SM::LD_S;
    constexpr int VE = 16 / sizeof(IO);  // IO elements per 16 bytes
    static_assert(sizeof(SM) <= 160 * 1024, "LDS budget");
    static_assert(DK % 64 == 0 && DVT % 16 == 0, "tile shape");
    using F = F16<IO>;
    using FR = Frag<IO>;
    using VecIO = typename Vec16<IO>::type;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SM& sm = *reinterpret_cast<SM*>(smem_raw);

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
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
    const float mu = a.mu_h ? a.mu_h[h] : a.mu;
    const float var_init = a.c0 ? a.c0[h] : 1.f;  // variance when no var0 is given
    const int nchunks = (T + C - 1) / C;
    auto n_valid = [&](int x) { return min(C, T - x * C); };
    // global offsets (elements) of token t's row for this head
    auto row_k = [&](int t) { return (((size_t)b * T + t) * H + h) * DK; };
    auto row_v = [&](int t) { return (((size_t)b * T + t) * H + h) * dv; };
    auto row_s = [&](int t) { return ((size_t)b * T + t) * H + h; };

    if (wave < NMM) {
        // ===================== memory waves =====================
        // wave w owns value columns jl = 16 w + c16 of the tile; the state
        // block Sacc[n] holds S[16 n + 4 g4 + r][j0 + jl]
        const int w = wave;
        f32x4 Sacc[DK / 16];
        if (a.S0) {
            const float* S0 = a.S0 + (size_t)bh * DK * dv + j0 + 16 * w + c16;
#pragma unroll
            for (int n = 0; n < DK / 16; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Sacc[n][r] = S0[(size_t)(16 * n + 4 * g4 + r) * dv];
        } else {
#pragma unroll
            for (int n = 0; n < DK / 16; ++n)
                Sacc[n] = zero4();
        }
        float* scratch = sm.scratch[sizeof(IO) == 4 ? w : 0];
        IO* __restrict__ og = reinterpret_cast<IO*>(a.o);

        // elementwise build of Kb, Qb, Ktp (and gC) of chunk Y
        auto elementwise = [&](auto full_tag, int Y) {
            constexpr bool FULL = decltype(full_tag)::value;
            const int nvY = FULL ? C : n_valid(Y);
            auto& st = sm.st[Y % NSTAGE];
            auto& op = sm.op[Y % NOPS];
            constexpr int UPR = DK / VE;
            constexpr int NU = C * UPR;
#pragma unroll
            for (int u0 = 0; u0 < NU; u0 += NMM * 64) {
                const int u = u0 + w * 64 + lane;
                if (NU % (NMM * 64) != 0 && u >= NU)
                    break;
                const int t = u / UPR, i0 = (u % UPR) * VE;
                const bool ok = FULL || t < nvY;
                float G[VE], P[VE], kf[VE], qf[VE];
#pragma unroll
                for (int e = 0; e < VE; e += 4) {
                    const f32x4 gv = *reinterpret_cast<const f32x4*>(&st.alpha[t * DK + i0 + e]);
                    f32x4 pv;
                    if constexpr (ISO) {
                        const float bv = sm.bh[Y % NRING][t];
                        pv = f32x4{bv, bv, bv, bv};
                    } else {
                        pv = *reinterpret_cast<const f32x4*>(&st.omega[t * DK + i0 + e]);
                    }
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        G[e + x] = gv[x];
                        P[e + x] = pv[x];
                    }
                }
                const VecIO kv = *reinterpret_cast<const VecIO*>(&st.k[t * DK + i0]);
                const VecIO qv = *reinterpret_cast<const VecIO*>(&st.q[t * DK + i0]);
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    kf[e] = ok ? to_f32(kv[e]) : 0.f;
                    qf[e] = ok ? to_f32(qv[e]) : 0.f;
                }
                VecIO kb, qb, kt;
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    kb[e] = from_f32<IO>(kf[e] * G[e]);
                    qb[e] = from_f32<IO>(qf[e] * G[e]);
                    if constexpr (ISO)
                        kt[e] = from_f32<IO>(P[e] * kf[e] * rcp(G[e]));
                    else
                        kt[e] = from_f32<IO>(P[e] * kf[e]);  // P = p^ / G
                }
                *reinterpret_cast<VecIO*>(&op.Kb[t * LD_K + i0]) = kb;
                *reinterpret_cast<VecIO*>(&op.Qb[t * LD_K + i0]) = qb;
                *reinterpret_cast<VecIO*>(&op.Ktp[t * LD_K + i0]) = kt;
                if (t == C - 1) {
#pragma unroll
                    for (int e = 0; e < VE; e += 4) {
                        *reinterpret_cast<f32x4*>(&op.gC[i0 + e]) =
                            f32x4{G[e], G[e + 1], G[e + 2], G[e + 3]};
                        *reinterpret_cast<f32x4*>(&op.cS[i0 + e]) =
                            *reinterpret_cast<const f32x4*>(&st.cS[i0 + e]);
                    }
                    if (i0 == 0) {
                        int f = 0;
#pragma unroll
                        for (int x = 0; x < NCW; ++x)
                            f |= st.cfl[x];
                        op.cfl = f;
                    }
                }
            }
        };
        // chunk c on the matrix cores: front products, then the rest
        f32x4 accR, accO;
        auto mm_front = [&](int c) {
            const auto& op = sm.op[c % NOPS];
            // a chunk whose decay takes a reference c != 1 (Kb, Qb from G / c,
            // Ktp from c / G) is applied to diag(c) S; its G_C / c brings the
            // state back to S
            if (__builtin_amdgcn_readfirstlane(op.cfl)) {
#pragma unroll
                for (int n = 0; n < DK / 16; ++n)
                    Sacc[n] *= *reinterpret_cast<const f32x4*>(&op.cS[16 * n + 4 * g4]);
            }
            // R = Kb S  ([t][j], negated later),  O^T = S^T Qb^T  ([j][t])
            accR = zero4();
            accO = zero4();
#pragma unroll
            for (int n = 0; n < DK / 16; ++n) {
                const typename F::type s = F::acc(Sacc[n], scratch, lane);
                const typename F::type kf = F::lds(op.Kb + 16 * n, LD_K, lane);
                const typename F::type qf = F::lds(op.Qb + 16 * n, LD_K, lane);
                F::mma(accR, kf, s);
                F::mma(accO, s, qf);
            }
        };
        auto mm_rest = [&](auto full_tag, int c) {
            constexpr bool FULL = decltype(full_tag)::value;
            const int nv = FULL ? C : n_valid(c);
            const auto& op = sm.op[c % NOPS];
            const auto& fc = sm.fac[c & 1];
            const IO* V = sm.v[c % 3];
            // R = V - Kb S.  v[t][j]: 16-byte block j / VE of row t sits at
            // block (j / VE) ^ (t & 7) of that row
            {
                float vv[4];
                if constexpr (sizeof(IO) == 2) {
                    // transpose read of the 16 x 16 block (rows t, columns 16 w ..)
                    const int L = lane;
                    const int t = 4 * (L >> 4) + ((L >> 2) & 3);
                    const int col = 16 * w + 4 * (L & 3);
                    const int pos = (col / VE) ^ (t & 7);
                    typedef short s16x4 __attribute__((ext_vector_type(4)));
                    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
                    const s16x4 r4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(V + t * DVT + pos * VE + (col % VE)));
                    const bf16x4 b4 = __builtin_bit_cast(bf16x4, r4);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        vv[r] = to_f32(b4[r]);
                } else {
                    const int jl = 16 * w + c16;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 4 * g4 + r;
                        vv[r] = to_f32(V[t * DVT + ((jl / VE) ^ (t & 7)) * VE + (jl % VE)]);
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    accR[r] = ((FULL || 4 * g4 + r < nv) ? vv[r] : 0.f) - accR[r];
            }
            // Delta' = T R
            f32x4 accD = zero4();
            F::mma(accD, F::lds(fc.T, LD_S, lane), F::acc(accR, scratch, lane));
            const typename F::type dfr = F::acc(accD, scratch, lane);
            // O^T += Delta'^T Aqk^T
            F::mma(accO, dfr, F::lds(fc.Aqk, LD_S, lane));
            if (FULL || c16 < nv) {
                IO* dst = og + row_v(c * C + c16) + j0 + 16 * w + 4 * g4;
                if constexpr (sizeof(IO) == 2)
                    *reinterpret_cast<bf16x4*>(dst) =
                        bf16x4{static_cast<bf16>(accO[0]), static_cast<bf16>(accO[1]),
                               static_cast<bf16>(accO[2]), static_cast<bf16>(accO[3])};
                else
                    *reinterpret_cast<f32x4*>(dst) = accO;
            }
            // S <- diag(G_C) (S + Ktp^T Delta')
#pragma unroll
            for (int n = 0; n < DK / 16; ++n) {
                F::mma(Sacc[n], F::lds_t(op.Ktp + 16 * n, LD_K, lane), dfr);
                const f32x4 gc = *reinterpret_cast<const f32x4*>(&op.gC[16 * n + 4 * g4]);
                Sacc[n] *= gc;
            }
        };
        const std::integral_constant<bool, true> full{};
        const std::integral_constant<bool, false> ragged{};

        for (int c = -LEAD; c < nchunks; ++c) {
            const int Y = c + 2;
            if (c >= 0 && Y < nchunks && n_valid(Y) == C) {
                // steady state: both pieces in one block so that the
                // elementwise work overlaps the matrix-core latency
                mm_front(c);
                elementwise(full, Y);
                mm_rest(full, c);
            } else {
                if (Y >= 0 && Y < nchunks) {
                    if (n_valid(Y) == C)
                        elementwise(full, Y);
                    else
                        elementwise(ragged, Y);
                }
                if (c >= 0) {
                    mm_front(c);
                    if (n_valid(c) == C)
                        mm_rest(full, c);
                    else
                        mm_rest(ragged, c);
                }
            }
            lds_barrier();
        }
        float* ST = a.S_T + (size_t)bh * DK * dv + j0 + 16 * w + c16;
#pragma unroll
        for (int n = 0; n < DK / 16; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ST[(size_t)(16 * n + 4 * g4 + r) * dv] = Sacc[n][r];
    } else if (wave < NMM + NCW) {
        __builtin_amdgcn_s_setprio(2);  // the serial recurrence is the critical path
        if constexpr (!ISO) {
            // ================ Diagonal chain: lane = key channel ================
            // writes G over alpha and p^ / G over omega
            const int i = (wave - NMM) * 64 + lane;
            float p = a.var0 ? a.var0[(size_t)bh * DK + i] : var_init;
            auto chain = [&](auto full_tag, int X) {
                constexpr bool FULL = decltype(full_tag)::value;
                const int nv = FULL ? C : n_valid(X);
                auto& st = sm.st[X % NSTAGE];
                const float* rr = sm.rr[X % NRING];
                // every read is issued before the first use
                float al[C], om[C], mk2[C], rv[C];
#pragma unroll
                for (int t = 0; t < C; ++t) {
                    const float kv = to_f32(st.k[t * DK + i]);
                    al[t] = st.alpha[t * DK + i];
                    om[t] = st.omega[t * DK + i];
                    mk2[t] = mu * kv * kv;
                    rv[t] = rr[t];
                }
                if constexpr (!FULL) {
#pragma unroll
                    for (int t = 0; t < C; ++t) {
                        const bool ok = t < nv;
                        al[t] = ok ? al[t] : 1.f;
                        om[t] = ok ? om[t] : 0.f;
                        mk2[t] = ok ? mk2[t] : 0.f;
                        rv[t] = ok ? rv[t] : 1.f;
                    }
                }
                // g = G_t / c: c = 1 unless the chunk's plain product of
                // alphas falls below 2^-100 (decay_plain_ok, decay_ref)
                float af[C], g = 1.f;
#pragma unroll
                for (int t = 0; t < C; ++t) {
                    af[t] = al[t];
                    g *= al[t];
                }
                DecayRef ref{false, 0};
                if (__ballot(!decay_plain_ok(g)) != 0) {
                    if (!decay_plain_ok(g)) {
                        ref = decay_ref(al);
#pragma unroll
                        for (int t = 0; t < C; ++t)
                            af[t] = decay_alpha(ref, al[t]);
                    }
                }
                g = __builtin_amdgcn_ldexpf(1.f, -ref.m);
#pragma unroll
                for (int t = 0; t < C; ++t) {
                    // p = p^ / (1 + mu k^2 p^ / r) = p^ r / (r + mu k^2 p^)
                    const float ph = al[t] * al[t] * p + om[t];
                    const float den = mk2[t] * ph + rv[t];
                    p = ph * rv[t] * rcp(den);
                    g *= af[t];
                    st.alpha[t * DK + i] = g;
                    st.omega[t * DK + i] = ph * rcp(g);  // p^ c / G
                }
                st.cS[i] = __builtin_amdgcn_ldexpf(1.f, ref.m);
                const bool any = __ballot(ref.m != 0) != 0;
                if (lane == 0)
                    st.cfl[wave - NMM] = any;
            };
            for (int c = -LEAD; c < nchunks; ++c) {
                const int X = c + 3;
                if (X >= 0 && X < nchunks) {
                    if (n_valid(X) == C)
                        chain(std::integral_constant<bool, true>{}, X);
                    else
                        chain(std::integral_constant<bool, false>{}, X);
                }
                lds_barrier();
            }
            if (tile == 0)
                a.var_T[(size_t)bh * DK + i] = p;
        } else {
            // ======== Isotropic chain: one wave, DK / 64 channels per lane ========
            constexpr int CPL = DK / 64;
            float bvar = a.var0 ? a.var0[bh] : var_init;
            for (int c = -LEAD; c < nchunks; ++c) {
                const int X = c + 3;
                if (X >= 0 && X < nchunks) {
                    const int nv = n_valid(X);
                    auto& st = sm.st[X % NSTAGE];
                    // per-lane partial sums over its channels; G / c over alpha
                    float sa[C], sk[C];
                    bool anyc = false;
#pragma unroll
                    for (int t = 0; t < C; ++t) {
                        sa[t] = 0.f;
                        sk[t] = 0.f;
                    }
#pragma unroll
                    for (int cc = 0; cc < CPL; ++cc) {
                        const int i = lane + 64 * cc;
                        float alv[C], kvv[C];
#pragma unroll
                        for (int t = 0; t < C; ++t) {
                            alv[t] = st.alpha[t * DK + i];
                            kvv[t] = to_f32(st.k[t * DK + i]);
                        }
                        if (nv < C) {
#pragma unroll
                            for (int t = 0; t < C; ++t) {
                                alv[t] = t < nv ? alv[t] : 1.f;
                                kvv[t] = t < nv ? kvv[t] : 0.f;
                            }
                        }
                        // g = G_t / c (decay_plain_ok, decay_ref)
                        float af[C], g = 1.f;
#pragma unroll
                        for (int t = 0; t < C; ++t) {
                            af[t] = alv[t];
                            g *= alv[t];
                        }
                        DecayRef ref{false, 0};
                        if (__ballot(!decay_plain_ok(g)) != 0) {
                            if (!decay_plain_ok(g)) {
                                ref = decay_ref(alv);
#pragma unroll
                                for (int t = 0; t < C; ++t)
                                    af[t] = decay_alpha(ref, alv[t]);
                            }
                        }
                        g = __builtin_amdgcn_ldexpf(1.f, -ref.m);
#pragma unroll
                        for (int t = 0; t < C; ++t) {
                            sa[t] += alv[t] * alv[t];
                            sk[t] += kvv[t] * kvv[t];
                            g *= af[t];
                            st.alpha[t * DK + i] = g;
                        }
                        st.cS[i] = __builtin_amdgcn_ldexpf(1.f, ref.m);
                        anyc |= ref.m != 0;
                    }
                    {
                        const bool any = __ballot(anyc) != 0;
                        if (lane == 0)
                            st.cfl[0] = any;
                    }
                    // transpose-reduce over the 64 lanes: each halving step
                    // keeps half the tokens and adds the partner lane's
                    // partials of them; lane l ends with token l >> 2
                    static_assert(C == 16, "reduction tree shape");
                    auto halve = [&](auto hs_tag) {
                        constexpr int hs = decltype(hs_tag)::value;
                        constexpr int m = 4 * hs;  // partner lane distance
                        const bool up = (lane & m) != 0;
#pragma unroll
                        for (int j = 0; j < hs; ++j) {
                            const float ra = __shfl_xor(up ? sa[j] : sa[j + hs], m);
                            const float rk = __shfl_xor(up ? sk[j] : sk[j + hs], m);
                            sa[j] = (up ? sa[j + hs] : sa[j]) + ra;
                            sk[j] = (up ? sk[j + hs] : sk[j]) + rk;
                        }
                    };
                    halve(std::integral_constant<int, 8>{});
                    halve(std::integral_constant<int, 4>{});
                    halve(std::integral_constant<int, 2>{});
                    halve(std::integral_constant<int, 1>{});
                    float ta = sa[0], tk = sk[0];
                    ta += __shfl_xor(ta, 1);
                    tk += __shfl_xor(tk, 1);
                    ta += __shfl_xor(ta, 2);
                    tk += __shfl_xor(tk, 2);
                    // scalar recurrence over the chunk (uniform over the wave)
                    const float* rr = sm.rr[X % NRING];
                    const float* wr = sm.wr[X % NRING];
                    float bhv[C], rv[C], wv[C];
#pragma unroll
                    for (int t = 0; t < C; ++t) {
                        rv[t] = rr[t];
                        wv[t] = wr[t];
                    }
#pragma unroll
                    for (int t = 0; t < C; ++t) {
                        const bool ok = t < nv;
                        const float A2 = __builtin_bit_cast(
                            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ta), 4 * t));
                        const float K2 = __builtin_bit_cast(
                            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tk), 4 * t));
                        const float rt = ok ? rv[t] : 1.f;
                        const float wt = ok ? wv[t] : 0.f;
                        const float bhat = A2 * (1.f / DK) * bvar + wt;
                        const float dr = (float)DK * rt;
                        bvar = bhat * dr * rcp(dr + mu * K2 * bhat);
                        bhv[t] = bhat;
                    }
                    if (lane == 0) {
#pragma unroll
                        for (int t = 0; t < C; t += 4)
                            *reinterpret_cast<f32x4*>(&sm.bh[X % NRING][t]) =
                                f32x4{bhv[t], bhv[t + 1], bhv[t + 2], bhv[t + 3]};
                    }
                }
                lds_barrier();
            }
            if (tile == 0 && lane == 0)
                a.var_T[bh] = bvar;
        }
    } else if (wave == NMM + NCW) {
        // ===================== factor wave =====================
        __builtin_amdgcn_s_setprio(2);
        float* fscratch = sm.scratch[sizeof(IO) == 4 ? NMM : 0];
        for (int c = -LEAD; c < nchunks; ++c) {
            const int Fc = c + 1;
            if (Fc >= 0 && Fc < nchunks) {
                const int nv = n_valid(Fc);
                const auto& op = sm.op[Fc % NOPS];
                auto& fc = sm.fac[Fc & 1];
                const float* rr = sm.rr[Fc % NRING];
                // L'[t][s] = Kb_t . Ktp_s,   Aqk^T[u][t] = Ktp_u . Qb_t
                f32x4 accL = zero4(), accQ = zero4();
#pragma unroll
                for (int k0 = 0; k0 < DK; k0 += FR::KSTEP) {
                    const typename FR::type kb = FR::load(op.Kb, LD_K, k0, lane);
                    const typename FR::type kt = FR::load(op.Ktp, LD_K, k0, lane);
                    const typename FR::type qb = FR::load(op.Qb, LD_K, k0, lane);
                    FR::mma(accL, kb, kt);
                    FR::mma(accQ, kt, qb);
                }
                // M^T[s][t] = L'[t][s]   (lane holds L'[4 g4 + r][c16])
                *reinterpret_cast<f32x4*>(&sm.Mt[c16 * 20 + 4 * g4]) = accL;
                if ((c16 >> 2) == g4) {
                    const int rs = c16 & 3;
                    const float z = rs == 0 ? accL[0] : rs == 1 ? accL[1] : rs == 2 ? accL[2] : accL[3];
                    const float rraw = rr[c16];
                    const float rt = c16 < nv ? rraw : 1.f;
                    const float dvz = rcp(rt + z);
                    sm.dinv[c16] = dvz;
                    // effective write strength of token c16 (one tile writes it)
                    if (a.beta && tile == 0 && c16 < nv)
                        a.beta[row_s(Fc * C + c16)] = z * dvz;
                }
                // Aqk[t][u] = Aqk^T[u][t] for u <= t, else 0
                {
                    f32x4 aq;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        aq[r] = (4 * g4 + r <= c16) ? accQ[r] : 0.f;
                    store4(&fc.Aqk[c16 * LD_S + 4 * g4], aq);
                }
                wave_lds_sync();
                // T = M^-1, column c16 per lane: forward substitution over the
                // columns of M (rows of M^T)
                // T = M^-1 in two levels: the 8 x 8 diagonal blocks by forward
                // substitution (lane c16: block c16 >> 3, column c16 & 7, over
                // the columns of M = rows of M^T), then the off-diagonal block
                // T21 = -T22 M21 T11 on the matrix cores (fp32)
                {
                    const int bb = (c16 >> 3) * 8, cc = c16 & 7;
                    float di[8], Mc[8][8], acc[8], x[8];
                    {
                        const f32x4 d0 = *reinterpret_cast<const f32x4*>(&sm.dinv[bb]);
                        const f32x4 d1 = *reinterpret_cast<const f32x4*>(&sm.dinv[bb + 4]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            di[e] = d0[e];
                            di[4 + e] = d1[e];
                        }
                    }
#pragma unroll
                    for (int qq = 0; qq < 7; ++qq)
#pragma unroll
                        for (int e = (qq + 1) >> 2; e < 2; ++e) {
                            const f32x4 m = *reinterpret_cast<const f32x4*>(
                                &sm.Mt[(bb + qq) * 20 + bb + 4 * e]);
#pragma unroll
                            for (int r4 = 0; r4 < 4; ++r4)
                                Mc[qq][4 * e + r4] = m[r4];
                        }
#pragma unroll
                    for (int r = 0; r < 8; ++r)
                        acc[r] = (r == cc) ? 1.f : 0.f;
#pragma unroll
                    for (int qq = 0; qq < 8; ++qq) {
                        x[qq] = acc[qq] * di[qq];
#pragma unroll
                        for (int r = qq + 1; r < 8; ++r)
                            acc[r] -= Mc[qq][r] * x[qq];
                    }
                    if (g4 == 0) {
#pragma unroll
                        for (int r = 0; r < 8; ++r)
                            sm.Tf[(bb + r) * 20 + bb + cc] = x[r];
                    }
                }
                wave_lds_sync();
                {
                    using FF = F16<float>;
                    // P = M21 T11 :  A[m][k] = M[m][k] = M^T[k][m]  (m >= 8, k < 8)
                    //                B[k][n] = T11[k][n]            (k, n < 8)
                    FF::type am = FF::lds_t(sm.Mt, 20, lane);
                    FF::type bt = FF::lds_t(sm.Tf, 20, lane);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int k = 4 * e + g4;
                        am.v[e] = (c16 >= 8 && k < 8) ? am.v[e] : 0.f;
                        bt.v[e] = (k < 8 && c16 < 8) ? bt.v[e] : 0.f;
                    }
                    f32x4 accP = zero4();
                    FF::mma(accP, am, bt);
                    // T21 = -T22 P :  A[m][k] = T22[m][k] (m, k >= 8), B = P
                    FF::type a2 = FF::lds(sm.Tf, 20, lane);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int k = 4 * e + g4;
                        a2.v[e] = (c16 >= 8 && k >= 8) ? a2.v[e] : 0.f;
                    }
                    const FF::type bp = FF::acc(accP, fscratch, lane);
                    f32x4 accT = zero4();
                    FF::mma(accT, a2, bp);
                    // T in D layout: lane holds rows 4 g4 + r of column c16
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = 4 * g4 + r, n = c16;
                        float tv;
                        if (m >= 8 && n < 8)
                            tv = -accT[r];
                        else if ((m >> 3) == (n >> 3) && n <= m)
                            tv = sm.Tf[m * 20 + n];
                        else
                            tv = 0.f;
                        fc.T[m * LD_S + n] = from_f32<IO>(tv);
                    }
                }
            }
            lds_barrier();
        }
    } else {
        // ===================== loader wave =====================
        // direct copies into LDS: raw inputs of chunk c + LEAD, v of chunk c + 2
        constexpr int LPR_A = DK * 4 / 16;                  // lanes per alpha / omega row
        constexpr int RPI_A = 64 / LPR_A, NI_A = C / RPI_A; // rows per copy, copies
        constexpr int LPR_K = DK * (int)sizeof(IO) / 16;    // lanes per k / q row
        constexpr int RPI_K = 64 / LPR_K, NI_K = C / RPI_K;
        constexpr int LPR_V = DVT * (int)sizeof(IO) / 16;   // lanes per v tile row
        constexpr int RPI_V = 64 / LPR_V, NI_V = C / RPI_V;
        static_assert(LPR_A <= 64 && LPR_K <= 64 && LPR_V == 8 && NI_A >= 1 && NI_K >= 1,
                      "row / lane split");
        constexpr int NSTG = NI_A * (ISO ? 1 : 2) + 2 * NI_K + 1 + (ISO ? 1 : 0);
        constexpr int NVI = NI_V;
        static_assert(2 * (NSTG + NVI) <= 63, "outstanding copies within the vmcnt range");
        const float* __restrict__ alg = a.alpha;
        const float* __restrict__ omg = a.omega;
        const IO* __restrict__ kg = reinterpret_cast<const IO*>(a.k);
        const IO* __restrict__ qg = reinterpret_cast<const IO*>(a.q);
        const IO* __restrict__ vg = reinterpret_cast<const IO*>(a.v);
        // per-lane element offsets inside a chunk (32-bit; the chunk base is
        // uniform); rows past the end of a ragged chunk repeat its last row
        const uint32_t tsk = (uint32_t)(H * DK), tsv = (uint32_t)(H * dv), tss = (uint32_t)H;
        auto off_a = [&](int j, int lim) {
            return (uint32_t)min(j * RPI_A + lane / LPR_A, lim) * tsk + (lane % LPR_A) * 4;
        };
        auto off_k = [&](int j, int lim) {
            return (uint32_t)min(j * RPI_K + lane / LPR_K, lim) * tsk + (lane % LPR_K) * VE;
        };
        auto off_v = [&](int j, int lim) {
            const int p = 64 * j + lane;
            const int tl = p / LPR_V;
            const int blk = (p % LPR_V) ^ (tl & 7);
            return (uint32_t)min(tl, lim) * tsv + blk * VE;
        };
        uint32_t oa[NI_A], ok_[NI_K], ov[NI_V];
#pragma unroll
        for (int j = 0; j < NI_A; ++j)
            oa[j] = off_a(j, C - 1);
#pragma unroll
        for (int j = 0; j < NI_K; ++j)
            ok_[j] = off_k(j, C - 1);
#pragma unroll
        for (int j = 0; j < NI_V; ++j)
            ov[j] = off_v(j, C - 1);
        for (int c = -LEAD; c < nchunks; ++c) {
            const int X = c + LEAD;
            const bool sv = X < nchunks;
            const int XV = c + 2;
            const bool vv = XV >= 0 && XV < nchunks;
            if (sv) {
                auto& st = sm.st[X % NSTAGE];
                const int tb = X * C;
                const int lim = n_valid(X) - 1;
                const size_t cb = row_k(tb);  // uniform
                const float* ab = alg + cb;
                const float* wb = omg + cb;
                const IO* kb = kg + cb;
                const IO* qb = qg + cb;
                auto copy_stage = [&](auto full_tag) {
                    constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
                    for (int j = 0; j < NI_A; ++j) {
                        const uint32_t o = FULL ? oa[j] : off_a(j, lim);
                        dma16(ab + o, &st.alpha[j * RPI_A * DK]);
                        if constexpr (!ISO)
                            dma16(wb + o, &st.omega[j * RPI_A * DK]);
                    }
#pragma unroll
                    for (int j = 0; j < NI_K; ++j) {
                        const uint32_t o = FULL ? ok_[j] : off_k(j, lim);
                        dma16(kb + o, &st.k[j * RPI_K * DK]);
                        dma16(qb + o, &st.q[j * RPI_K * DK]);
                    }
                };
                if (lim == C - 1)
                    copy_stage(std::integral_constant<bool, true>{});
                else
                    copy_stage(std::integral_constant<bool, false>{});
                if (lane < C) {
                    const uint32_t o = (uint32_t)min(lane, lim) * tss;
                    const size_t sb = row_s(tb);
                    dma4(a.r + sb + o, sm.rr[X % NRING]);
                    if constexpr (ISO)
                        dma4(omg + sb + o, sm.wr[X % NRING]);
                }
            }
            if (vv) {
                IO* vdst = sm.v[XV % 3];
                const int lim = n_valid(XV) - 1;
                const IO* vb = vg + row_v(XV * C) + j0;  // uniform
                // LDS block p = 64 j + lane holds row p / 8 and data block
                // (p % 8) ^ (row & 7) of that row
                if (lim == C - 1) {
#pragma unroll
                    for (int j = 0; j < NI_V; ++j)
                        dma16(vb + ov[j], vdst + 64 * j * VE);
                } else {
#pragma unroll
                    for (int j = 0; j < NI_V; ++j)
                        dma16(vb + off_v(j, lim), vdst + 64 * j * VE);
                }
            }
            if (sv && vv)
                vm_wait<NSTG + NVI>();
            else if (sv)
                vm_wait<NSTG>();
            else if (vv)
                vm_wait<NVI>();
            else
                vm_wait<0>();
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
    hipError_t e = set_lds_limit_once(kern, smem);
    if (e != hipSuccess)
        return e;
    const int nblk = a.B * a.H * (a.dv / DVT);
    hipLaunchKernelGGL(kern, dim3(nblk), dim3(KDN_CHUNK_THREADS(DK, DVT, ISO)), smem, stream, a);
    return hipGetLastError();
}

hipError_t launch_chunk_fwd_f32(const FwdArgs& a, bool iso, hipStream_t stream)
{
    return iso ? launch_one<float, 64, 32, true>(a, stream)
               : launch_one<float, 64, 32, false>(a, stream);
}

}  // namespace kdn
