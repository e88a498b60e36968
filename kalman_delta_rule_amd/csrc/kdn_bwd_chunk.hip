// kdn_bwd_chunk.hip -- the memory part of the KDN backward in 16-token chunks
// on the matrix cores (fp32 16x16x4 products), gfx950.
//
// Given the gains kap_t (the gain recompute of kdn_bwd.hip), the memory
// recurrence of method part §2 / §4-§5 (Diagonal) and §7 (Isotropic, where
// kap_t = beta_t k_t),
//   S_t = D_t S_{t-1} + kap_t delta_t^T,  delta_t = v_t - (D_t S_{t-1})^T k_t,
//   o_t = S_t^T q_t,
// is, over a 16-token chunk with G_t = prod_{s <= t} alpha_s (per channel),
// Kb = k G, Qb = q G, Kt = kap / G (rows = tokens) and chunk-start state S0
// (the compact-WY form of Appendix D):
//   delta = T (V - Kb S0),  T = (I + tril(Kb Kt^T, -1))^-1,
//   O = Qb S0 + A delta,     A = tril(Qb Kt^T),
//   S_C = diag(G_15) (S0 + Kt^T delta).
// Its reverse, for incoming dO and dS_C, with E = diag(G_15) dS_C:
//   ddelta = Kt E + A^T dO,  dR = T^T ddelta,  dV = dR,
//   dS0 = E + Qb^T dO - Kb^T dR                      (carried to the chunk before),
//   dL = -tril(dR delta^T, -1),  dA = tril(dO delta^T),
//   dKb = dL Kt - dR S0^T,  dQb = dA Kt + dO S0^T,  dKt = dL^T Kb + dA^T Qb + delta E^T,
// and per token and channel dq = dQb G, dk = dKb G, kapbar = dKt / G,
//   dG_t = dKb k + dQb q - kapbar Kt  (+ rowsum(dS_C . X) at t = 15, X = S0 + Kt^T delta),
//   dalpha_s = sum_{t >= s} dG_t G_t / alpha_s = G_{s-1} W_s,  W_s = dG_s + alpha_{s+1} W_{s+1},
// the last form free of divisions by alpha.  Each chunk channel takes the decay
// reference of the forward (a power of two c, G' = G / c, S0' = c S0, floored
// alphas below 2^-224 of chunk decay; the chunk formulas hold with the primed
// quantities and dS0 = c dS0'); where the floor raises an alpha, its memory
// gradient is that of the raised value (zero).
//
// One workgroup of four waves per (batch, head, 64 value columns).  A forward
// pass over the chunks stores every chunk-start state (this block's columns;
// skipped when the caller's state-only forward walk has stored them), then
// the reverse pass takes the chunks last first.  The carried state (and then
// its adjoint) stays in LDS, each wave owning the rows of its key channels;
// every product is an fp32 16x16x4 matrix-core product with operands from
// LDS (or an accumulator tile as the B operand over its own row index), the
// products of a phase run as one software pipeline (mm_stream), and a
// chunk's inputs are loaded into registers one chunk ahead.  Everything per
// token and key channel is linear in
// dKb, dQb, dKt and the rowsum term, which sum over the value columns: each
// block writes its partials of those, and a second kernel (one thread per
// chunk and channel) sums the blocks and forms dq, kapbar and the memory's
// dk and dalpha, the last through the recurrence above.
#include "kdn_common.h"
#include "kdn_internal.h"
#include "kdn_ops.h"

#include <type_traits>

// lambdas that must not become calls (a call would pass the captures through
// scratch memory)
#define KDN_INLINE __attribute__((always_inline))

namespace kdn {
namespace cbwd {

constexpr int C = 16;       // tokens per chunk
constexpr int NC = 64;      // value columns per workgroup
constexpr int LC = NC + 4;  // row stride of the [.][NC] arrays
constexpr int LM = C + 1;   // row stride of the 16 x 16 matrices

template <int DK>
struct Smem {
    static constexpr int LK = DK + 4;
    float Kb[C][LK];   // k G'
    float Qb[C][LK];   // q G'
    float Kt[C][LK];   // kap / G'
    float S0[DK][LC];  // c S0, this block's columns
    float E[DK][LC];   // the carried state / adjoint (G'_15 dS_C while a reverse chunk uses it)
    float V[C][LC];
    float dO[C][LC];
    float D[C][LC];    // delta
    float mR[C][LC];   // a partial of Kb (c S0) while delta is formed, then -dR
    float Rp[2][C][LC];  // the other two partials of Kb (c S0)
    float Tm[C][LM];
    float Am[C][LM];
    float dLm[C][LM];  // also the powers of M while T is formed
    float dAm[C][LM];  // also half of Qb Kt^T while A is formed
    float Mp[2][C][LM];  // Kb Kt^T over each half of the key channels
    float cS[DK];      // c per channel
    float gL[DK];      // G'_15 per channel
    float rsum[DK];    // the last token's rowsum, its (c S0) part (the wave's own rows)
    // the chunk's per-channel inputs as loaded (rows of tokens), read back
    // one channel per thread for the factors
    float inA[C][DK];  // alpha
    float inP[C][DK];  // kappa (Diagonal); beta in inP[t][0] (Isotropic)
    uint4 inK[2 * C * DK * 4 / 16];  // k, then q, in the io type: [2][C][DK] (room for fp32)
};

// One chunk channel's decay reference and cumulative decays (the forward's
// rule, the same operations in both kernels here): g[0] = 1 / c, g[t + 1] =
// G'_t; alf[t] the decay the memory applies (floored where the reference
// floors), bit t of `raised` set where the floor raised alpha_t.  Tokens
// past a ragged end are al = 1.
struct ChanDecay {
    float g[C + 1];
    float alf[C];
    uint32_t raised;
    int m;
};
__device__ __forceinline__ void chan_decay(const float (&al)[C], ChanDecay& d)
{
    float P = 1.f;
#pragma unroll
    for (int t = 0; t < C; ++t)
        P *= al[t];
    DecayRef ref{false, 0};
    if (!decay_plain_ok(P))
        ref = decay_ref(al);
    d.m = ref.m;
    d.raised = 0;
    float G = __builtin_amdgcn_ldexpf(1.f, -ref.m);
    d.g[0] = G;
#pragma unroll
    for (int t = 0; t < C; ++t) {
        const float ad = decay_alpha(ref, al[t]);
        d.raised |= (ad != al[t] ? 1u : 0u) << t;
        d.alf[t] = ad;
        G *= ad;
        d.g[t + 1] = G;
    }
}

// acc[m][n] += sum_k A(m, k) B(k, n) over K (multiple of 4), operands in LDS:
// A(m, k) = A[m am + k ak], B(k, n) = B[k bk + n bn]; the 16x16x4 product
// takes A(lane & 15, k0 + (lane >> 4)) and B(k0 + (lane >> 4), lane & 15).
// Software-pipelined: the operands of step s + D are read before the
// product of step s is issued (scheduling barriers keep that order), so each
// product finds its operands landed; at most 2 D LDS reads are in flight,
// within the 4-bit count of outstanding LDS operations.
template <int K>
__device__ __forceinline__ void mmk(f32x4& acc, const float* A, int am, int ak, const float* B,
                                    int bk, int bn, int lane)
{
    const int i = lane & 15, g = lane >> 4;
    constexpr int NS = K / 4, D = NS < 6 ? NS : 6;
    float a[NS], b[NS];
#pragma unroll
    for (int s = 0; s < D; ++s) {
        a[s] = A[i * am + (4 * s + g) * ak];
        b[s] = B[(4 * s + g) * bk + i * bn];
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if (s + D < NS) {
            a[s + D] = A[i * am + (4 * (s + D) + g) * ak];
            b[s + D] = B[(4 * (s + D) + g) * bk + i * bn];
        }
        __builtin_amdgcn_sched_barrier(0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
    }
}

// acc += A X with X a 16 x 16 accumulator (lane holds X[4 (lane >> 4) + r][lane & 15]):
// step r contracts over k = 4 g + r, g = 0..3, which is exactly the lane's
// own X[r] as the B operand.
__device__ __forceinline__ void mm_acc(f32x4& acc, const float* A, int am, int ak, const f32x4& X,
                                       int lane)
{
    const int i = lane & 15, g = lane >> 4;
    float a[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        a[r] = A[i * am + (4 * g + r) * ak];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], X[r], acc, 0, 0, 0);
}

// Several products as one software pipeline of NS fp32 16x16x4 steps: step
// s reads this lane's operands through op(s, a, b) (A(lane & 15, k) and
// B(k, lane & 15) for the step's k = 4 s' + (lane >> 4)) and accumulates into
// acc[slot(s)]; the operands of step s + D are read before the product of
// step s is issued, across the products' boundaries (a product of its own
// would drain the pipeline and wait for its first operands).  s is a
// constant in every call, so op and slot fold to plain LDS reads and a
// fixed register tile.
// An op may also read a factor c for the A value, which the step applies
// (scale(s) true) only when it issues the product, once the reads are in.
template <int NS, int NA, typename Op, typename Slot, typename Scale>
__device__ __forceinline__ void mm_stream(f32x4 (&acc)[NA], Op op, Slot slot, Scale scale)
{
    constexpr int D = NS < 6 ? NS : 6;
    float a[NS], b[NS], c[NS];
#pragma unroll
    for (int s = 0; s < D; ++s)
        op(s, a[s], b[s], c[s]);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if (s + D < NS)
            op(s + D, a[s + D], b[s + D], c[s + D]);
        __builtin_amdgcn_sched_barrier(0);
        const float av = scale(s) ? a[s] * c[s] : a[s];
        acc[slot(s)] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b[s], acc[slot(s)], 0, 0, 0);
    }
}
template <int NS, int NA, typename Op, typename Slot>
__device__ __forceinline__ void mm_stream(f32x4 (&acc)[NA], Op op, Slot slot)
{
    mm_stream<NS>(acc, [&](int s, float& a, float& b, float&) { op(s, a, b); }, slot,
                  [](int) { return false; });
}

// an accumulator tile to / from LDS: element (4 g + r, i) at p[(4 g + r) ld + i]
__device__ __forceinline__ void tile_store(float* p, int ld, const f32x4& x, int lane)
{
    const int i = lane & 15, g = lane >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        p[(4 * g + r) * ld + i] = x[r];
}
__device__ __forceinline__ f32x4 tile_load(const float* p, int ld, int lane)
{
    const int i = lane & 15, g = lane >> 4;
    f32x4 x;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        x[r] = p[(4 * g + r) * ld + i];
    return x;
}

// Sum over the 16 lanes of a row (lanes 16 g .. 16 g + 15), in every lane of
// it, by DPP exchanges in the vector ALU: lane l ^ 8 and l ^ 4 through a row
// shift one way for the lanes whose bit is clear and the other way for the
// rest (chosen by the bank mask: banks are the four 4-lane groups of a row),
// then the quad permutes [2,3,0,1] and [1,0,3,2].
template <int CTRL, int BANK>
__device__ __forceinline__ float dpp_sel(float old, float src)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                 __builtin_bit_cast(int, src),
                                                                 CTRL, 0xF, BANK, false));
}
__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp_sel<0x118, 0xC>(dpp_sel<0x108, 0x3>(x, x), x);  // + lane ^ 8
    x += dpp_sel<0x114, 0xA>(dpp_sel<0x104, 0x5>(x, x), x);  // + lane ^ 4
    x += dpp_sel<0x4E, 0xF>(x, x);                           // + lane ^ 2
    x += dpp_sel<0xB1, 0xF>(x, x);                           // + lane ^ 1
    return x;
}

// A barrier that orders LDS only: global loads and stores stay in flight
// (a full __syncthreads would wait for every store of the chunk).  The
// kernel reads no global memory that another wave wrote, except the
// chunk-start states, which a full barrier between the passes orders.
__device__ __forceinline__ void barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A row-major [token][channel] array of a chunk in 16-byte pieces, NP of
// them, dealt to the 256 threads: thread (w, lane) takes pieces
// 64 w + 256 j + lane.  rows_load reads them from global memory into
// registers (row(e) gives the global element index of element e of the
// chunk), rows_store writes them to LDS in the same row-major order.  The
// loads are unconditional, so that the pieces stay in registers.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <int NP, int NT, int NR, typename Row>
__device__ __forceinline__ void rows_load(u32x4 (&dst)[NR], const void* src, int esz, int w,
                                          int lane, Row row)
{
    const int per = 16 / esz;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        // a wave past the last piece loads the last piece (and stores nothing)
        const int p = min(64 * w + NT * j + lane, NP - 1);
        dst[j] = *reinterpret_cast<const u32x4*>((const char*)src + row(p * per) * esz);
    }
}
template <int NP, int NT, int NR>
__device__ __forceinline__ void rows_store(void* dst, const u32x4 (&src)[NR], int w, int lane)
{
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        const int p0 = 64 * w + NT * j;
        if (p0 < NP)
            reinterpret_cast<u32x4*>(dst)[p0 + lane] = src[j];
    }
}

// ADJ: the adjoint only.  No forward pass and no per-token output: the
// reverse pass carries dS from gS_T (zero when null) back through the chunks
// (E, dO, the factors, T and A only) and writes the adjoint at the start into
// gS0.  The sequence split of the backward uses it for each segment's adjoint
// from its own outputs.
template <typename IO, bool ISO, int DK, bool ADJ, int NW>
__global__ __launch_bounds__(64 * NW, 1) void kdn_bwd_chunk_kernel(BwdArgs args)
{
    const BwdArgs a = args;
    using SM = Smem<DK>;
    static_assert(sizeof(SM) <= 160 * 1024, "LDS budget");
    constexpr int LK = SM::LK;
    constexpr int NT = 64 * NW;               // threads
    constexpr int CT = DK / (16 * NW);        // 16-channel tiles per wave
    static_assert(CT >= 1, "a wave holds at least one 16-row tile of the state");
    constexpr int NCK = DK * NC / (4 * NT);   // chunk-start state pieces (4 floats) per thread
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SM& sm = *reinterpret_cast<SM*>(smem_raw);
    // distances in floats between arrays of equal shape, for choosing one by
    // an offset (a choice between two LDS pointers compiles poorly)
    constexpr int OFF_KB_QB = (int)((offsetof(SM, Kb) - offsetof(SM, Qb)) / sizeof(float));
    constexpr int OFF_MR_DO = (int)((offsetof(SM, mR) - offsetof(SM, dO)) / sizeof(float));
    constexpr int OFF_RP0_MR = (int)((offsetof(SM, Rp) - offsetof(SM, mR)) / sizeof(float));
    constexpr int OFF_RP1_MR = OFF_RP0_MR + C * LC;
    constexpr int OFF_DAM_AM = (int)((offsetof(SM, dAm) - offsetof(SM, Am)) / sizeof(float));

    const int blk = blockIdx.x, nblk = gridDim.x, bh = blockIdx.y;
    const int H = a.H, T = a.T, dv = a.dv;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int i16 = lane & 15, g4 = lane >> 4;
    const int col0 = blk * NC;       // first value column of this block
    const int chw = w * (DK / NW);   // first key channel of this wave's state rows
    const int nch = (T + C - 1) / C;
    const size_t ntok = (size_t)a.B * T * H;
    const size_t ks = (size_t)nblk * ntok * DK;  // stride between the partial arrays
    auto tok_of = [&](int t) { return ((size_t)b * T + t) * H + h; };
    float* const ck_wg = a.ckpt + ((size_t)bh * nblk + blk) * (size_t)nch * (DK * NC);
    const IO* kg = reinterpret_cast<const IO*>(a.k);
    const IO* qg = reinterpret_cast<const IO*>(a.q);
    const IO* vg = reinterpret_cast<const IO*>(a.v);
    const IO* og = reinterpret_cast<const IO*>(a.go);
    IO* dvg = reinterpret_cast<IO*>(a.gv);
    // the factors: 256 / DK threads per key channel (one per wave group of
    // DK / 64 waves), each its channel's decays and a share of the tokens
    constexpr int FP = NT / DK, FT = C / FP;  // threads per channel, tokens per thread
    const int ch = (w % (DK / 64)) * 64 + lane, fpart = w / (DK / 64);  // fpart wave-uniform
    // V and dO: the first 256 threads, 4 elements each of a [C][NC] block
    const bool vth = tid < C * NC / 4;
    const int et = (tid * 4) / NC, ec = (tid * 4) % NC;

    // The chunk's inputs, loaded one chunk ahead into registers (16 bytes
    // per lane and piece of a row-major [token][channel] array, each wave a
    // share of the pieces), as soon as the factors of the chunk before have
    // read the staging arrays, and written to LDS at the start of their
    // chunk.  (A direct global -> LDS copy would make every later LDS access
    // of the wave wait for it: the compiler cannot tell the copy's LDS
    // destination from the arrays the chunk works on.)
    constexpr int NPA = C * DK * 4 / 16, NPK = C * DK * (int)sizeof(IO) / 16;  // pieces per array
    constexpr int RA = (NPA + NT - 1) / NT, RK = (NPK + NT - 1) / NT;          // per lane
    u32x4 ra[RA], rp[RA], rk[RK], rq[RK];
    // four consecutive io elements of V and dO, kept packed until they land
    // (unpacking at the load would wait for it)
    using Raw4 = typename std::conditional<sizeof(IO) == 2, u32x2, u32x4>::type;
    auto raw_f32 = [](const Raw4& x, int j) {
        if constexpr (sizeof(IO) == 2)
            return __uint_as_float((j & 1) ? (x[j >> 1] & 0xffff0000u) : (x[j >> 1] << 16));
        else
            return __uint_as_float(x[j]);
    };
    Raw4 vraw, oraw;
    float braw = 0.f;
    bool vok = false;
    auto issue = [&](int c, bool rev) {
        const int t0 = c * C, len = min(C, T - t0);
        auto row = [&](int e) { return tok_of(t0 + min(e / DK, len - 1)) * DK + e % DK; };
        rows_load<NPA, NT>(ra, a.alpha, 4, w, lane, row);
        if constexpr (!ISO)
            rows_load<NPA, NT>(rp, a.kap, 4, w, lane, row);
        static_assert(2 * C * DK * sizeof(IO) <= sizeof(sm.inK), "staging size");
        rows_load<NPK, NT>(rk, kg, (int)sizeof(IO), w, lane, row);
        if (rev)
            rows_load<NPK, NT>(rq, qg, (int)sizeof(IO), w, lane, row);
        if constexpr (ISO)
            if (tid < C)
                braw = a.gsc[tok_of(t0 + min(tid, len - 1)) * 4];
        vok = et < len;
        // (threads past the block load a clamped in-range row and store nothing)
        const size_t r = tok_of(t0 + min(et, len - 1)) * dv + col0 + ec;
        if (!ADJ)
            vraw = *reinterpret_cast<const Raw4*>(vg + r);
        if (rev)
            oraw = *reinterpret_cast<const Raw4*>(og + r);
    };
    // the issued inputs into LDS (V and dO as fp32); the caller's barrier follows
    auto land = [&](bool rev) {
        rows_store<NPA, NT>(&sm.inA[0][0], ra, w, lane);
        if constexpr (!ISO)
            rows_store<NPA, NT>(&sm.inP[0][0], rp, w, lane);
        rows_store<NPK, NT>(&sm.inK[0], rk, w, lane);
        if (rev)
            rows_store<NPK, NT>(reinterpret_cast<char*>(&sm.inK[0]) + C * DK * sizeof(IO), rq, w, lane);
        if (vth) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (!ADJ)
                    sm.V[et][ec + j] = vok ? raw_f32(vraw, j) : 0.f;
                if (rev)
                    sm.dO[et][ec + j] = vok ? raw_f32(oraw, j) : 0.f;
            }
        }
        if constexpr (ISO)
            if (tid < C)
                sm.inP[tid][0] = braw;
    };
    auto factors_part = [&](auto part_tag, int c, bool rev) KDN_INLINE {
        constexpr int tb = decltype(part_tag)::value * FT;  // this thread's first token
        const int t0 = c * C, len = min(C, T - t0);
        const IO* sk = reinterpret_cast<const IO*>(&sm.inK[0]);
        float al[C], kk[FT], qq[FT], kap[FT];
#pragma unroll
        for (int t = 0; t < C; ++t)
            al[t] = t < len ? sm.inA[t][ch] : 1.f;
#pragma unroll
        for (int u = 0; u < FT; ++u) {
            const int t = tb + u;
            const bool ok = t < len;
            const float kv = to_f32(sk[t * DK + ch]);
            const float pv = ISO ? sm.inP[t][0] : sm.inP[t][ch];
            kk[u] = ok ? kv : 0.f;
            qq[u] = ok && rev ? to_f32(sk[C * DK + t * DK + ch]) : 0.f;
            kap[u] = ok ? (ISO ? pv * kv : pv) : 0.f;
        }
        ChanDecay d;
        chan_decay(al, d);  // every thread of the channel: the same operations
#pragma unroll
        for (int u = 0; u < FT; ++u) {
            const float G = d.g[tb + u + 1];
            sm.Kb[tb + u][ch] = kk[u] * G;
            sm.Qb[tb + u][ch] = qq[u] * G;
            sm.Kt[tb + u][ch] = kap[u] * rcp(G);
        }
        if (tb == 0) {
            sm.cS[ch] = __builtin_amdgcn_ldexpf(1.f, d.m);
            sm.gL[ch] = d.g[C];
        }
    };
    auto factors = [&](int c, bool rev) KDN_INLINE {
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2 % FP>;
        using I3 = std::integral_constant<int, 3 % FP>;
        if (fpart == 0)
            factors_part(I0{}, c, rev);
        else if (fpart == 1)
            factors_part(I1{}, c, rev);
        else if (fpart == 2)
            factors_part(I2{}, c, rev);
        else
            factors_part(I3{}, c, rev);
    };
    // M = Kb Kt^T, by waves 2 and 3 over half of the key channels each
    auto form_M_parts = [&]() {
        if (w == 2 || w == 3) {
            const int k0 = (w - 2) * (DK / 2);
            f32x4 m = zero4();
            mmk<DK / 2>(m, &sm.Kb[0][k0], LK, 1, &sm.Kt[0][k0], 1, LK, lane);
            tile_store(&sm.Mp[w - 2][0][0], LM, m, lane);
        }
    };
    // Qb Kt^T (reverse pass), by waves 0 and 1 over half of the key
    // channels each, into Am and dAm; wave 0 sums them into A after the barrier
    auto form_A_parts = [&]() {
        if (w < 2) {
            const int k0 = w * (DK / 2);
            f32x4 m = zero4();
            mmk<DK / 2>(m, &sm.Qb[0][k0], LK, 1, &sm.Kt[0][k0], 1, LK, lane);
            tile_store(&sm.Am[0][0] + (w == 0 ? 0 : OFF_DAM_AM), LM, m, lane);
        }
    };
    // After form_M_parts and a barrier: wave 0 forms T = (I + M)^-1 with
    // M = tril(Kb Kt^T, -1) nilpotent, (I + M)^-1 = (I - M)(I + M^2)(I + M^4)
    // (I + M^8), each factor a 16x16 product on the matrix cores (the powers of
    // M through LDS), and in the reverse pass A = tril(Qb Kt^T) from its two
    // halves; meanwhile waves 1-3 form the products Kb (c S0) over a third of
    // the key channels each, for all four column tiles (into mR, Rp[0], Rp[1]).
    constexpr int KQ = ((DK / 4 + 2) / 3) * 4;  // key channels of waves 1 and 2 (wave 3: the rest)
    auto form_T_and_R = [&](bool rev) {
        if (w == 0) {
            if (rev) {
                f32x4 m = tile_load(&sm.Am[0][0], LM, lane) + tile_load(&sm.dAm[0][0], LM, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    m[r] = 4 * g4 + r >= i16 ? m[r] : 0.f;
                tile_store(&sm.Am[0][0], LM, m, lane);
            }
            f32x4 m = tile_load(&sm.Mp[0][0][0], LM, lane) + tile_load(&sm.Mp[1][0][0], LM, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                m[r] = 4 * g4 + r > i16 ? m[r] : 0.f;
            f32x4 tt;  // I - M
#pragma unroll
            for (int r = 0; r < 4; ++r)
                tt[r] = (4 * g4 + r == i16 ? 1.f : 0.f) - m[r];
            f32x4 pw = m;  // M^(2^j)
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                tile_store(&sm.dLm[0][0], LM, pw, lane);
                wave_lds_sync();
                f32x4 sq = zero4();
                mm_acc(sq, &sm.dLm[0][0], LM, 1, pw, lane);  // M^(2^(j+1))
                wave_lds_sync();
                tile_store(&sm.dLm[0][0], LM, sq, lane);
                wave_lds_sync();
                const f32x4 tp = tt;
                mm_acc(tt, &sm.dLm[0][0], LM, 1, tp, lane);  // (I + M^(2^(j+1))) tt
                wave_lds_sync();
                pw = sq;
            }
            tile_store(&sm.Tm[0][0], LM, tt, lane);
        } else if (!ADJ && w < 4) {
            auto part = [&](auto kc, int k0, float* dst) {
                constexpr int K = decltype(kc)::value;
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    f32x4 p = zero4();
                    mmk<K>(p, &sm.Kb[0][k0], LK, 1, &sm.S0[k0][16 * n], LC, 1, lane);
                    tile_store(dst + 16 * n, LC, p, lane);
                }
            };
            if (w == 1)
                part(std::integral_constant<int, KQ>{}, 0, &sm.mR[0][0]);
            else if (w == 2)
                part(std::integral_constant<int, KQ>{}, KQ, &sm.mR[0][0] + OFF_RP0_MR);
            else
                part(std::integral_constant<int, DK - 2 * KQ>{}, 2 * KQ, &sm.mR[0][0] + OFF_RP1_MR);
        }
    };
    // delta = T (V - Kb (c S0)) for column tile w, into LDS
    auto form_delta = [&]() {
        if (w >= 4)
            return;
        f32x4 d = zero4();
        float ta[4], rb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int k = 4 * s + g4, col = 16 * w + i16;
            ta[s] = sm.Tm[i16][k];
            rb[s] = sm.V[k][col] - ((sm.mR[k][col] + sm.Rp[0][k][col]) + sm.Rp[1][k][col]);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
            d = __builtin_amdgcn_mfma_f32_16x16x4f32(ta[s], rb[s], d, 0, 0, 0);
        tile_store(&sm.D[0][16 * w], LC, d, lane);
    };
    // the state rows this wave holds: tile (j, n) = channels chw + 16 j + 4 g + r, columns 16 n + i
    auto state_rows = [&](int j) { return chw + 16 * j; };

    // The carried state (forward pass) and its adjoint (reverse pass) live in
    // the E array, unscaled, each wave owning the rows of its channels.
    auto state_init = [&](const float* src) {
#pragma unroll
        for (int j = 0; j < CT; ++j)
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                f32x4 x;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = state_rows(j) + 4 * g4 + r;
                    x[r] = src ? src[((size_t)bh * DK + row) * dv + col0 + 16 * n + i16] : 0.f;
                }
                tile_store(&sm.E[state_rows(j)][16 * n], LC, x, lane);
            }
    };

    // ---------------- forward pass: every chunk-start state ----------------
    // (not when the caller's forward walk has stored the chunk-start states)
    if (!ADJ && !a.ckpt_given) {
        state_init(a.S0);
        if (nch > 0)
            issue(0, false);
        for (int c = 0; c < nch; ++c) {
            land(false);
            barrier();  // inputs staged, V
            factors(c, false);
            barrier();  // factors, cS; the staging arrays are free
            if (c + 1 < nch)
                issue(c + 1, false);
            form_M_parts();
            // c S0 into LDS; the chunk-start state to the workspace (rows in
            // fours: the lane's four rows of a tile are one 16-byte store)
            float* ckc = ck_wg + (size_t)c * (DK * NC);
#pragma unroll
            for (int j = 0; j < CT; ++j)
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    f32x4 x = tile_load(&sm.E[state_rows(j)][16 * n], LC, lane);
                    const int rq = (state_rows(j) + 4 * g4) / 4;
                    *reinterpret_cast<f32x4*>(ckc + (rq * NC + 16 * n + i16) * 4) = x;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        x[r] *= sm.cS[state_rows(j) + 4 * g4 + r];
                    tile_store(&sm.S0[state_rows(j)][16 * n], LC, x, lane);
                }
            barrier();  // M parts, c S0
            form_T_and_R(false);
            barrier();  // T, R
            form_delta();
            barrier();  // delta
            f32x4 xs[4 * CT];
#pragma unroll
            for (int q = 0; q < 4 * CT; ++q)
                xs[q] = tile_load(&sm.S0[state_rows(q / 4)][16 * (q % 4)], LC, lane);
            // S_C = G'_15 (c S0 + Kt^T delta), the state tiles q = (j, n) as one stream
            mm_stream<4 * CT * (C / 4)>(
                xs,
                [&](int st, float& av, float& bv) {
                    const int q = st / 4, k = 4 * (st % 4) + g4;
                    av = sm.Kt[k][state_rows(q / 4) + i16];
                    bv = sm.D[k][16 * (q % 4) + i16];
                },
                [&](int st) { return st / 4; });
#pragma unroll
            for (int q = 0; q < 4 * CT; ++q) {
                f32x4 x = xs[q];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    x[r] *= sm.gL[state_rows(q / 4) + 4 * g4 + r];
                tile_store(&sm.E[state_rows(q / 4)][16 * (q % 4)], LC, x, lane);
            }
            barrier();  // readers of this chunk's factors done
        }

        // every chunk-start state stored is visible to the whole workgroup
        __syncthreads();
    }

    // ---------------- reverse pass ----------------
    state_init(a.gS_T);
    // this block's chunk-start states, loaded one chunk ahead with the inputs
    // Thread (tid / 16, tid % 16) takes the four columns 4 (tid % 16) .. + 3
    // of row quads tid / 16 + (NT / 16) jq: four 16-byte pieces per quad, which it
    // writes to LDS as four 16-byte rows (a 4 x 4 transpose in registers).
    static_assert(NCK % 4 == 0 && NC == 64, "chunk-start state pieces");
    f32x4 ck[NCK];
    const int ck_cg = tid % 16, ck_rq = tid / 16;
    auto issue_rev = [&](int c) {
        if constexpr (!ADJ) {
            const f32x4* src = reinterpret_cast<const f32x4*>(ck_wg + (size_t)c * (DK * NC));
#pragma unroll
            for (int jq = 0; jq < NCK / 4; ++jq)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    ck[4 * jq + u] = src[(ck_rq + (NT / 16) * jq) * NC + 4 * ck_cg + u];
        }
        issue(c, true);
    };
    if (nch > 0)
        issue_rev(nch - 1);
    for (int c = nch - 1; c >= 0; --c) {
        const int t0 = c * C, len = min(C, T - t0);
        land(true);
        barrier();  // inputs staged, V, dO
        factors(c, true);
        barrier();  // factors, cS, gL; the staging arrays are free
        if constexpr (!ADJ) {
#pragma unroll
            for (int jq = 0; jq < NCK / 4; ++jq)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 4 * (ck_rq + (NT / 16) * jq) + r;
                    const f32x4 v{ck[4 * jq][r], ck[4 * jq + 1][r], ck[4 * jq + 2][r], ck[4 * jq + 3][r]};
                    *reinterpret_cast<f32x4*>(&sm.S0[row][4 * ck_cg]) = v * sm.cS[row];
                }
        }
        if (c > 0)
            issue_rev(c - 1);
        // E holds dS_C; its uses below apply E = G'_15 dS_C themselves
        // (the operand Kt G'_15, the delta E^T result, the dS0 update)
        form_M_parts();
        form_A_parts();
        barrier();  // c S0, M parts, A parts, E
        form_T_and_R(true);
        barrier();  // T, R
        if constexpr (!ADJ) {
            form_delta();
            barrier();  // delta
        }
        {
            // ddelta = Kt E + A^T dO for column tile w, as one stream.  The
            // last token's dG also takes rowsum(dS_C . X'), X' = c S0 + Kt^T
            // delta, over this block's columns; by linearity it is
            // rowsum(dS_C . c S0) (here, into rsum) plus sum_t Kt[t] (delta
            // dS_C^T)[t], which the next phase's delta E^T product gives.
            if constexpr (!ADJ) {
#pragma unroll
                for (int j = 0; j < CT; ++j) {
                    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int n = 0; n < 4; ++n) {
                        const f32x4 e = tile_load(&sm.E[state_rows(j)][16 * n], LC, lane);
                        const f32x4 x = tile_load(&sm.S0[state_rows(j)][16 * n], LC, lane);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            rs[r] = fmaf(e[r], x[r], rs[r]);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float sum = row16_sum(rs[r]);
                        if (i16 == 0)
                            sm.rsum[state_rows(j) + 4 * g4 + r] = sum;
                    }
                }
            }
            if (w < 4) {  // ddelta and dR: one column tile per wave of the first four
                f32x4 acc[1];
                acc[0] = zero4();
                // T^T for dR = T^T ddelta, read ahead: A(m, k) = T(k, m), k = 4 g + r
                float tA[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    tA[r] = sm.Tm[4 * g4 + r][i16];
                mm_stream<DK / 4 + C / 4>(
                    acc,
                    [&](int st, float& av, float& bv, float& cv) {
                        if (st < DK / 4) {  // Kt E = (Kt G'_15) dS_C
                            const int k = 4 * st + g4;
                            av = sm.Kt[i16][k];
                            cv = sm.gL[k];
                            bv = sm.E[k][16 * w + i16];
                        } else {  // A^T dO
                            const int k = 4 * (st - DK / 4) + g4;
                            av = sm.Am[k][i16];
                            bv = sm.dO[k][16 * w + i16];
                        }
                    },
                    [&](int) { return 0; }, [&](int st) { return st < DK / 4; });
                // dR = T^T ddelta, ddelta's accumulator as the B operand
                f32x4 dR = zero4();
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dR = __builtin_amdgcn_mfma_f32_16x16x4f32(tA[r], acc[0][r], dR, 0, 0, 0);
                tile_store(&sm.mR[0][16 * w], LC, -dR, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 4 * g4 + r;
                    if (!ADJ && t < len)
                        dvg[tok_of(t0 + t) * dv + col0 + 16 * w + i16] = from_f32<IO>(dR[r]);
                }
            }
        }
        barrier();  // -dR; every wave's reads of all E rows done
        // One stream: delta E^T for this wave's channels (slots 0 .. CT - 1,
        // from their E rows before the update; not in the adjoint-only mode),
        // dS0' = E + Qb^T dO + Kb^T (-dR) for its state tiles (slots CT ..
        // 5 CT - 1), and on waves 0 and 1 the strictly lower -dR delta^T (dL)
        // and the lower dO delta^T (dA) (slot 5 CT).
        constexpr int NG = ADJ ? 0 : CT * (NC / 4);  // delta E^T steps
        constexpr int NU = 4 * CT * (2 * C / 4);     // state-adjoint steps
        f32x4 g6[5 * CT + 1];
#pragma unroll
        for (int j = 0; j < CT; ++j)
            g6[j] = zero4();
        // dS_C tiles, read now and added as E = G'_15 dS_C after the stream
        f32x4 es[4 * CT];
#pragma unroll
        for (int q = 0; q < 4 * CT; ++q) {
            es[q] = tile_load(&sm.E[state_rows(q / 4)][16 * (q % 4)], LC, lane);
            g6[CT + q] = zero4();
        }
        g6[5 * CT] = zero4();
        auto op6 = [&](int st, float& av, float& bv) {
            if (st < NG) {  // delta E^T, tile j
                const int j = st / (NC / 4), k = 4 * (st % (NC / 4)) + g4;
                av = sm.D[i16][k];
                bv = sm.E[state_rows(j) + i16][k];
            } else if (st < NG + NU) {  // Qb^T dO, then Kb^T (-dR), tile q = (j, n)
                const int u = st - NG, q = u / 8, h = u % 8, k = 4 * (h % 4) + g4;
                const int row = state_rows(q / 4) + i16, col = 16 * (q % 4) + i16;
                // Qb / Kb and dO / -dR by an offset from one array (same shapes)
                const float* qk = &sm.Qb[0][0] + (h < 4 ? 0 : OFF_KB_QB);
                const float* om = &sm.dO[0][0] + (h < 4 ? 0 : OFF_MR_DO);
                av = qk[k * LK + row];
                bv = om[k * LC + col];
            } else {  // (-dR or dO) delta^T
                const int k = 4 * (st - NG - NU) + g4;
                const float* om = &sm.dO[0][0] + (w == 0 ? OFF_MR_DO : 0);
                av = om[i16 * LC + k];
                bv = sm.D[i16][k];
            }
        };
        auto slot6 = [&](int st) {
            return st < NG ? st / (NC / 4) : st < NG + NU ? CT + (st - NG) / 8 : 5 * CT;
        };
        if (!ADJ && w < 2)
            mm_stream<NG + NU + NC / 4>(g6, op6, slot6);
        else
            mm_stream<NG + NU>(g6, op6, slot6);
#pragma unroll
        for (int q = 0; q < 4 * CT; ++q) {
            f32x4 x;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = state_rows(q / 4) + 4 * g4 + r;
                x[r] = sm.cS[row] * fmaf(sm.gL[row], es[q][r], g6[CT + q][r]);
            }
            tile_store(&sm.E[state_rows(q / 4)][16 * (q % 4)], LC, x, lane);
        }
        if constexpr (ADJ) {
            barrier();  // the next chunk's inputs overwrite the LDS arrays
            continue;
        }
        if (w < 2) {
            const f32x4 m = g6[5 * CT];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g4 + r;
                if (w == 0)
                    sm.dLm[t][i16] = t > i16 ? m[r] : 0.f;
                else
                    sm.dAm[t][i16] = t >= i16 ? m[r] : 0.f;
            }
        }
        barrier();  // dL, dA
        // One stream: the rest of the row-space products for this wave's
        // channels, per 16-channel tile j: dKb' = -dR (c S0)^T + dL Kt (slot
        // 3 j), dQb' = dO (c S0)^T + dA Kt (slot 3 j + 1), dKt' += dL^T Kb +
        // dA^T Qb (slot 3 j + 2); then their partials (arrays 0, 1, 2)
        // the last token's rowsum: its (c S0) part plus sum_t Kt[t][k] (delta
        // dS_C^T)[t][k] (the sum over t: four rows in the lane, then the
        // four lane groups), for channel k = this wave's row of lane i16
#pragma unroll
        for (int j = 0; j < CT; ++j) {
            float v = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                v = fmaf(sm.Kt[4 * g4 + r][state_rows(j) + i16], g6[j][r], v);
            // lanes l and l ^ 32, then l and l ^ 16: with both operands v,
            // each swap leaves the lane's and its partner's value in the pair
            const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                              false, false);
            v = __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
            const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                              false, false);
            v = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
            if (g4 == 0) {
                const int row = state_rows(j) + i16;
                a.part[3 * ks + ((size_t)blk * ntok + tok_of(t0 + len - 1)) * DK + row] =
                    sm.rsum[row] + v;
            }
        }
        f32x4 g7[3 * CT];
#pragma unroll
        for (int j = 0; j < CT; ++j) {
            g7[3 * j] = zero4();
            g7[3 * j + 1] = zero4();
            // delta E^T = (delta dS_C^T) G'_15, by the channel of the lane's column
            g7[3 * j + 2] = g6[j] * sm.gL[state_rows(j) + i16];
        }
        constexpr int PJ = 2 * (NC / 4) + 4 * (C / 4);  // steps per tile
        mm_stream<CT * PJ>(
            g7,
            [&](int st, float& av, float& bv) {
                const int c0 = state_rows(st / PJ), u = st % PJ;
                if (u < NC / 4) {  // -dR (c S0)^T
                    const int k = 4 * u + g4;
                    av = sm.mR[i16][k];
                    bv = sm.S0[c0 + i16][k];
                } else if (u < NC / 4 + C / 4) {  // dL Kt
                    const int k = 4 * (u - NC / 4) + g4;
                    av = sm.dLm[i16][k];
                    bv = sm.Kt[k][c0 + i16];
                } else if (u < 2 * (NC / 4) + C / 4) {  // dO (c S0)^T
                    const int k = 4 * (u - NC / 4 - C / 4) + g4;
                    av = sm.dO[i16][k];
                    bv = sm.S0[c0 + i16][k];
                } else if (u < 2 * (NC / 4) + 2 * (C / 4)) {  // dA Kt
                    const int k = 4 * (u - 2 * (NC / 4) - C / 4) + g4;
                    av = sm.dAm[i16][k];
                    bv = sm.Kt[k][c0 + i16];
                } else if (u < 2 * (NC / 4) + 3 * (C / 4)) {  // dL^T Kb
                    const int k = 4 * (u - 2 * (NC / 4) - 2 * (C / 4)) + g4;
                    av = sm.dLm[k][i16];
                    bv = sm.Kb[k][c0 + i16];
                } else {  // dA^T Qb
                    const int k = 4 * (u - 2 * (NC / 4) - 3 * (C / 4)) + g4;
                    av = sm.dAm[k][i16];
                    bv = sm.Qb[k][c0 + i16];
                }
            },
            [&](int st) {
                const int j = st / PJ, u = st % PJ;
                return 3 * j + (u < NC / 4 + C / 4 ? 0 : u < 2 * (NC / 4) + 2 * (C / 4) ? 1 : 2);
            });
#pragma unroll
        for (int j = 0; j < CT; ++j) {
            const int c0 = state_rows(j);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g4 + r;
                if (t < len) {
                    float* pp = a.part + ((size_t)blk * ntok + tok_of(t0 + t)) * DK + c0 + i16;
                    pp[0] = g7[3 * j][r];
                    pp[ks] = g7[3 * j + 1][r];
                    pp[2 * ks] = g7[3 * j + 2][r];
                }
            }
        }
        barrier();  // the next chunk's inputs overwrite the LDS arrays
    }
    if (a.gS0) {
#pragma unroll
        for (int j = 0; j < CT; ++j)
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const f32x4 x = tile_load(&sm.E[state_rows(j)][16 * n], LC, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = state_rows(j) + 4 * g4 + r;
                    a.gS0[((size_t)bh * DK + row) * dv + col0 + 16 * n + i16] = x[r];
                }
            }
    }
}

// Sum of the column blocks' partials and the per-channel finishing, one
// thread per (chunk, key channel): with G' recomputed from alpha by the rule
// the memory kernel used, and the summed dKb', dQb', dKt' and rowsum term R,
//   dq = dQb' G',  dk (memory) = dKb' G',  kapbar = dKt' / G',
//   dG'_t = dKb' k + dQb' q - kapbar Kt'  (+ R at the chunk's last token),
//   dalpha_s = G'_{s-1} W_s,  W_s = dG'_s + alpha_{s+1} W_{s+1}  (zero where the floor raised alpha).
// dq is written in the io type; kapbar, dk and dalpha go to block 0 of
// arrays 1, 2, 3 (where the gain backward reads them), after this thread
// has read every partial of its own tokens there.
template <typename IO, bool ISO, int DK>
__global__ __launch_bounds__(DK) void kdn_bwd_chunk_finish_kernel(BwdArgs args, int nblk)
{
    const BwdArgs a = args;
    const int nch = (a.T + C - 1) / C;
    const int bh = blockIdx.x / nch, c = blockIdx.x % nch, ch = threadIdx.x;
    const int b = bh / a.H, h = bh % a.H;
    const int t0 = c * C, len = min(C, a.T - t0);
    const size_t ntok = (size_t)a.B * a.T * a.H, ks = (size_t)nblk * ntok * DK;
    auto tok_of = [&](int t) { return ((size_t)b * a.T + t0 + t) * a.H + h; };
    const IO* kg = reinterpret_cast<const IO*>(a.k);
    const IO* qg = reinterpret_cast<const IO*>(a.q);
    float al[C], kk[C], qq[C], kap[C];
#pragma unroll
    for (int t = 0; t < C; ++t) {
        const size_t e = tok_of(min(t, len - 1)) * DK + ch;
        al[t] = a.alpha[e];
        kk[t] = to_f32(kg[e]);
        qq[t] = to_f32(qg[e]);
        kap[t] = ISO ? a.gsc[tok_of(min(t, len - 1)) * 4] : a.kap[e];
    }
#pragma unroll
    for (int t = 0; t < C; ++t) {
        const bool ok = t < len;
        al[t] = ok ? al[t] : 1.f;
        kk[t] = ok ? kk[t] : 0.f;
        qq[t] = ok ? qq[t] : 0.f;
        kap[t] = ok ? (ISO ? kap[t] * kk[t] : kap[t]) : 0.f;
    }
    ChanDecay d;
    chan_decay(al, d);
    float dG[C];
    IO* dq = reinterpret_cast<IO*>(a.gq);
#pragma unroll
    for (int t = 0; t < C; ++t) {
        dG[t] = 0.f;
        if (t < len) {
            const size_t e = tok_of(t) * DK + ch;
            float skb = 0.f, sqb = 0.f, skt = 0.f, srs = 0.f;
            for (int bl = 0; bl < nblk; ++bl) {
                const float* p = a.part + (size_t)bl * ntok * DK + e;
                skb += p[0];
                sqb += p[ks];
                skt += p[2 * ks];
                if (t == len - 1)
                    srs += p[3 * ks];
            }
            const float G = d.g[t + 1], iG = rcp(G);
            const float kbar = skt * iG;
            dG[t] = skb * kk[t] + sqb * qq[t] - kbar * (kap[t] * iG) + srs;
            dq[e] = from_f32<IO>(sqb * G);
            a.part[ks + e] = kbar;
            a.part[2 * ks + e] = skb * G;
        }
    }
    float W = 0.f;
#pragma unroll
    for (int s = C - 1; s >= 0; --s) {
        if (s < len) {
            W = dG[s] + (s + 1 < len ? d.alf[s + 1] * W : 0.f);
            a.part[3 * ks + tok_of(s) * DK + ch] = ((d.raised >> s) & 1u) ? 0.f : d.g[s] * W;
        }
    }
}

template <typename IO, bool ISO, int DK>
static hipError_t launch_t(const BwdArgs& a, bool adj, hipStream_t stream)
{
    // four waves; the adjoint-only mode at d_k = 128 runs eight (two per
    // SIMD, 16 state rows each: its register set fits the 256 of two waves
    // per SIMD, the full pass's does not)
    constexpr int NWA = DK == 128 ? 8 : 4;
    auto kern = kdn_bwd_chunk_kernel<IO, ISO, DK, false, 4>;
    int nw = 4;
    if (adj) {  // the sequence split runs Diagonal with bf16 io only
        if constexpr (sizeof(IO) == 2 && !ISO) {
            kern = kdn_bwd_chunk_kernel<IO, ISO, DK, true, NWA>;
            nw = NWA;
        } else {
            return hipErrorInvalidValue;
        }
    }
    const size_t smem = sizeof(Smem<DK>);
    hipError_t e = set_lds_limit_once(kern, smem);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3(a.dv / NC, a.B * a.H), dim3(64 * nw), smem, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int nch = (a.T + C - 1) / C;
    if (nch > 0 && !adj) {
        hipLaunchKernelGGL((kdn_bwd_chunk_finish_kernel<IO, ISO, DK>), dim3(a.B * a.H * nch),
                           dim3(DK), 0, stream, a, a.dv / NC);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace cbwd

hipError_t launch_bwd_chunk_mem(const BwdArgs& a, bool iso, int io_dtype, bool adj,
                                hipStream_t stream)
{
    using namespace cbwd;
    const bool bf = io_dtype == 1;
    if (a.dk == 128) {
        if (iso)
            return bf ? launch_t<bf16, true, 128>(a, adj, stream)
                      : launch_t<float, true, 128>(a, adj, stream);
        return bf ? launch_t<bf16, false, 128>(a, adj, stream)
                  : launch_t<float, false, 128>(a, adj, stream);
    }
    if (iso)
        return bf ? launch_t<bf16, true, 64>(a, adj, stream) : launch_t<float, true, 64>(a, adj, stream);
    return bf ? launch_t<bf16, false, 64>(a, adj, stream) : launch_t<float, false, 64>(a, adj, stream);
}

}  // namespace kdn
