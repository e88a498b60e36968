// kdn_walk.hip -- chunkwise KDN forward for bf16 q/k/v, gfx950.
//
// One workgroup owns one (batch, head, tile of DVT value columns) and walks
// the sequence in chunks of C = 16 tokens.  The memory state S (dk x DVT,
// fp32) stays in matrix-core accumulators for the whole sequence; the
// variance state stays in registers of the builder lanes.
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
// (G taken relative to a per-channel power of two c where a chunk decays by
// more than 2^100: Kb, Qb from G / c, Ktp from c / G, the chunk applied to
// diag(c) S and G_C / c bringing it back; see decay_ref)
//   L' = Kb Ktp^T  (diagonal = z_t),  Aqk = tril(Qb Ktp^T) (inclusive)
//   M  = diag(r + z) + tril(L', -1),   T = M^-1
//   Delta' = T (V - Kb S),   O = Qb S + Aqk Delta',
//   S <- diag(G_C) (S + Ktp^T Delta')
// which equals the token recurrence in exact arithmetic.  Ragged tails are
// padded with identity tokens (k = q = v = 0, alpha = 1, omega = 0, r = 1).
//
// Diagonal variance in homogeneous form (§6): p = n / d with
//   n_t = alpha^2 n_{t-1} + omega d_{t-1}       (so p^_t = n_t / d_{t-1})
//   d_t = d_{t-1} + u_t n_t,  u_t = mu k_t^2 / r_t
// i.e. the 2x2 Moebius factor [[alpha^2, omega], [u alpha^2, 1 + u omega]]
// applied to [n; d].  The recurrence needs no division; both coordinates are
// rescaled by the same power of two every four tokens, which leaves every
// ratio n / d bit-identical.  Ktp = k n_t / (d_{t-1} G_t) takes the one
// reciprocal per token and channel, off the recurrence's dependency chain.
//
// The memory update is the compact-WY correction of the notes' Appendix D
// summary, Delta' = T (V - Kb S), formed in that order: Kb S costs the same
// matrix-core work as W S with W = T Kb, and then no W has to be formed or
// staged.  V - Kb S is a lane-local subtraction, because the accumulator
// layout of Kb S is the operand layout of V.
//
// Workgroup roles, one LDS barrier per step.  In step c:
//   loader wave    copies the raw inputs (alpha, k, q, r, and Isotropic
//                  omega) of chunk c + LR straight from global memory into
//                  LDS, and v of chunk c + 2;
//   isotropic wave (Isotropic only) reduces alpha^2 and k^2 over channels per
//                  token of chunk c + 4 and runs the scalar variance
//                  recurrence;
//   builder waves  (lane = key channel) run the per-channel recurrence of
//                  chunk c + 3 (Diagonal omega prefetched from global memory
//                  into registers) and write its bf16 operands to LDS: Ktp and
//                  G_C, plus Kb and Qb for Isotropic; for Diagonal an
//                  elementwise wave forms Kb and Qb (two channels per lane);
//   factor waves   the first forms L', Aqk and the diagonal 8 x 8 blocks of
//                  T = M^-1 of chunk c + 2 (one lane per column, or per row
//                  for the lower block); the second forms the off-diagonal
//                  block on the matrix cores and assembles T of chunk
//                  c + 1;
//   memory waves   apply chunk c to their value columns (16 NB each).
// Every buffer is indexed by chunk number modulo its lifetime, so no role
// waits for another inside a step.
#include "kdn_common.h"
#include "kdn_internal.h"

#include <type_traits>

// The roles' step bodies are lambdas; each must be inlined into the kernel
// (an outlined call spills the role's registers to scratch on every step).
#define KDN_INLINE __attribute__((always_inline))

namespace kdn {
namespace walk {

constexpr int C = 16;     // tokens per chunk
constexpr int NRING = 8;  // per-token scalar rings (r, isotropic omega and b^)

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Direct global -> LDS copy: lane l's 16 (or 4) bytes, read at base + off
// (base uniform, off the lane's byte offset), land at LDS byte address
// lds + 16 l (4 l); lds is uniform.  Completion is tracked by vmcnt.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds)
{
    __builtin_amdgcn_global_load_lds((glb_void_t*)((const char*)base + off),
                                     (lds_void_t*)(size_t)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* base, uint32_t off, uint32_t lds)
{
    __builtin_amdgcn_global_load_lds((glb_void_t*)((const char*)base + off),
                                     (lds_void_t*)(size_t)lds, 4, 0, 0);
}

// Order this wave's LDS writes before its later LDS reads (lanes read what
// other lanes of the same wave wrote).  Only LDS operations are waited for.
__device__ __forceinline__ void lds_wave_sync()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Buffer descriptor over a gate tensor from `base` to its end (`bytes` left,
// clamped to the 2^31 - 1 byte range of the record count): loads through it
// are range-checked, and reads past the end of the tensor (the rows after the
// last token of a ragged final chunk) return 0 instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gate_rsrc(const void* base, size_t bytes)
{
    const int nrec = bytes > 0x7fffffffull ? 0x7fffffff : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
}
__device__ __forceinline__ float gate_ld1(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0u, 0));
}
// a bf16 gate pre-activation, zero-extended into the low half of the result
// (kept as the bit pattern of a float until it is used)
__device__ __forceinline__ float gate_ld1_bf16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0u, 0));
}

// Start a role that prefetches from global memory into a register ring with
// nothing in flight.  The wait is free there, and it resets the compiler's
// count of outstanding memory operations: the mix of operation kinds that
// may still be pending from code before the role dispatch otherwise turns
// every later wait in the loop into a full drain, including the prefetch
// issued just before it.
__device__ __forceinline__ void settle_counters()
{
    __builtin_amdgcn_s_waitcnt(0);
}

// Keep every LDS read issued above this point ahead of all the arithmetic
// below it.  The scheduler otherwise interleaves reads with their consumers
// to save registers, which turns one trip through the LDS queue into several
// back-to-back ones.
__device__ __forceinline__ void reads_issued()
{
    __builtin_amdgcn_sched_barrier(0);
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

// ds_read_b64_tr_b16: inside each group of 16 lanes, lane j receives element
// j & 3 of the 8-byte segments addressed by lanes 4 e + (j >> 2), e = 0..3.
__device__ __forceinline__ bf16x4 ds_read_tr(const bf16* p)
{
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat8(const bf16x4& a, const bf16x4& b)
{
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// round to nearest even, two values per conversion instruction
__device__ __forceinline__ bf16x4 cvt4(const f32x4& x)
{
    return __builtin_convertvector(x, bf16x4);
}

__device__ __forceinline__ float bcast(float x, int lane)
{
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

__device__ __forceinline__ void mfma16(f32x4& d, const bf16x4& a, const bf16x4& b)
{
    d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, d, 0, 0, 0);
}
// acc += X^T Y for 16 x 16 fp32 matrices held in the accumulator layout
// (lane (g, c) holds X[4 g + r][c], r = 0..3).  Step r of the four
// 16x16x4 products takes k = 4 g + r: lane (g, c) supplies A[c][k] =
// X[4 g + r][c] and B[k][c] = Y[4 g + r][c].
__device__ __forceinline__ void mma_tn(f32x4& acc, const f32x4& X, const f32x4& Y)
{
#pragma unroll
    for (int r = 0; r < 4; ++r)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[r], Y[r], acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma32(f32x4& d, const bf16x8& a, const bf16x8& b)
{
    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, d, 0, 0, 0);
}

// Wave roles of one workgroup.
enum Role { R_MEM, R_BLD, R_ELT, R_FAC1, R_FAC2, R_LDR, R_ISO };

template <int DK_, int NB_, int NMW_, bool ISO_, bool X3_ = false, bool OF32_ = false,
          int SO_ = 0, int PRE_ = 0>
struct Cfg {
    static constexpr int DK = DK_;
    static constexpr int NB = NB_;    // 16-column blocks per memory wave
    static constexpr int NMW = NMW_;  // memory waves
    static constexpr bool ISO = ISO_;
    // split products (Diagonal only): every matrix-core operand is a pair of
    // bf16 values hi + lo with lo = bf16(x - hi), and every contraction is the
    // three bf16 products hi.hi + lo.hi + hi.lo accumulated in fp32, which
    // carries about 16 significant bits per operand instead of 8
    static constexpr bool X3 = X3_;
    static_assert(!(X3_ && ISO_), "split products are built for the Diagonal variant");
    // o written in fp32 (split products only): the output keeps the
    // contractions' precision instead of rounding to bf16
    static constexpr bool OF32 = OF32_;
    static_assert(!OF32_ || X3_, "fp32 output comes with split products");
    // state-only walks (S_T and the variance, no outputs): SO_ = 1 reads no q
    // and writes no o; SO_ = 2 also takes v = 0 without reading it, so that
    // the innovation is -Kb S
    static constexpr int SO = SO_;
    static constexpr bool NOQ = SO_ > 0;
    static constexpr bool NOV = SO_ == 2;
    static_assert(SO_ >= 0 && SO_ <= 2 && !(SO_ && OF32_), "state-only mode");
    // gates from their bf16 pre-activations (PRE_ = 1: alpha, for
    // Isotropic; 2: alpha and the Diagonal omega): the loader copies a (the
    // pre-activation of alpha) into the second half of a raw slot's alpha
    // array and turns it into alpha = sigmoid(a) in place one step later;
    // with PRE_ = 2 the Diagonal builders load w and form omega = softplus(w)
    // themselves.  The per-token gates (r, Isotropic omega) arrive as fp32.
    static constexpr bool PRE = PRE_ > 0;
    static constexpr bool PREW = PRE_ == 2;
    static_assert(PRE_ >= 0 && PRE_ <= 2 && !(PRE_ && (SO_ || OF32_)) && !(PREW && ISO_),
                  "pre-activation mode");
    static constexpr int DVT = 16 * NB * NMW;
    // builder waves, one lane per key channel.  Diagonal splits the builder
    // work: these waves run the variance recurrence and form Ktp and G_C,
    // one more wave (elementwise) forms Kb and Qb
    static constexpr int NBW = DK / 64;
    static constexpr bool SPLIT = !ISO;
    static constexpr int NEW = SPLIT ? 1 : 0;
    static constexpr int NWAVES = NMW + NBW + NEW + 3 + (ISO ? 1 : 0);
    // Hardware wave w runs on SIMD w % 4; the layout pairs each heavy role
    // (memory, builders, first factor) with a lighter one on its SIMD.  With
    // split products the memory waves set the step, and the SIMDs they run
    // on take the two factor waves (measured: 3% faster than the loader
    // beside a memory wave, and 5% with pre-activations, whose sigmoids the
    // loader evaluates); single products keep the first factor wave beside a
    // builder (measured faster there).
    // Entry w: role * 8 + index within the role.
    static constexpr int layout(int w)
    {
        if constexpr (DK == 128 && NMW == 2 && !ISO && X3_) {
            constexpr int L[8] = {R_MEM * 8, R_MEM * 8 + 1, R_BLD * 8, R_BLD * 8 + 1,
                                  R_FAC2 * 8, R_FAC1 * 8, R_LDR * 8, R_ELT * 8};
            return L[w];
        } else if constexpr (DK == 128 && NMW == 2 && !ISO) {
            constexpr int L[8] = {R_MEM * 8, R_MEM * 8 + 1, R_BLD * 8, R_BLD * 8 + 1,
                                  R_FAC2 * 8, R_LDR * 8, R_FAC1 * 8, R_ELT * 8};
            return L[w];
        } else if constexpr (DK == 128 && NMW == 2 && ISO) {
            constexpr int L[8] = {R_MEM * 8, R_MEM * 8 + 1, R_FAC1 * 8, R_ISO * 8,
                                  R_FAC2 * 8, R_LDR * 8, R_BLD * 8, R_BLD * 8 + 1};
            return L[w];
        } else {
            // memory, builders, elementwise, factor, factor, loader, isotropic
            if (w < NMW)
                return R_MEM * 8 + w;
            if (w < NMW + NBW)
                return R_BLD * 8 + (w - NMW);
            if (w < NMW + NBW + NEW)
                return R_ELT * 8;
            const int k = w - (NMW + NBW + NEW);
            return (k == 0 ? R_FAC1 : k == 1 ? R_FAC2 : k == 2 ? R_LDR : R_ISO) * 8;
        }
    }
    // pipeline leads (steps between a role's work on a chunk and the memory
    // waves applying it): builders 3, isotropic wave 4, raw copies LR (two
    // steps in flight before their first reader)
    static constexpr int LB = 3;
    static constexpr int LR = ISO ? 6 : 5;
    static constexpr int NRAW = LR - LB + 1;  // raw-input slots: copy issue .. builders read
    static constexpr int NOPS = 4;        // operand slots (builders -> factor -> memory)
    // operands in token-quad layout: element (t, i) at [t >> 2][i][t & 3];
    // the quad stride is padded by 32 bytes so that the four quads of one
    // channel sit on different banks
    static constexpr int QS = DK * 4 + 16;
    static constexpr int LDF = C + 4;  // Aqk rows (40 bytes)
};

template <typename CF>
struct Smem {
    static constexpr int DK = CF::DK;
    struct Ops {  // builders -> factor, memory
        alignas(16) bf16 Kb[4 * CF::QS];
        alignas(16) bf16 Qb[4 * CF::QS];
        alignas(16) bf16 Ktp[4 * CF::QS];
        alignas(16) float gC[DK];
        alignas(16) float cS[DK];  // per-channel decay reference c (a power of two)
        int cfl[4];                // per builder wave: some c != 1 in this chunk
    };
    struct Tri {  // first factor wave -> second factor wave, memory
        alignas(16) float Mt[C * 20];         // M^T (fp32): Mt[s][t] = M[t][s], rows padded to 20
        alignas(16) float Mr[8 * 20];         // lower-right block of M, indices reversed:
                                              //   Mr[k][j] = M[15 - k][15 - j]
        alignas(16) float dinv[C];            // 1 / (r_t + z_t)
        alignas(16) float dinvr[8];           // dinv[15 - k]
        alignas(16) float Xs[C * 8];          // row c < 8: T[7 - j][c] (column c of T11,
                                              // reversed); row c >= 8: T[c][8 + j] (T22 row)
        alignas(16) bf16 T[C * C];            // T = M^-1 (bf16, row-major)
        alignas(16) bf16 Aqk[C * CF::LDF];    // Aqk (bf16)
    };
    struct Raw {  // raw inputs of one chunk, rows of tokens as in global memory
        alignas(16) float alpha[C * DK];
        alignas(16) bf16 k[C * DK];
        alignas(16) bf16 q[C * DK];
    };
    // the arrays the memory waves read every step come first, so that their
    // addresses stay within reach of the LDS instructions' immediate offsets
    Ops op[CF::NOPS];
    Tri tri[3];
    alignas(16) bf16 v[3][C * CF::DVT];  // rows of DVT; 16-byte block b of row t at b ^ (t & 7)
    alignas(16) float rr[NRING][C];  // r_t
    alignas(16) float wr[NRING][C];  // isotropic omega_t
    alignas(16) float bh[NRING][C];  // isotropic b^_t
    Raw raw[CF::NRAW];
};

// LDS of the split-product walk.  Kb and Qb (hi and lo) live from the
// elementwise wave's write (step X - 3) to the memory waves' fetch during step
// X - 1, so three slots suffice; Ktp (hi and lo) and G_C are read by the memory
// waves in step X itself and keep four.  The second factor wave forms Aqk one
// step later than in the single-product walk, so the memory waves read it with
// T after the barrier.
template <typename CF>
struct SmemX3 {
    static constexpr int DK = CF::DK;
    struct KQ {  // elementwise wave -> first factor wave, second factor wave, memory
        alignas(16) bf16 Kb[4 * CF::QS];
        alignas(16) bf16 Kl[4 * CF::QS];
        alignas(16) bf16 Qb[4 * CF::QS];
        alignas(16) bf16 Ql[4 * CF::QS];
    };
    struct KT {  // builders -> factor waves, memory
        alignas(16) bf16 Ktp[4 * CF::QS];
        alignas(16) bf16 Ktl[4 * CF::QS];
        alignas(16) float gC[DK];
        alignas(16) float cS[DK];
        int cfl[4];
    };
    struct Tri {
        alignas(16) float Mt[C * 20];
        alignas(16) float Mr[8 * 20];
        alignas(16) float dinv[C];
        alignas(16) float dinvr[8];
        alignas(16) float Xs[C * 8];
        alignas(16) bf16 T[C * C];
        alignas(16) bf16 Tl[C * C];
        alignas(16) bf16 Aqk[C * CF::LDF];
        alignas(16) bf16 Aql[C * CF::LDF];
    };
    struct Raw {
        alignas(16) float alpha[C * DK];
        alignas(16) bf16 k[C * DK];
        alignas(16) bf16 q[C * DK];
    };
    KT kt[4];
    Tri tri[3];
    alignas(16) bf16 v[3][C * CF::DVT];
    alignas(16) float rr[NRING][C];
    alignas(16) float wr[NRING][C];
    alignas(16) float bh[NRING][C];
    KQ kq[3];
    Raw raw[CF::NRAW];
};

// hi / lo halves of a split operand: hi = bf16(x), lo = bf16(x - hi), both
// rounded to nearest even; hi is widened back by a shift or a mask of its
// packed pair, so four values take 12 vector instructions
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split4(const f32x4& x, bf16x4& hi, bf16x4& lo)
{
    hi = cvt4(x);
    const u32x2 w = __builtin_bit_cast(u32x2, hi);
    f32x4 r;
    r[0] = x[0] - __uint_as_float(w[0] << 16);
    r[1] = x[1] - __uint_as_float(w[0] & 0xffff0000u);
    r[2] = x[2] - __uint_as_float(w[1] << 16);
    r[3] = x[3] - __uint_as_float(w[1] & 0xffff0000u);
    lo = cvt4(r);
}

// Offset (elements) of the 8-byte segment that lane (g, l16) addresses in a
// token-quad operand so that ds_read_tr returns, in lane (g, c), the values
// X[t = c][4 g + e], e = 0..3 (channel offset i0 adds 4 i0 elements).
template <int QS>
__device__ __forceinline__ int quad_tr_lane(int lane)
{
    const int g = lane >> 4, l16 = lane & 15;
    return (l16 & 3) * QS + (4 * g + (l16 >> 2)) * 4;
}

// A / B fragment of one K = 32 step over channels 32 m + {4 g + e, 16 + 4 g + e}
// (the order in which two 16-row accumulator blocks of S feed the same step)
__device__ __forceinline__ bf16x8 quad_frag32(const bf16* lane_base, int m)
{
    return cat8(ds_read_tr(lane_base + 128 * m), ds_read_tr(lane_base + 128 * m + 64));
}

template <typename CF>
__global__ __launch_bounds__(64 * CF::NWAVES, 1) void kdn_walk_fwd_kernel(FwdArgs a)
{
    using SM = std::conditional_t<CF::X3, SmemX3<CF>, Smem<CF>>;
    constexpr int DK = CF::DK;
    constexpr int NB = CF::NB;
    constexpr int NMW = CF::NMW;
    constexpr int DVT = CF::DVT;
    constexpr int QS = CF::QS;
    constexpr int LDF = CF::LDF;
    constexpr int LR = CF::LR;
    constexpr int LB = CF::LB;
    constexpr int NRAW = CF::NRAW;
    constexpr int NOPS = CF::NOPS;
    constexpr bool ISO = CF::ISO;
    static_assert(sizeof(SM) <= 160 * 1024, "LDS budget");
    static_assert(DK % 64 == 0 && DVT % 64 == 0, "tile shape");
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SM& sm = *reinterpret_cast<SM*>(smem_raw);

    const int lane = threadIdx.x & 63;
    const int slot = CF::layout(threadIdx.x >> 6);
    const int role = slot >> 3, ridx = slot & 7;
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
    auto row_k = [&](int t) { return (((size_t)b * T + t) * H + h) * DK; };
    auto row_v = [&](int t) { return (((size_t)b * T + t) * H + h) * dv; };
    auto row_s = [&](int t) { return ((size_t)b * T + t) * H + h; };
    // Range-checked descriptor over gate tensor g from the first token of
    // chunk x (clamped into the sequence) to the end of the tensor.  With no
    // chunks at all it covers nothing: every load through it returns 0
    // without an access.
    const size_t gate_elems = (size_t)a.B * T * H * DK;
    auto gate_desc = [&](const void* g, int x) {
        constexpr size_t es = CF::PREW ? 2 : 4;  // bf16 pre-activations or fp32 gates
        if (nchunks == 0)
            return gate_rsrc(g, 0);
        const size_t cb = row_k(min(max(x, 0), nchunks - 1) * C);
        return gate_rsrc((const char*)g + es * cb, es * (gate_elems - cb));
    };

    if (role == R_MEM) {
        // ===================== memory waves =====================
        // block nb of wave w covers value columns jl = 16 (NB w + nb) + c16;
        // Sacc[nb][n] holds S[16 n + 4 g4 + r][j0 + jl]
        const int w = ridx;
        f32x4 Sacc[NB][DK / 16];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int col = j0 + 16 * (NB * w + nb) + c16;
            if (a.S0) {
                const float* S0 = a.S0 + (size_t)bh * DK * dv + col;
#pragma unroll
                for (int n = 0; n < DK / 16; ++n)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Sacc[nb][n][r] = S0[(size_t)(16 * n + 4 * g4 + r) * dv];
            } else {
#pragma unroll
                for (int n = 0; n < DK / 16; ++n)
                    Sacc[nb][n] = zero4();
            }
        }
        // A chunk whose decay takes a reference c != 1 (its Kb, Qb hold G / c
        // and its Ktp c / G) is applied to diag(c) S (its flag arrives with its
        // operands, fetched during the step before), and its G_C / c brings
        // the state back to S at the end of the step.
        // (bit w of the flag: builder wave w, channels 64 w .. 64 w + 63)
        auto chunk_flag = [&](const int (&cfl)[4]) KDN_INLINE {
            int f = cfl[0];
#pragma unroll
            for (int w2 = 1; w2 < CF::NBW; ++w2)
                f |= cfl[w2] << w2;
            return f;
        };
        auto scale_state = [&](int flag, const float* cS) KDN_INLINE {
#pragma unroll
            for (int w2 = 0; w2 < CF::NBW; ++w2) {
                if (flag & (1 << w2)) {
#pragma unroll
                    for (int n = 4 * w2; n < 4 * w2 + 4; ++n) {
                        const f32x4 cs = *reinterpret_cast<const f32x4*>(&cS[16 * n + 4 * g4]);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            Sacc[nb][n] *= cs;
                    }
                }
            }
        };
        // lane parts of the LDS addresses (elements)
        const int tr_lane = quad_tr_lane<QS>(lane);   // Kb, Qb transpose reads
        const int kt_lane = g4 * QS + c16 * 4;        // Ktp^T rows: quad g4, channel c16
        const int fr_lane = c16 * LDF + 4 * g4;       // Aqk rows
        int v_lane[NB];                               // v tile transpose reads
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int t = 4 * g4 + ((lane >> 2) & 3);
            const int col = 16 * (NB * w + nb) + 4 * (lane & 3);
            v_lane[nb] = t * DVT + (((col >> 3) ^ (t & 7)) << 3) + (col & 7);
        }
        // o rows of this lane (token c16 of each chunk), advanced per chunk
        const size_t o_step = (size_t)C * H * dv;
        const size_t o_el = row_v(min(c16, max(T - 1, 0))) + j0 + 16 * NB * w + 4 * g4;
        bf16* orow = reinterpret_cast<bf16*>(reinterpret_cast<char*>(a.o) +
                                             o_el * (CF::OF32 ? sizeof(float) : sizeof(bf16)));

        if constexpr (CF::X3) {
            // ---- split products: Kb and Qb (hi, lo) of chunk c + 1 are
            // fetched during step c, into the registers the front products of
            // chunk c have just consumed; T and Aqk (hi, lo) are read after
            // the barrier with v
            // The state-only walk from the real v (SO = 1) can also store the
            // state at every chunk start (the backward's checkpoints): per
            // (b, h, tile) and chunk a [DK / 4][DVT][4] block, rows in fours,
            // so each accumulator tile is one 16-byte store per lane.
            float* ck = nullptr;
            if constexpr (CF::SO == 1)
                if (a.ckpt)
                    ck = a.ckpt + ((size_t)bh * ntiles + tile) * nchunks * (size_t)(DK * DVT) +
                         (size_t)(g4 * DVT + 16 * NB * w + c16) * 4;
            struct MemOpsX {
                bf16x8 kh[DK / 32], kl[DK / 32], qh[DK / 32], ql[DK / 32];
                int cfl;  // the chunk's decay-reference flag
            };
            auto fetchx = [&](int c, MemOpsX& m) KDN_INLINE {
                const auto& kq = sm.kq[c % 3];
                m.cfl = chunk_flag(sm.kt[c & 3].cfl);
#pragma unroll
                for (int mm = 0; mm < DK / 32; ++mm) {
                    m.kh[mm] = quad_frag32(kq.Kb + tr_lane, mm);
                    m.kl[mm] = quad_frag32(kq.Kl + tr_lane, mm);
                    if constexpr (!CF::NOQ) {
                        m.qh[mm] = quad_frag32(kq.Qb + tr_lane, mm);
                        m.ql[mm] = quad_frag32(kq.Ql + tr_lane, mm);
                    }
                }
            };
            const bf16x4 z4{};
            auto applyx = [&](auto full_tag, int c, MemOpsX& m) KDN_INLINE {
                constexpr bool FULL = decltype(full_tag)::value;
                const int nv = FULL ? C : n_valid(c);
                const auto& kt = sm.kt[c & 3];
                const auto& tri = sm.tri[c % 3];
                const bf16* V = sm.v[c % 3];
                const int cfl = m.cfl;
                if constexpr (CF::SO == 1) {
                    if (ck) {  // the chunk-start state, before any decay reference
                        float* p = ck + (size_t)c * (DK * DVT);
#pragma unroll
                        for (int n = 0; n < DK / 16; ++n)
#pragma unroll
                            for (int nb = 0; nb < NB; ++nb)
                                *reinterpret_cast<f32x4*>(p + (4 * n * DVT + 16 * nb) * 4) = Sacc[nb][n];
                    }
                }
                const bf16x4 th = *reinterpret_cast<const bf16x4*>(tri.T + c16 * C + 4 * g4);
                const bf16x4 tl = *reinterpret_cast<const bf16x4*>(tri.Tl + c16 * C + 4 * g4);
                bf16x4 ah{}, al{};
                if constexpr (!CF::NOQ) {
                    ah = *reinterpret_cast<const bf16x4*>(tri.Aqk + fr_lane);
                    al = *reinterpret_cast<const bf16x4*>(tri.Aql + fr_lane);
                }
                bf16x4 vfr[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    vfr[nb] = CF::NOV ? bf16x4{} : ds_read_tr(V + v_lane[nb]);
                reads_issued();
                if constexpr (!FULL && !CF::NOV) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (4 * g4 + e >= nv)
                                vfr[nb][e] = static_cast<bf16>(0.f);
                }
                // front: Y = Kb S, O^T = S^T Qb^T, each as hi.hi + lo.hi + hi.lo
                f32x4 accY[NB], accO[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    accY[nb] = zero4();
                    accO[nb] = zero4();
                }
                // S's next 32 rows are split while the current 32 rows'
                // products run, so vector and matrix work can overlap
                auto split_rows = [&](int mm, bf16x8 (&sh)[NB], bf16x8 (&sl)[NB]) KDN_INLINE {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        bf16x4 h0, l0, h1, l1;
                        split4(Sacc[nb][2 * mm], h0, l0);
                        split4(Sacc[nb][2 * mm + 1], h1, l1);
                        sh[nb] = cat8(h0, h1);
                        sl[nb] = cat8(l0, l1);
                    }
                };
                if (const int f = __builtin_amdgcn_readfirstlane(cfl))
                    scale_state(f, kt.cS);
                bf16x8 sh[NB], sl[NB];
                split_rows(0, sh, sl);
                reads_issued();
#pragma unroll
                for (int mm = 0; mm < DK / 32; ++mm) {
                    bf16x8 nh[NB], nl[NB];
                    if (mm + 1 < DK / 32)
                        split_rows(mm + 1, nh, nl);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        mfma32(accY[nb], m.kh[mm], sh[nb]);
                        if constexpr (!CF::NOQ)
                            mfma32(accO[nb], sh[nb], m.qh[mm]);
                        mfma32(accY[nb], m.kl[mm], sh[nb]);
                        if constexpr (!CF::NOQ)
                            mfma32(accO[nb], sh[nb], m.ql[mm]);
                        mfma32(accY[nb], m.kh[mm], sl[nb]);
                        if constexpr (!CF::NOQ)
                            mfma32(accO[nb], sl[nb], m.qh[mm]);
                    }
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        sh[nb] = nh[nb];
                        sl[nb] = nl[nb];
                    }
                }
                // the next chunk's Kb and Qb, into the registers the front has
                // just consumed
                reads_issued();
                if (c + 1 < nchunks)
                    fetchx(c + 1, m);
                reads_issued();
                // Delta' = T (V - Y) and O^T += Delta'^T Aqk^T: hi.hi + lo.hi as
                // one K = 32 product, hi.lo as a K = 32 product with a zero
                // upper half, so every accumulation chain stays on one opcode
                bf16x4 dh[NB], dl[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    f32x4 res;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        res[e] = CF::NOV ? -accY[nb][e] : static_cast<float>(vfr[nb][e]) - accY[nb][e];
                    bf16x4 rh, rl;
                    split4(res, rh, rl);
                    f32x4 accD = zero4();
                    mfma32(accD, cat8(th, tl), cat8(rh, rh));
                    mfma32(accD, cat8(th, z4), cat8(rl, z4));
                    split4(accD, dh[nb], dl[nb]);
                    if constexpr (CF::NOQ)
                        continue;
                    mfma32(accO[nb], cat8(dh[nb], dl[nb]), cat8(ah, ah));
                    mfma32(accO[nb], cat8(dh[nb], z4), cat8(al, z4));
                    if (FULL || c16 < nv) {
                        if constexpr (CF::OF32)
                            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(orow) + 16 * nb) = accO[nb];
                        else
                            *reinterpret_cast<bf16x4*>(orow + 16 * nb) = cvt4(accO[nb]);
                    }
                }
                // S <- diag(G_C) (S + Ktp^T Delta'), Ktp and G_C of 16 rows at a
                // time read two blocks ahead of their products
                constexpr int PD = 2;
                bf16x4 kth[PD + 1], ktl[PD + 1];
                f32x4 gcf[PD + 1];
                auto ldk = [&](int n, int s) KDN_INLINE {
                    kth[s] = *reinterpret_cast<const bf16x4*>(kt.Ktp + kt_lane + 64 * n);
                    ktl[s] = *reinterpret_cast<const bf16x4*>(kt.Ktl + kt_lane + 64 * n);
                    gcf[s] = *reinterpret_cast<const f32x4*>(&kt.gC[16 * n + 4 * g4]);
                };
#pragma unroll
                for (int n = 0; n < PD; ++n)
                    ldk(n, n);
#pragma unroll
                for (int n = 0; n < DK / 16; ++n) {
                    if (n + PD < DK / 16)
                        ldk(n + PD, (n + PD) % (PD + 1));
                    reads_issued();
                    const int s = n % (PD + 1);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        mfma32(Sacc[nb][n], cat8(kth[s], ktl[s]), cat8(dh[nb], dh[nb]));
                        mfma32(Sacc[nb][n], cat8(kth[s], z4), cat8(dl[nb], z4));
                        Sacc[nb][n] *= gcf[s];
                    }
                }
            };
            for (int c = -LR; c < 0; ++c)
                lds_barrier();
            MemOpsX ops;
            if (nchunks > 0)
                fetchx(0, ops);
            const int nfull = T / C;
            // o advances one chunk of rows per step (twice the elements' bytes
            // with fp32 output, counted in bf16 units)
            const size_t ostep = CF::OF32 ? 2 * o_step : o_step;
            for (int c = 0; c < nfull; ++c) {
                applyx(std::integral_constant<bool, true>{}, c, ops);
                orow += ostep;
                lds_barrier();
            }
            if (nfull < nchunks) {
                applyx(std::integral_constant<bool, false>{}, nfull, ops);
                lds_barrier();
            }
        } else {
        // operands of one chunk that were written two or more steps before
        // the memory waves apply it; they are fetched during the previous
        // step, after that step's own reads have landed, which takes them
        // out of the read burst after each barrier
        struct MemOps {
            bf16x8 kf[DK / 32], qf[DK / 32];  // Kb, Qb transposed fragments
            bf16x4 afr;                       // Aqk row
            int cfl;                          // decay-reference flag
        };
        auto fetch = [&](int c, MemOps& m) KDN_INLINE {
            const auto& op = sm.op[c & (NOPS - 1)];
            m.cfl = chunk_flag(op.cfl);
#pragma unroll
            for (int mm = 0; mm < DK / 32; ++mm) {
                m.kf[mm] = quad_frag32(op.Kb + tr_lane, mm);
                if constexpr (!CF::NOQ)
                    m.qf[mm] = quad_frag32(op.Qb + tr_lane, mm);
            }
            if constexpr (!CF::NOQ)
                m.afr = *reinterpret_cast<const bf16x4*>(sm.tri[c % 3].Aqk + fr_lane);
        };

        auto apply = [&](auto full_tag, int c, const MemOps& cur, MemOps& nxt) KDN_INLINE {
            constexpr bool FULL = decltype(full_tag)::value;
            const int nv = FULL ? C : n_valid(c);
            const auto& op = sm.op[c & (NOPS - 1)];
            const auto& tri = sm.tri[c % 3];
            const bf16* V = sm.v[c % 3];
            const int cfl = cur.cfl;
            // this step's first reads: T (formed in the previous step) and v
            const bf16x4 tfr = *reinterpret_cast<const bf16x4*>(tri.T + c16 * C + 4 * g4);  // T[c16][4 g4 + e]
            bf16x4 vfr[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                vfr[nb] = CF::NOV ? bf16x4{} : ds_read_tr(V + v_lane[nb]);
            reads_issued();
            if constexpr (!FULL && !CF::NOV) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * g4 + e >= nv)
                            vfr[nb][e] = static_cast<bf16>(0.f);
            }
            if (const int f = __builtin_amdgcn_readfirstlane(cfl))
                scale_state(f, op.cS);
            // front:  Y = Kb S  ([t][j]),   O^T = S^T Qb^T  ([j][t])
            f32x4 accY[NB], accO[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                accY[nb] = zero4();
                accO[nb] = zero4();
            }
#pragma unroll
            for (int m = 0; m < DK / 32; ++m) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const bf16x8 s = cat8(cvt4(Sacc[nb][2 * m]), cvt4(Sacc[nb][2 * m + 1]));
                    mfma32(accY[nb], cur.kf[m], s);
                    if constexpr (!CF::NOQ)
                        mfma32(accO[nb], s, cur.qf[m]);
                }
            }
            // Ktp and G_C for the state update at the end of the step, then the
            // next chunk's operands behind them
            reads_issued();
            bf16x4 ktf[DK / 16];
            f32x4 gcf[DK / 16];
#pragma unroll
            for (int n = 0; n < DK / 16; ++n) {
                ktf[n] = *reinterpret_cast<const bf16x4*>(op.Ktp + kt_lane + 64 * n);
                gcf[n] = *reinterpret_cast<const f32x4*>(&op.gC[16 * n + 4 * g4]);
            }
            if (c + 1 < nchunks)
                fetch(c + 1, nxt);
            reads_issued();
            bf16x4 dfr[NB];
            // Aqk^T fragment as a K = 32 operand whose upper 16 k are zero
            const bf16x8 afr32 = CF::NOQ ? bf16x8{} : cat8(cur.afr, bf16x4{});
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                // Delta' = T (V - Y): lane (g, c) holds V[4 g + e][c] as an
                // operand and Y[4 g + e][c] as an accumulator
                f32x4 res;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    res[e] = CF::NOV ? -accY[nb][e] : static_cast<float>(vfr[nb][e]) - accY[nb][e];
                f32x4 accD = zero4();
                mfma16(accD, tfr, cvt4(res));
                dfr[nb] = cvt4(accD);
                if constexpr (CF::NOQ)
                    continue;
                // O^T += Delta'^T Aqk^T, issued as a zero-padded K = 32 product:
                // the accumulator comes from 16x16x32 products, and on gfx950 a
                // 16x16x16 product reading it as its accumulator needs more
                // independent instructions in between than are inserted for it
                mfma32(accO[nb], cat8(dfr[nb], bf16x4{}), afr32);
                if (FULL || c16 < nv)
                    *reinterpret_cast<bf16x4*>(orow + 16 * nb) = cvt4(accO[nb]);
            }
            // S <- diag(G_C) (S + Ktp^T Delta')
#pragma unroll
            for (int n = 0; n < DK / 16; ++n) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    mfma16(Sacc[nb][n], ktf[n], dfr[nb]);
                    Sacc[nb][n] *= gcf[n];
                }
            }
        };
        // pipeline fill, the full chunks (two per iteration, alternating
        // operand sets), then at most one ragged chunk (one barrier per step
        // as in every role; separate loops keep S in place)
        for (int c = -LR; c < 0; ++c)
            lds_barrier();
        MemOps opA, opB;
        if (nchunks > 0)
            fetch(0, opA);
        const int nfull = T / C;
        int c = 0;
        for (; c + 1 < nfull; c += 2) {
            apply(std::integral_constant<bool, true>{}, c, opA, opB);
            orow += o_step;
            lds_barrier();
            apply(std::integral_constant<bool, true>{}, c + 1, opB, opA);
            orow += o_step;
            lds_barrier();
        }
        bool inB = false;
        if (c < nfull) {
            apply(std::integral_constant<bool, true>{}, c, opA, opB);
            orow += o_step;
            lds_barrier();
            inB = true;
        }
        if (nfull < nchunks) {
            if (inB)
                apply(std::integral_constant<bool, false>{}, nfull, opB, opA);
            else
                apply(std::integral_constant<bool, false>{}, nfull, opA, opB);
            lds_barrier();
        }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            float* ST = a.S_T + (size_t)bh * DK * dv + j0 + 16 * (NB * w + nb) + c16;
#pragma unroll
            for (int n = 0; n < DK / 16; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    ST[(size_t)(16 * n + 4 * g4 + r) * dv] = Sacc[nb][n][r];
        }
    } else if (role == R_BLD) {
        // ================ builder waves: lane = key channel ================
        const int i = ridx * 64 + lane;
        // Diagonal: homogeneous variance [n; d];  Isotropic: no state here
        float vn = (!ISO && a.var0) ? a.var0[(size_t)bh * DK + i] : var_init;
        float vd = 1.f;
        // Diagonal omega of this lane's channel comes straight from global
        // memory, OPF chunks ahead, into a register ring of OPF + 1 slots
        // (16 loads per step, so at most 16 (OPF + 1) - 1 = 63 outstanding)
        constexpr int OPF = 3;
        float rw[OPF + 1][ISO ? 1 : C];
        // (with pre-activations: w as bf16 bits, turned into omega at use)
        uint32_t goff[C];
#pragma unroll
        for (int t = 0; t < C; ++t)
            goff[t] = (CF::PREW ? 2u : 4u) * ((uint32_t)t * (uint32_t)(H * DK) + (uint32_t)i);
        auto load_omega = [&](auto slot_tag, int X) KDN_INLINE {
            if constexpr (!ISO) {
                constexpr int S = decltype(slot_tag)::value;
                if constexpr (CF::PREW) {
                    const auto rom = gate_desc(a.w_pre, X);
#pragma unroll
                    for (int t = 0; t < C; ++t)
                        rw[S][t] = gate_ld1_bf16(rom, goff[t]);
                } else {
                    const auto rom = gate_desc(a.omega, X);
#pragma unroll
                    for (int t = 0; t < C; ++t)
                        rw[S][t] = gate_ld1(rom, goff[t]);
                }
            }
        };
        auto build = [&](auto full_tag, int X, const float (&omr)[ISO ? 1 : C]) KDN_INLINE {
            constexpr bool FULL = decltype(full_tag)::value;
            const int nv = FULL ? C : n_valid(X);
            const auto& raw = sm.raw[X % NRAW];
            // per-token scalars, computed by lanes 0..15 and broadcast:
            // Diagonal mu / r_t, Isotropic b^_t
            const float tokr = ISO ? sm.bh[X % NRING][c16] : sm.rr[X % NRING][c16];
            float al[C], om[C], kf[C], qf[C];
            bf16 kr[C], qr[C];
#pragma unroll
            for (int t = 0; t < C; ++t) {
                al[t] = raw.alpha[t * DK + i];
                kr[t] = raw.k[t * DK + i];
                if constexpr (!CF::SPLIT && !CF::NOQ)
                    qr[t] = raw.q[t * DK + i];
            }
            // (Diagonal only: the Isotropic builders measured faster with the
            // compiler's interleaving)
            if constexpr (!ISO)
                reads_issued();
            const float tok = ISO ? tokr : mu * rcp(tokr);
#pragma unroll
            for (int t = 0; t < C; ++t) {
                if constexpr (CF::PREW)
                    om[t] = gate_softplus(bf16_bits_to_f32(__float_as_uint(omr[t])), 0.f);
                else if constexpr (!ISO)
                    om[t] = omr[t];
                kf[t] = static_cast<float>(kr[t]);
                if constexpr (!CF::SPLIT && !CF::NOQ)
                    qf[t] = static_cast<float>(qr[t]);
            }
            if constexpr (!FULL) {
#pragma unroll
                for (int t = 0; t < C; ++t) {
                    const bool ok = t < nv;
                    al[t] = ok ? al[t] : 1.f;
                    if constexpr (!ISO)
                        om[t] = ok ? om[t] : 0.f;
                    kf[t] = ok ? kf[t] : 0.f;
                    if constexpr (!CF::SPLIT && !CF::NOQ)
                        qf[t] = ok ? qf[t] : 0.f;
                }
            }
            float kb[C], qb[C], kt[C];
            // the chunk's decay, G = G_t / c: first with c = 1 (the plain
            // product); channels whose chunk decays past 2^-100 take their
            // reference (decay_plain_ok, decay_ref) and are recomputed, which a
            // wave skips when none of its channels needs it
            float G = 1.f;
            float kn_s[C], vd_s[C];  // Diagonal: p^_t k_t vd_{t-1} and vd_{t-1}
            if constexpr (!ISO) {
                // with split builders Kb and Qb come from the elementwise wave
#pragma unroll
                for (int t = 0; t < C; ++t) {
                    const float n1 = fmaf(om[t], vd, (al[t] * al[t]) * vn);  // p^_t = n1 / vd
                    const float kn = kf[t] * n1;
                    G *= al[t];
                    kt[t] = kn * rcp(vd * G);                    // p^_t k_t c / G_t
                    kn_s[t] = kn;
                    vd_s[t] = vd;
                    vd = fmaf(kf[t] * bcast(tok, t), kn, vd);    // d_t = d_{t-1} + (mu k^2 / r) n_t
                    vn = n1;
                    if ((t & 3) == 3) {
                        // rescale [n; d] by 2^-e(d): exact, keeps n / d
                        const int ex = __builtin_amdgcn_frexp_expf(vd);
                        vn = __builtin_amdgcn_ldexpf(vn, -ex);
                        vd = __builtin_amdgcn_ldexpf(vd, -ex);
                    }
                }
            } else {
#pragma unroll
                for (int t = 0; t < C; ++t) {
                    G *= al[t];
                    kb[t] = kf[t] * G;
                    if constexpr (!CF::NOQ)
                        qb[t] = qf[t] * G;
                }
            }
            DecayRef ref{false, 0};
            bool any = false;  // some channel of this wave takes c != 1
            if (__ballot(!decay_plain_ok(G)) != 0) {
                if (!decay_plain_ok(G)) {
                    ref = decay_ref(al);
                    G = __builtin_amdgcn_ldexpf(1.f, -ref.m);
#pragma unroll
                    for (int t = 0; t < C; ++t) {
                        G *= decay_alpha(ref, al[t]);
                        if constexpr (!ISO) {
                            kt[t] = kn_s[t] * rcp(vd_s[t] * G);
                        } else {
                            kb[t] = kf[t] * G;
                            if constexpr (!CF::NOQ)
                                qb[t] = qf[t] * G;
                        }
                    }
                }
                any = __ballot(ref.m != 0) != 0;
            }
            if constexpr (ISO) {
                // c / G_t = (c / G_C) prod_{s > t} alpha_s, accumulated from
                // c / G_C down, so every partial product stays in the
                // reference's range
                float suf = rcp(G);
#pragma unroll
                for (int t = C - 1; t >= 0; --t) {
                    kt[t] = bcast(tok, t) * kf[t] * suf;
                    suf *= decay_alpha(ref, al[t]);
                }
            }
            // token-quad writes: channel i's four tokens 4 tq .. +3 as 8 bytes
            if constexpr (CF::X3) {
                auto& ks = sm.kt[X & 3];
#pragma unroll
                for (int tq = 0; tq < 4; ++tq) {
                    const int o = tq * QS + i * 4;
                    bf16x4 hi, lo;
                    split4(f32x4{kt[4 * tq], kt[4 * tq + 1], kt[4 * tq + 2], kt[4 * tq + 3]}, hi, lo);
                    *reinterpret_cast<bf16x4*>(ks.Ktp + o) = hi;
                    *reinterpret_cast<bf16x4*>(ks.Ktl + o) = lo;
                }
                ks.gC[i] = G;
                // c of this wave's channels, read only under this wave's flag
                if (any)
                    ks.cS[i] = __builtin_amdgcn_ldexpf(1.f, ref.m);
                if (lane == 0)
                    ks.cfl[ridx] = any;
            } else {
                auto& op = sm.op[X & (NOPS - 1)];
#pragma unroll
                for (int tq = 0; tq < 4; ++tq) {
                    const int o = tq * QS + i * 4;
                    if constexpr (!CF::SPLIT) {
                        *reinterpret_cast<bf16x4*>(op.Kb + o) =
                            bf16x4{static_cast<bf16>(kb[4 * tq]), static_cast<bf16>(kb[4 * tq + 1]),
                                   static_cast<bf16>(kb[4 * tq + 2]), static_cast<bf16>(kb[4 * tq + 3])};
                        if constexpr (!CF::NOQ)
                            *reinterpret_cast<bf16x4*>(op.Qb + o) =
                                bf16x4{static_cast<bf16>(qb[4 * tq]), static_cast<bf16>(qb[4 * tq + 1]),
                                       static_cast<bf16>(qb[4 * tq + 2]), static_cast<bf16>(qb[4 * tq + 3])};
                    }
                    *reinterpret_cast<bf16x4*>(op.Ktp + o) =
                        bf16x4{static_cast<bf16>(kt[4 * tq]), static_cast<bf16>(kt[4 * tq + 1]),
                               static_cast<bf16>(kt[4 * tq + 2]), static_cast<bf16>(kt[4 * tq + 3])};
                }
                op.gC[i] = G;
                if (any)
                    op.cS[i] = __builtin_amdgcn_ldexpf(1.f, ref.m);
                if (lane == 0)
                    op.cfl[ridx] = any;
            }
        };
        settle_counters();
        // slot of chunk X: (X - LB + LR) mod (OPF + 1); the first step
        // consumes chunk LB - LR from slot 0, so prime chunks LB - LR ..
        // LB - LR + OPF - 1 into slots 0 .. OPF - 1
        static_assert(OPF == 3, "four-slot ring");
        load_omega(std::integral_constant<int, 0>{}, LB - LR);
        load_omega(std::integral_constant<int, 1>{}, LB - LR + 1);
        load_omega(std::integral_constant<int, 2>{}, LB - LR + 2);
        auto step = [&](auto slot_tag, int c) KDN_INLINE {
            constexpr int S = decltype(slot_tag)::value;
            const int X = c + LB;
            if (X >= 0 && X < nchunks) {
                if (n_valid(X) == C)
                    build(std::integral_constant<bool, true>{}, X, rw[S]);
                else
                    build(std::integral_constant<bool, false>{}, X, rw[S]);
            }
            load_omega(std::integral_constant<int, (S + OPF) % (OPF + 1)>{}, X + OPF);
            lds_barrier();
        };
        int c = -LR;
        for (; c + 3 < nchunks; c += 4) {
            step(std::integral_constant<int, 0>{}, c);
            step(std::integral_constant<int, 1>{}, c + 1);
            step(std::integral_constant<int, 2>{}, c + 2);
            step(std::integral_constant<int, 3>{}, c + 3);
        }
        if (c < nchunks)
            step(std::integral_constant<int, 0>{}, c);
        if (c + 1 < nchunks)
            step(std::integral_constant<int, 1>{}, c + 1);
        if (c + 2 < nchunks)
            step(std::integral_constant<int, 2>{}, c + 2);
        if constexpr (!ISO) {
            if (tile == 0)
                a.var_T[(size_t)bh * DK + i] = vn / vd;
        }
    } else if (role == R_FAC1) {
        // ============ first factor wave: L', Aqk and T of chunk c + 2 ============
        const int tr_lane = quad_tr_lane<QS>(lane);
        for (int c = -LR; c < nchunks; ++c) {
            const int F = c + 2;
            if (F >= 0 && F < nchunks) {
                const int nv = n_valid(F);
                auto& tr = sm.tri[F % 3];
                const float* rr = sm.rr[F % NRING];
                // L'[t][s] = Kb_t . Ktp_s,   Aqk^T[u][t] = Ktp_u . Qb_t
                f32x4 accL = zero4(), accQ = zero4();
                if constexpr (CF::X3) {
                    // L' only (Aqk is the second factor wave's), as
                    // hi.hi + (lo.hi + hi.lo), the small terms summed first
                    const auto& kq = sm.kq[F % 3];
                    const auto& ks = sm.kt[F & 3];
                    bf16x8 kbh[DK / 32], kbl[DK / 32], kth[DK / 32], ktl[DK / 32];
#pragma unroll
                    for (int m = 0; m < DK / 32; ++m) {
                        kbh[m] = quad_frag32(kq.Kb + tr_lane, m);
                        kbl[m] = quad_frag32(kq.Kl + tr_lane, m);
                        kth[m] = quad_frag32(ks.Ktp + tr_lane, m);
                        ktl[m] = quad_frag32(ks.Ktl + tr_lane, m);
                    }
                    f32x4 accS = zero4();
#pragma unroll
                    for (int m = 0; m < DK / 32; ++m) {
                        mfma32(accL, kbh[m], kth[m]);
                        mfma32(accS, kbl[m], kth[m]);
                        mfma32(accS, kbh[m], ktl[m]);
                    }
                    accL += accS;
                } else {
                    const auto& op = sm.op[F & (NOPS - 1)];
                    bf16x8 kbf[DK / 32], ktf[DK / 32], qbf[DK / 32];
#pragma unroll
                    for (int m = 0; m < DK / 32; ++m) {
                        kbf[m] = quad_frag32(op.Kb + tr_lane, m);
                        ktf[m] = quad_frag32(op.Ktp + tr_lane, m);
                        if constexpr (!CF::NOQ)
                            qbf[m] = quad_frag32(op.Qb + tr_lane, m);
                    }
#pragma unroll
                    for (int m = 0; m < DK / 32; ++m) {
                        mfma32(accL, kbf[m], ktf[m]);
                        if constexpr (!CF::NOQ)
                            mfma32(accQ, ktf[m], qbf[m]);
                    }
                }
                // M^T[s][t] = L'[t][s]   (lane holds L'[4 g4 + r][c16]); the
                // second factor wave reads its lower-left block
                *reinterpret_cast<f32x4*>(&tr.Mt[c16 * 20 + 4 * g4]) = accL;
                // lower-right block with both indices reversed
                if (g4 >= 2 && c16 >= 8) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        tr.Mr[(15 - 4 * g4 - r) * 20 + (15 - c16)] = accL[r];
                }
                if ((c16 >> 2) == g4) {
                    const int rs = c16 & 3;
                    const float z = rs == 0 ? accL[0] : rs == 1 ? accL[1] : rs == 2 ? accL[2] : accL[3];
                    const float rt = c16 < nv ? rr[c16] : 1.f;
                    const float dv = rcp(rt + z);
                    tr.dinv[c16] = dv;
                    if (c16 >= 8)
                        tr.dinvr[15 - c16] = dv;
                    // effective write strength of token c16 (one tile writes it)
                    if (a.beta && tile == 0 && c16 < nv)
                        a.beta[row_s(F * C + c16)] = z * dv;
                }
                // Aqk[t][u] = Aqk^T[u][t] for u <= t, else 0
                if constexpr (!CF::X3 && !CF::NOQ) {
                    f32x4 aq;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        aq[r] = (4 * g4 + r <= c16) ? accQ[r] : 0.f;
                    *reinterpret_cast<bf16x4*>(&tr.Aqk[c16 * LDF + 4 * g4]) = cvt4(aq);
                }
                lds_wave_sync();
                // Diagonal blocks of T = M^-1, one 8-step substitution per lane
                // (the four lane groups repeat it):
                //   c16 < 8:  column c16 of T11 = M11^-1, forward substitution
                //             with the rows of M11^T;
                //   c16 >= 8: row c16 - 8 of T22 = column of (M22^T)^-1, a back
                //             substitution, run forward in reversed indices
                //             (coefficients Mr, pivots dinvr).
                // Both read as x[k] = acc[k] d[k];  acc[j] -= cof[k][j] x[k], j > k.
                const int blk = c16 >> 3, j0 = c16 & 7;
                const float* cof = blk ? tr.Mr : tr.Mt;
                const float* dp = blk ? tr.dinvr : tr.dinv;
                float d[8];
                {
                    const f32x4 d0 = *reinterpret_cast<const f32x4*>(dp);
                    const f32x4 d1 = *reinterpret_cast<const f32x4*>(dp + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        d[e] = d0[e];
                        d[4 + e] = d1[e];
                    }
                }
                const int e0 = blk ? 7 - j0 : j0;
                float acc[8], x[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[j] = (j == e0) ? 1.f : 0.f;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    x[k] = acc[k] * d[k];
#pragma unroll
                    for (int q4 = (k + 1) >> 2; q4 < 2; ++q4) {
                        const f32x4 row = *reinterpret_cast<const f32x4*>(cof + k * 20 + 4 * q4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int j = 4 * q4 + e;
                            if (j > k)
                                acc[j] = fmaf(-row[e], x[k], acc[j]);
                        }
                    }
                }
                // row c16 of Xs: x reversed (T11: T[7 - j][c16]; T22: x[7 - j] = T[c16][8 + j])
                if (g4 == 0) {
                    *reinterpret_cast<f32x4*>(&tr.Xs[c16 * 8]) = f32x4{x[7], x[6], x[5], x[4]};
                    *reinterpret_cast<f32x4*>(&tr.Xs[c16 * 8 + 4]) = f32x4{x[3], x[2], x[1], x[0]};
                }
            }
            lds_barrier();
        }
    } else if (role == R_FAC2) {
        // ============ second factor wave: T21 and T of chunk c + 1 ============
        // T21 = -T22 M21 T11 on the fp32 matrix cores, both products in the
        // X^T Y form of mma_tn:
        //   Q = M21^T T22^T,   R = T11^T (E - Q)  with E the identity on the
        //   upper-left block;  rows 0..7 of R hold T^T: R[i][j] = T[j][i]
        //   (T11 for j < 8, T21 for j >= 8).
        // A-operand fragment of T (lane (g, c): T[c][4 g + e]): R for g < 2,
        // the T22 row for g >= 2 (zero for c < 8).
        const bool v11 = c16 < 8 && g4 < 2, v22 = c16 >= 8 && g4 >= 2;
        const bool v21 = c16 < 8 && g4 >= 2;
        const int xs_off = c16 * 8 + (c16 < 8 ? 4 - 4 * (g4 & 1) : 4 * (g4 & 1));
        const int tr_lane = quad_tr_lane<QS>(lane);
        for (int c = -LR; c < nchunks; ++c) {
            const int F = c + 1;
            if (F >= 0 && F < nchunks) {
                auto& tr = sm.tri[F % 3];
                const f32x4 mt = *reinterpret_cast<const f32x4*>(&tr.Mt[c16 * 20 + 4 * g4]);
                const f32x4 xv = *reinterpret_cast<const f32x4*>(&tr.Xs[xs_off]);
                f32x4 m21, t22t, t11;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    m21[r] = v21 ? mt[r] : 0.f;       // M[4 g + r][c], block (2, 1)
                    t22t[r] = v22 ? xv[r] : 0.f;      // T22^T[4 g + r - 8][c - 8]
                    t11[r] = v11 ? xv[3 - r] : 0.f;   // T11[4 g + r][c]
                }
                f32x4 q = zero4();
                mma_tn(q, m21, t22t);
                f32x4 y;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    y[r] = (4 * g4 + r == c16 && c16 < 8) ? 1.f - q[r] : -q[r];
                f32x4 rt = zero4();
                mma_tn(rt, t11, y);
                if constexpr (CF::X3) {
                    bf16x4 hi, lo;
                    split4(g4 < 2 ? rt : t22t, hi, lo);
                    *reinterpret_cast<bf16x4*>(&tr.T[c16 * C + 4 * g4]) = hi;
                    *reinterpret_cast<bf16x4*>(&tr.Tl[c16 * C + 4 * g4]) = lo;
                    if constexpr (!CF::NOQ) {
                        // Aqk of the same chunk: Aqk^T[u][t] = Ktp_u . Qb_t in split
                        // products, then Aqk[t][u] for u <= t (hi and lo)
                        const auto& kq = sm.kq[F % 3];
                        const auto& ks = sm.kt[F & 3];
                        bf16x8 qbh[DK / 32], qbl[DK / 32], kth[DK / 32], ktl[DK / 32];
#pragma unroll
                        for (int m = 0; m < DK / 32; ++m) {
                            qbh[m] = quad_frag32(kq.Qb + tr_lane, m);
                            qbl[m] = quad_frag32(kq.Ql + tr_lane, m);
                            kth[m] = quad_frag32(ks.Ktp + tr_lane, m);
                            ktl[m] = quad_frag32(ks.Ktl + tr_lane, m);
                        }
                        f32x4 accQ = zero4(), accS = zero4();
#pragma unroll
                        for (int m = 0; m < DK / 32; ++m) {
                            mfma32(accQ, kth[m], qbh[m]);
                            mfma32(accS, ktl[m], qbh[m]);
                            mfma32(accS, kth[m], qbl[m]);
                        }
                        accQ += accS;
                        f32x4 aq;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            aq[r] = (4 * g4 + r <= c16) ? accQ[r] : 0.f;
                        split4(aq, hi, lo);
                        *reinterpret_cast<bf16x4*>(&tr.Aqk[c16 * LDF + 4 * g4]) = hi;
                        *reinterpret_cast<bf16x4*>(&tr.Aql[c16 * LDF + 4 * g4]) = lo;
                    }
                } else {
                    *reinterpret_cast<bf16x4*>(&tr.T[c16 * C + 4 * g4]) = cvt4(g4 < 2 ? rt : t22t);
                }
            }
            lds_barrier();
        }
    } else if (role == R_LDR) {
        // ===================== loader wave =====================
        // direct copies into LDS: raw inputs of chunk c + LR, v of chunk c + 2
        constexpr int VE = 8;                               // bf16 per 16 bytes
        constexpr int LPR_A = DK * 4 / 16;                  // lanes per alpha / omega row
        constexpr int RPI_A = 64 / LPR_A, NI_A = C / RPI_A; // rows per copy, copies
        constexpr int LPR_K = DK * 2 / 16;                  // lanes per k / q row
        constexpr int RPI_K = 64 / LPR_K, NI_K = C / RPI_K;
        constexpr int LPR_V = DVT * 2 / 16;                 // lanes per v tile row
        constexpr int RPI_V = 64 / LPR_V, NI_V = C / RPI_V;
        static_assert(LPR_A <= 64 && LPR_K <= 64 && LPR_V == 8 && NI_A >= 1 && NI_K >= 1,
                      "row / lane split");
        constexpr int NSTG = (CF::PRE ? NI_K : NI_A) + (CF::NOQ ? 1 : 2) * NI_K + 1 + (ISO ? 1 : 0);
        constexpr int NVI = NI_V;
        static_assert(NSTG + NVI <= 63, "outstanding copies within the vmcnt range");
        // LDS byte addresses of the copy targets (uniform)
        const uint32_t lds0 = (uint32_t)(size_t)(lds_void_t*)smem_raw;
        auto lds_addr = [&](const void* p) {
            return lds0 + (uint32_t)((const unsigned char*)p - smem_raw);
        };
        // per-lane byte offsets inside a chunk (the chunk base is uniform);
        // rows past the end of a ragged chunk repeat its last row
        const uint32_t tsk = (uint32_t)(H * DK), tsv = (uint32_t)(H * dv), tss = (uint32_t)H;
        auto off_a = [&](int j, int lim) {  // alpha / omega (4 bytes per element)
            return 4u * ((uint32_t)min(j * RPI_A + lane / LPR_A, lim) * tsk + (lane % LPR_A) * 4);
        };
        auto off_k = [&](int j, int lim) {  // k / q (2 bytes per element)
            return 2u * ((uint32_t)min(j * RPI_K + lane / LPR_K, lim) * tsk + (lane % LPR_K) * VE);
        };
        auto off_v = [&](int j, int lim) {
            const int p = 64 * j + lane;
            const int tl = p / LPR_V;
            const int blk = (p % LPR_V) ^ (tl & 7);
            return 2u * ((uint32_t)min(tl, lim) * tsv + blk * VE);
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
        for (int c = -LR; c < nchunks; ++c) {
            const int X = c + LR;
            const bool sv = X < nchunks;
            const int XV = c + 2;
            const bool vv = !CF::NOV && XV >= 0 && XV < nchunks;
            if (sv) {
                const auto& st = sm.raw[X % NRAW];
                const int tb = X * C;
                const int lim = n_valid(X) - 1;
                const size_t cb = row_k(tb);  // uniform
                const bf16* kb = reinterpret_cast<const bf16*>(a.k) + cb;
                const bf16* qb = reinterpret_cast<const bf16*>(a.q) + cb;
                const uint32_t la = lds_addr(st.alpha), lk = lds_addr(st.k), lq = lds_addr(st.q);
                auto copy_stage = [&](auto full_tag) KDN_INLINE {
                    constexpr bool FULL = decltype(full_tag)::value;
                    if constexpr (CF::PRE) {
                        // a (bf16, laid out as k) into the second half of the
                        // alpha array
                        const bf16* ab = reinterpret_cast<const bf16*>(a.a_pre) + cb;
#pragma unroll
                        for (int j = 0; j < NI_K; ++j) {
                            const uint32_t o = FULL ? ok_[j] : off_k(j, lim);
                            dma16(ab, o, la + C * DK * 2 + j * RPI_K * DK * 2);
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < NI_A; ++j) {
                            const uint32_t o = FULL ? oa[j] : off_a(j, lim);
                            dma16(a.alpha + cb, o, la + j * RPI_A * DK * 4);
                        }
                    }
#pragma unroll
                    for (int j = 0; j < NI_K; ++j) {
                        const uint32_t o = FULL ? ok_[j] : off_k(j, lim);
                        dma16(kb, o, lk + j * RPI_K * DK * 2);
                        if constexpr (!CF::NOQ)
                            dma16(qb, o, lq + j * RPI_K * DK * 2);
                    }
                };
                if (lim == C - 1)
                    copy_stage(std::integral_constant<bool, true>{});
                else
                    copy_stage(std::integral_constant<bool, false>{});
                if (lane < C) {
                    const uint32_t o = 4u * ((uint32_t)min(lane, lim) * tss);
                    const size_t sb = row_s(tb);
                    dma4(a.r + sb, o, lds_addr(sm.rr[X % NRING]));
                    if constexpr (ISO)
                        dma4(a.omega + sb, o, lds_addr(sm.wr[X % NRING]));
                }
            }
            if (vv) {
                const uint32_t lv = lds_addr(sm.v[XV % 3]);
                const int lim = n_valid(XV) - 1;
                const bf16* vb = reinterpret_cast<const bf16*>(a.v) + row_v(XV * C) + j0;  // uniform
                // LDS block p = 64 j + lane holds row p / 8 and data block
                // (p % 8) ^ (row & 7) of that row
                if (lim == C - 1) {
#pragma unroll
                    for (int j = 0; j < NI_V; ++j)
                        dma16(vb, ov[j], lv + 64 * j * 16);
                } else {
#pragma unroll
                    for (int j = 0; j < NI_V; ++j)
                        dma16(vb, off_v(j, lim), lv + 64 * j * 16);
                }
            }
            // the copies of the previous step have landed
            if (sv && vv)
                vm_wait<NSTG + NVI>();
            else if (sv)
                vm_wait<NSTG>();
            else if (vv)
                vm_wait<NVI>();
            else
                vm_wait<0>();
            if constexpr (CF::PRE) {
                // alpha = sigmoid(a) of the chunk copied in the previous step
                // (landed: only this step's copies are still in flight), in
                // place: every lane reads its four-value groups of a before
                // any lane writes, and the wave's LDS operations run in order
                const int Y = c + LR - 1;
                if (Y >= 0 && Y < nchunks) {
                    float* dst = sm.raw[Y % NRAW].alpha;
                    const float* src = dst + C * DK / 2;
                    constexpr int NG = C * DK / 256;  // groups of four per lane
                    float2 pv[NG];
#pragma unroll
                    for (int m = 0; m < NG; ++m)
                        pv[m] = *reinterpret_cast<const float2*>(src + 2 * (64 * m + lane));
                    lds_wave_sync();
#pragma unroll
                    for (int m = 0; m < NG; ++m) {
                        const uint32_t w0 = __float_as_uint(pv[m].x), w1 = __float_as_uint(pv[m].y);
                        const f32x4 g{gate_sigmoid(__uint_as_float(w0 << 16)),
                                      gate_sigmoid(__uint_as_float(w0 & 0xffff0000u)),
                                      gate_sigmoid(__uint_as_float(w1 << 16)),
                                      gate_sigmoid(__uint_as_float(w1 & 0xffff0000u))};
                        *reinterpret_cast<f32x4*>(dst + 4 * (64 * m + lane)) = g;
                    }
                }
            }
            lds_barrier();
        }
    } else if (role == R_ELT) {
        // ======= elementwise wave (Diagonal): Kb = k G, Qb = q G of chunk c + 3 =======
        // lane owns channels CPL lane .. + CPL - 1; G_t = prod_{s <= t} alpha_s
        if constexpr (CF::SPLIT) {
            constexpr int CPL = DK / 64;
            static_assert(CPL == 1 || CPL == 2, "channels per lane");
            auto build = [&](auto full_tag, int X) KDN_INLINE {
                constexpr bool FULL = decltype(full_tag)::value;
                const int nv = FULL ? C : n_valid(X);
                const auto& raw = sm.raw[X % NRAW];
                // destinations: Kb, Qb (and their lo halves with split products)
                bf16 *dKb, *dQb, *dKl = nullptr, *dQl = nullptr;
                if constexpr (CF::X3) {
                    auto& kq = sm.kq[X % 3];
                    dKb = kq.Kb;
                    dQb = kq.Qb;
                    dKl = kq.Kl;
                    dQl = kq.Ql;
                } else {
                    auto& op = sm.op[X & (NOPS - 1)];
                    dKb = op.Kb;
                    dQb = op.Qb;
                }
                float al[CPL][C], kf[CPL][C], qf[CPL][C];
                if constexpr (CPL == 2) {
                    float2 a2[C];
                    uint32_t kk[C], qq[C];
#pragma unroll
                    for (int t = 0; t < C; ++t) {
                        a2[t] = *reinterpret_cast<const float2*>(&raw.alpha[t * DK + 2 * lane]);
                        kk[t] = *reinterpret_cast<const uint32_t*>(&raw.k[t * DK + 2 * lane]);
                        qq[t] = CF::NOQ ? 0u : *reinterpret_cast<const uint32_t*>(&raw.q[t * DK + 2 * lane]);
                    }
#pragma unroll
                    for (int t = 0; t < C; ++t) {
                        al[0][t] = a2[t].x;
                        al[1][t] = a2[t].y;
                        kf[0][t] = __uint_as_float(kk[t] << 16);
                        kf[1][t] = __uint_as_float(kk[t] & 0xffff0000u);
                        qf[0][t] = __uint_as_float(qq[t] << 16);
                        qf[1][t] = __uint_as_float(qq[t] & 0xffff0000u);
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < C; ++t) {
                        al[0][t] = raw.alpha[t * DK + lane];
                        kf[0][t] = static_cast<float>(raw.k[t * DK + lane]);
                        qf[0][t] = CF::NOQ ? 0.f : static_cast<float>(raw.q[t * DK + lane]);
                    }
                }
                bf16 kb[CPL][C], qb[CPL][C], kl[CPL][C], ql[CPL][C];
                float xk[CPL][C], xq[CPL][C];
                // G_t / c with each channel's decay reference, taken as in the
                // builders from the same alphas: the plain product first, the
                // channels past 2^-100 recomputed (padded tokens: alpha = 1,
                // k = q = 0)
                bool slow[CPL];
#pragma unroll
                for (int e = 0; e < CPL; ++e) {
                    float G = 1.f;
#pragma unroll
                    for (int t = 0; t < C; ++t) {
                        const bool ok = FULL || t < nv;
                        G *= ok ? al[e][t] : 1.f;
                        xk[e][t] = ok ? kf[e][t] * G : 0.f;
                        xq[e][t] = ok ? qf[e][t] * G : 0.f;
                    }
                    slow[e] = !decay_plain_ok(G);
                }
                bool any_slow = false;
#pragma unroll
                for (int e = 0; e < CPL; ++e)
                    any_slow |= slow[e];
                if (__ballot(any_slow) != 0) {
#pragma unroll
                    for (int e = 0; e < CPL; ++e) {
                        if (slow[e]) {
                            float a1[C];
#pragma unroll
                            for (int t = 0; t < C; ++t)
                                a1[t] = (FULL || t < nv) ? raw.alpha[t * DK + CPL * lane + e] : 1.f;
                            const DecayRef ref = decay_ref(a1);
                            float G = __builtin_amdgcn_ldexpf(1.f, -ref.m);
#pragma unroll
                            for (int t = 0; t < C; ++t) {
                                const bool ok = FULL || t < nv;
                                G *= decay_alpha(ref, a1[t]);
                                xk[e][t] = ok ? kf[e][t] * G : 0.f;
                                xq[e][t] = ok ? qf[e][t] * G : 0.f;
                            }
                        }
                    }
                }
#pragma unroll
                for (int e = 0; e < CPL; ++e) {
#pragma unroll
                    for (int t = 0; t < C; t += 4) {
                        const f32x4 k4{xk[e][t], xk[e][t + 1], xk[e][t + 2], xk[e][t + 3]};
                        const f32x4 q4{xq[e][t], xq[e][t + 1], xq[e][t + 2], xq[e][t + 3]};
                        bf16x4 kh, qh, klo, qlo;
                        if constexpr (CF::X3) {
                            split4(k4, kh, klo);
                            split4(q4, qh, qlo);
                        } else {
                            kh = cvt4(k4);
                            qh = cvt4(q4);
                        }
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            kb[e][t + j] = kh[j];
                            qb[e][t + j] = qh[j];
                            if constexpr (CF::X3) {
                                kl[e][t + j] = klo[j];
                                ql[e][t + j] = qlo[j];
                            }
                        }
                    }
                }
                // token-quad writes: the lane's channels are adjacent, so the
                // four tokens of each sit in one 8 * CPL byte run
                auto put = [&](bf16* dst, const bf16 (&x)[CPL][C], int tq) KDN_INLINE {
                    const int o = tq * QS + CPL * lane * 4;
                    if constexpr (CPL == 2) {
                        *reinterpret_cast<bf16x8*>(dst + o) =
                            bf16x8{x[0][4 * tq], x[0][4 * tq + 1], x[0][4 * tq + 2], x[0][4 * tq + 3],
                                   x[1][4 * tq], x[1][4 * tq + 1], x[1][4 * tq + 2], x[1][4 * tq + 3]};
                    } else {
                        *reinterpret_cast<bf16x4*>(dst + o) =
                            bf16x4{x[0][4 * tq], x[0][4 * tq + 1], x[0][4 * tq + 2], x[0][4 * tq + 3]};
                    }
                };
#pragma unroll
                for (int tq = 0; tq < 4; ++tq) {
                    put(dKb, kb, tq);
                    if constexpr (!CF::NOQ)
                        put(dQb, qb, tq);
                    if constexpr (CF::X3) {
                        put(dKl, kl, tq);
                        if constexpr (!CF::NOQ)
                            put(dQl, ql, tq);
                    }
                }
            };
            for (int c = -LR; c < nchunks; ++c) {
                const int X = c + LB;
                if (X >= 0 && X < nchunks) {
                    if (n_valid(X) == C)
                        build(std::integral_constant<bool, true>{}, X);
                    else
                        build(std::integral_constant<bool, false>{}, X);
                }
                lds_barrier();
            }
        }
    } else if constexpr (ISO) {
        // ============ isotropic wave: DK / 64 channels per lane ============
        // Per token t of chunk c + 4: a_t = mean_i alpha_t,i^2 and
        // |k_t|^2, then the scalar variance recurrence; b^_t goes to the
        // builders.  Lane l sums channels CPL l .. CPL l + CPL - 1 of every
        // token; a transpose-reduce over the lanes leaves one token's totals
        // per lane (four lanes per token).
        constexpr int CPL = DK / 64;
        static_assert(CPL == 1 || CPL == 2, "channels per lane");
        static_assert(C == 16, "reduction tree shape");
        // Halving steps: a lane keeps half of its token slots and adds the
        // partner lane's partials of them.  Distances 32 and 16 exchange
        // slots with v_permlane32_swap / v_permlane16_swap (after the swap
        // both registers of a lane hold partials of the same token); the
        // in-row steps pair lanes through DPP row_mirror (l <-> 15 - l) and
        // row_half_mirror (l <-> 7 - l), then a quad reduction finishes.
        auto swap32 = [](float& x, float& y) {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y),
                                                            false, false);
            x = __uint_as_float(r[0]);
            y = __uint_as_float(r[1]);
        };
        auto swap16 = [](float& x, float& y) {
            const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y),
                                                            false, false);
            x = __uint_as_float(r[0]);
            y = __uint_as_float(r[1]);
        };
        auto dpp = [](float x, auto ctrl_tag) {
            constexpr int CTRL = decltype(ctrl_tag)::value;
            return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
        };
        using MIRROR = std::integral_constant<int, 0x140>;
        using HALF_MIRROR = std::integral_constant<int, 0x141>;
        using QP_1032 = std::integral_constant<int, 0xb1>;  // quad_perm [1,0,3,2]
        using QP_2301 = std::integral_constant<int, 0x4e>;  // quad_perm [2,3,0,1]
        const bool up3 = (lane & 8) != 0, up2 = (lane & 4) != 0;
        // v[16] -> one value per lane; every lane's slots go through the
        // same network, so the token a lane ends with is fixed
        auto reduce = [&](float (&v)[C]) KDN_INLINE {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                swap32(v[j], v[j + 8]);
                v[j] += v[j + 8];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                swap16(v[j], v[j + 4]);
                v[j] += v[j + 4];
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float keep = up3 ? v[j + 2] : v[j], send = up3 ? v[j] : v[j + 2];
                v[j] = keep + dpp(send, MIRROR{});
            }
            {
                const float keep = up2 ? v[1] : v[0], send = up2 ? v[0] : v[1];
                v[0] = keep + dpp(send, HALF_MIRROR{});
            }
            float x = v[0];
            x += dpp(x, QP_1032{});
            x += dpp(x, QP_2301{});
            return x;
        };
        // the token each lane ends with: run the token numbers through the
        // same exchanges; tok_lane[t] is a lane holding token t
        int tok_lane[C], mine_i;
        {
            float id[C];
#pragma unroll
            for (int t = 0; t < C; ++t)
                id[t] = (float)t;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                swap32(id[j], id[j + 8]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                swap16(id[j], id[j + 4]);
            const float mine = up2 ? (up3 ? id[3] : id[1]) : (up3 ? id[2] : id[0]);
            mine_i = (int)mine;
#pragma unroll
            for (int t = 0; t < C; ++t)
                tok_lane[t] = __builtin_amdgcn_readfirstlane(
                    (int)__builtin_ctzll(__ballot(mine_i == t)));
        }
        const float inv_dk = 1.f / (float)DK;
        // homogeneous variance b = n / d (see the Diagonal builders):
        //   n_t = a_t n_{t-1} + omega_t d_{t-1},  d_t = d_{t-1} + u_t n_t,
        //   u_t = mu |k_t|^2 / (d_k r_t),  b^_t = n_t / d_{t-1}
        float nn = a.var0 ? a.var0[bh] : var_init, dd = 1.f;
        for (int c = -LR; c < nchunks; ++c) {
            const int X = c + LB + 1;
            if (X >= 0 && X < nchunks) {
                const int nv = n_valid(X);
                const auto& st = sm.raw[X % NRAW];
                // all reads first (kept ahead of the arithmetic), then the
                // per-lane partial sums
                float sa[C], sk[C];
                if constexpr (CPL == 2) {
                    float2 al[C];
                    uint32_t kk[C];
#pragma unroll
                    for (int t = 0; t < C; ++t) {
                        al[t] = *reinterpret_cast<const float2*>(&st.alpha[t * DK + 2 * lane]);
                        kk[t] = *reinterpret_cast<const uint32_t*>(&st.k[t * DK + 2 * lane]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int t = 0; t < C; ++t) {
                        const float k0 = __uint_as_float(kk[t] << 16);
                        const float k1 = __uint_as_float(kk[t] & 0xffff0000u);
                        sa[t] = fmaf(al[t].x, al[t].x, al[t].y * al[t].y);
                        sk[t] = fmaf(k0, k0, k1 * k1);
                    }
                } else {
                    float al[C];
                    bf16 kv[C];
#pragma unroll
                    for (int t = 0; t < C; ++t) {
                        al[t] = st.alpha[t * DK + lane];
                        kv[t] = st.k[t * DK + lane];
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int t = 0; t < C; ++t) {
                        const float kf = static_cast<float>(kv[t]);
                        sa[t] = al[t] * al[t];
                        sk[t] = kf * kf;
                    }
                }
                const float ta = reduce(sa), tk = reduce(sk);
                // per-token inputs of the recurrence, each formed in a lane
                // holding that token (padded tokens of a ragged chunk are
                // identities: a = 1, u = 0, omega = 0)
                const bool okl = mine_i < nv;
                const float rl = sm.rr[X % NRING][mine_i], wl = sm.wr[X % NRING][mine_i];
                const float al = okl ? ta * inv_dk : 1.f;
                const float ul = okl ? mu * tk * rcp((float)DK * rl) : 0.f;
                const float wo = okl ? wl : 0.f;
                // serial recurrence on wave-uniform values
                float bhv[C];
#pragma unroll
                for (int t = 0; t < C; ++t) {
                    const float at = bcast(al, tok_lane[t]);
                    const float ut = bcast(ul, tok_lane[t]);
                    const float wt = bcast(wo, tok_lane[t]);
                    const float dprev = dd;
                    nn = fmaf(at, nn, wt * dd);
                    dd = fmaf(ut, nn, dd);
                    bhv[t] = nn * rcp(dprev);
                    if ((t & 3) == 3) {
                        // exact power-of-two rescale of both coordinates
                        const int e = __builtin_amdgcn_frexp_expf(dd);
                        nn = __builtin_ldexpf(nn, -e);
                        dd = __builtin_ldexpf(dd, -e);
                    }
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
        const float bvar = nn / dd;
        if (tile == 0 && lane == 0)
            a.var_T[bh] = bvar;
    }
}

template <typename CF>
static hipError_t launch_cfg(const FwdArgs& a, hipStream_t stream)
{
    using SM = std::conditional_t<CF::X3, SmemX3<CF>, Smem<CF>>;
    auto kern = kdn_walk_fwd_kernel<CF>;
    const size_t smem = sizeof(SM);
    hipError_t e = set_lds_limit_once(kern, smem);
    if (e != hipSuccess)
        return e;
    const int nblk = a.B * a.H * (a.dv / CF::DVT);
    hipLaunchKernelGGL(kern, dim3(nblk), dim3(64 * CF::NWAVES), smem, stream, a);
    return hipGetLastError();
}

}  // namespace walk

namespace walk {

// state-only walks: SO = 1 (no q, no o) or 2 (also v = 0)
template <int SO>
static hipError_t launch_state_only(const FwdArgs& a, bool iso, hipStream_t stream)
{
    if (iso)
        return a.dk == 128 ? launch_cfg<Cfg<128, 2, 2, true, false, false, SO>>(a, stream)
                           : launch_cfg<Cfg<64, 2, 2, true, false, false, SO>>(a, stream);
    if (a.split)
        return a.dk == 128 ? launch_cfg<Cfg<128, 2, 2, false, true, false, SO>>(a, stream)
                           : launch_cfg<Cfg<64, 2, 2, false, true, false, SO>>(a, stream);
    return a.dk == 128 ? launch_cfg<Cfg<128, 2, 2, false, false, false, SO>>(a, stream)
                       : launch_cfg<Cfg<64, 2, 2, false, false, false, SO>>(a, stream);
}

}  // namespace walk

hipError_t launch_walk_fwd(const FwdArgs& a, bool iso, hipStream_t stream)
{
    using namespace walk;
    // chunk-start states: the split-product Diagonal state-only walk only
    if (a.ckpt && (iso || !a.split || a.state_only != 1 || a.a_pre))
        return hipErrorInvalidValue;
    if (a.a_pre) {
        if (a.state_only || a.o_f32)
            return hipErrorInvalidValue;
        if (iso)
            return a.dk == 128 ? launch_cfg<Cfg<128, 2, 2, true, false, false, 0, 1>>(a, stream)
                               : launch_cfg<Cfg<64, 2, 2, true, false, false, 0, 1>>(a, stream);
        if (!a.w_pre)
            return hipErrorInvalidValue;
        if (a.split)
            return a.dk == 128 ? launch_cfg<Cfg<128, 2, 2, false, true, false, 0, 2>>(a, stream)
                               : launch_cfg<Cfg<64, 2, 2, false, true, false, 0, 2>>(a, stream);
        return a.dk == 128 ? launch_cfg<Cfg<128, 2, 2, false, false, false, 0, 2>>(a, stream)
                           : launch_cfg<Cfg<64, 2, 2, false, false, false, 0, 2>>(a, stream);
    }
    if (a.state_only == 1)
        return launch_state_only<1>(a, iso, stream);
    if (a.state_only == 2)
        return launch_state_only<2>(a, iso, stream);
    if (iso)
        return a.dk == 128 ? launch_cfg<Cfg<128, 2, 2, true>>(a, stream)
                           : launch_cfg<Cfg<64, 2, 2, true>>(a, stream);
    if (a.split && a.o_f32)
        return a.dk == 128 ? launch_cfg<Cfg<128, 2, 2, false, true, true>>(a, stream)
                           : launch_cfg<Cfg<64, 2, 2, false, true, true>>(a, stream);
    if (a.split)
        return a.dk == 128 ? launch_cfg<Cfg<128, 2, 2, false, true>>(a, stream)
                           : launch_cfg<Cfg<64, 2, 2, false, true>>(a, stream);
    return a.dk == 128 ? launch_cfg<Cfg<128, 2, 2, false>>(a, stream)
                       : launch_cfg<Cfg<64, 2, 2, false>>(a, stream);
}

}  // namespace kdn
