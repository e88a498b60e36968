// kdn_common.h -- device-side helpers shared by the KDN kernels (gfx950).
//
// Matrix-core conventions used throughout (CDNA 16x16 MFMA, wave64):
//   accumulator D (16x16 fp32, 4 values per lane): lane l holds
//       D[4*(l>>4) + r][l & 15],  r = 0..3
//   "NT" operands: A is [16 rows][K], B is [16 rows][K], both with K
//   contiguous, so that acc[m][n] += sum_k A[m][k] * B[n][k].
//     bf16 16x16x32: lane l reads A[l&15][8*(l>>4) .. +7]  (one 16-byte read)
//     bf16 16x16x16: lane l reads A[l&15][4*(l>>4) .. +3]  (one 8-byte read)
//     fp32 16x16x4:  lane l reads A[l&15][l>>4]
//   (same pattern for B with its own rows).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// Fast reciprocal (v_rcp_f32, ~1 ulp).
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Gates from their pre-activations (KDN reading notes, method part §8:
// alpha = sigmoid(a), omega = softplus(w), r = r_min + softplus(rho)).  Every
// kernel that forms a gate calls these, written with explicit hardware
// operations (v_exp_f32 / v_log_f32 are base 2, ~1 ulp each) and no
// multiply-add the compiler could contract, so that the separate gate pass
// and the forward that reads pre-activations itself produce the same bits.
//   sigmoid(x) = 1 / (1 + 2^(-x log2 e)), saturating to 0 or 1;
//   softplus(x) = max(x, 0) + log1p(e), e = 2^(-|x| log2 e) in (0, 1], which
//   equals log(1 + e^x) without overflow.  log1p(e) is log(u) e / (u - 1) with
//   u = 1 + e (Goldberg, "What every computer scientist should know about
//   floating-point arithmetic", Thm. 4): u - 1 is exact and the ratio cancels
//   the rounding of u, so small e keeps its relative accuracy; u == 1 gives e.
constexpr float kLog2e = 1.44269504088896341f, kLn2 = 0.693147180559945309f;
__device__ __forceinline__ float gate_sigmoid(float x)
{
    return rcp(1.f + __builtin_amdgcn_exp2f(x * -kLog2e));
}
__device__ __forceinline__ float gate_softplus(float x, float add)
{
    const float e = __builtin_amdgcn_exp2f(fabsf(x) * -kLog2e);
    const float u = 1.f + e;
    const float l1p = u == 1.f ? e : (__builtin_amdgcn_logf(u) * kLn2) * (e * rcp(u - 1.f));
    return (add + fmaxf(x, 0.f)) + l1p;
}
// a bf16 value held in the low 16 bits of a 32-bit word, widened to fp32
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t w) { return __uint_as_float(w << 16); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Decay reference of one 16-token chunk and channel (chunked forward
// kernels).  The chunk products pair G_t / c with c / G_s (Kb, Qb against
// Ktp), so both must stay finite and normal for every t, s of the chunk,
// G_t in [G_15, 1].  L = sum_t (e_t - 1), with e_t
// the binary exponent of alpha_t, is an integer with 2^L <= G_15 < 2^(L + 16).
//   L >= -100:  c = 1 (G_t and 1 / G_t within 2^100 of one);
//   else:       c = 2^ceil(L / 2), which puts G_t / c and c / G_t within
//               2^(L / 2) of one, at most 2^112 away for L >= -224;
//   L < -224:   the chunk decays by more than fp32 can span; every alpha of the
//               channel below 2^-14 is raised to 2^-14 for the memory decay
//               (the variance recurrence keeps the true alpha), which brings
//               L to -224 or above and perturbs the state by at most 2^-14 of
//               its previous value per raised token.
// An alpha below 2^-120 (zero included) counts as below the floor.  The rule
// applies where the chunk's plain fp32 product of alphas (multiplied in token
// order from 1) is below 2^-100 (decay_plain_ok); elsewhere c = 1, which the
// kernels take without evaluating L.
constexpr float kAlphaFloor = 0x1p-14f;
constexpr int kLFree = -100, kLFloor = -224, kEFloor = -14;
__device__ __forceinline__ int decay_lb(float a)
{
    return a >= 0x1p-120f ? __builtin_amdgcn_frexp_expf(a) - 1 : -1000;
}
struct DecayRef {
    bool floor;  // alphas raised to kAlphaFloor for the memory decay
    int m;       // c = 2^m, m <= 0
};
template <int N>
__device__ __forceinline__ DecayRef decay_ref(const float (&al)[N])
{
    static_assert(N == 16, "the bounds above assume 16 tokens");
    int L = 0;
#pragma unroll
    for (int t = 0; t < N; ++t)
        L += decay_lb(al[t]);
    DecayRef r{L < kLFloor, 0};
    if (r.floor) {
        L = 0;
#pragma unroll
        for (int t = 0; t < N; ++t)
            L += max(decay_lb(al[t]), kEFloor);
    }
    r.m = L >= kLFree ? 0 : -((-L) >> 1);
    return r;
}
__device__ __forceinline__ bool decay_plain_ok(float product) { return product >= 0x1p-100f; }
__device__ __forceinline__ float decay_alpha(const DecayRef& r, float a)
{
    return r.floor ? fmaxf(a, kAlphaFloor) : a;
}

// Order this wave's LDS writes before its later LDS reads (other lanes of the
// same wave read what a lane wrote).  No cross-wave effect.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// acc += A[16 x K] * B[16 x K]^T, operands in LDS (K contiguous, row strides
// lda / ldb in elements).  K must be a multiple of 16 (bf16) or 4 (fp32).
__device__ __forceinline__ void mma_nt(f32x4& acc, const bf16* A, int lda, const bf16* B,
                                       int ldb, int K, int lane)
{
    const int row = lane & 15;
    int k0 = 0;
    for (; k0 + 32 <= K; k0 += 32) {
        const int kk = k0 + 8 * (lane >> 4);
        bf16x8 a = *reinterpret_cast<const bf16x8*>(A + row * lda + kk);
        bf16x8 b = *reinterpret_cast<const bf16x8*>(B + row * ldb + kk);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
    for (; k0 + 16 <= K; k0 += 16) {
        const int kk = k0 + 4 * (lane >> 4);
        bf16x4 a = *reinterpret_cast<const bf16x4*>(A + row * lda + kk);
        bf16x4 b = *reinterpret_cast<const bf16x4*>(B + row * ldb + kk);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
    }
}

__device__ __forceinline__ void mma_nt(f32x4& acc, const float* A, int lda, const float* B,
                                       int ldb, int K, int lane)
{
    const int row = lane & 15, kq = lane >> 4;
    for (int k0 = 0; k0 < K; k0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[row * lda + k0 + kq],
                                                   B[row * ldb + k0 + kq], acc, 0, 0, 0);
}

// Two contractions sharing the B operand:  accA += A0 B^T,  accB += A1 B^T.
// All fragments of the K loop are read from LDS before the first MFMA is
// issued, so the LDS latency is paid once per call instead of once per MFMA.
template <int K>
__device__ __forceinline__ void mma2_nt(f32x4& acc0, f32x4& acc1, const bf16* A0,
                                        const bf16* A1, int lda, const bf16* B, int ldb,
                                        int lane)
{
    static_assert(K % 32 == 0, "K multiple of 32");
    constexpr int NK = K / 32;
    const int row = lane & 15, kg = 8 * (lane >> 4);
    bf16x8 a0[NK], a1[NK], b[NK];
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        b[k] = *reinterpret_cast<const bf16x8*>(B + row * ldb + 32 * k + kg);
        a0[k] = *reinterpret_cast<const bf16x8*>(A0 + row * lda + 32 * k + kg);
        a1[k] = *reinterpret_cast<const bf16x8*>(A1 + row * lda + 32 * k + kg);
    }
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[k], b[k], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[k], b[k], acc1, 0, 0, 0);
    }
}

template <int K>
__device__ __forceinline__ void mma2_nt(f32x4& acc0, f32x4& acc1, const float* A0,
                                        const float* A1, int lda, const float* B, int ldb,
                                        int lane)
{
    static_assert(K % 4 == 0, "K multiple of 4");
    constexpr int NK = K / 4;
    const int row = lane & 15, kq = lane >> 4;
    float a0[NK], a1[NK], b[NK];
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        b[k] = B[row * ldb + 4 * k + kq];
        a0[k] = A0[row * lda + 4 * k + kq];
        a1[k] = A1[row * lda + 4 * k + kq];
    }
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[k], b[k], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[k], b[k], acc1, 0, 0, 0);
    }
}

// Operand fragments of one K-step of a 16x16 MFMA, by element type:
//   bf16: 16x16x32 (K-step 32, 8 values per lane); fp32: 16x16x4 (K-step 4).
// frag(base, ld, k0, lane) reads rows (lane & 15) of a [16][K] operand.
template <typename T>
struct Frag;
template <>
struct Frag<bf16> {
    using type = bf16x8;
    static constexpr int KSTEP = 32;
    static __device__ __forceinline__ type load(const bf16* base, int ld, int k0, int lane)
    {
        return *reinterpret_cast<const bf16x8*>(base + (lane & 15) * ld + k0 + 8 * (lane >> 4));
    }
    static __device__ __forceinline__ void mma(f32x4& acc, const type& a, const type& b)
    {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
};
template <>
struct Frag<float> {
    using type = float;
    static constexpr int KSTEP = 4;
    static __device__ __forceinline__ type load(const float* base, int ld, int k0, int lane)
    {
        return base[(lane & 15) * ld + k0 + (lane >> 4)];
    }
    static __device__ __forceinline__ void mma(f32x4& acc, const type& a, const type& b)
    {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
};

// acc += A * X where A is a 16x16 operand in LDS (rows at A, K = 16
// contiguous) and X (K x N = 16 x 16) is an accumulator in D layout (lane
// holds X[4*(l>>4) + r][l & 15]).  For bf16 that layout is exactly the B
// operand of the 16x16x16 MFMA, so X never leaves registers (it is rounded to
// bf16, as any MFMA operand); fp32 takes a hop through `scratch` ([16][17]
// floats of wave-private LDS) because its 16x16x4 B layout differs.
template <typename T>
struct AccB;
template <>
struct AccB<bf16> {
    static __device__ __forceinline__ void mma(f32x4& acc, const bf16* A, int lda, const f32x4& x,
                                               float* scratch, int lane)
    {
        (void)scratch;
        const bf16x4 a = *reinterpret_cast<const bf16x4*>(A + (lane & 15) * lda + 4 * (lane >> 4));
        const bf16x4 b = bf16x4{static_cast<bf16>(x[0]), static_cast<bf16>(x[1]),
                                static_cast<bf16>(x[2]), static_cast<bf16>(x[3])};
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
    }
};
template <>
struct AccB<float> {
    static __device__ __forceinline__ void mma(f32x4& acc, const float* A, int lda, const f32x4& x,
                                               float* scratch, int lane)
    {
        const int g = lane >> 4, c = lane & 15;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            scratch[(4 * g + r) * 17 + c] = x[r];
        wave_lds_sync();
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[c * lda + k0 + g],
                                                       scratch[(k0 + g) * 17 + c], acc, 0, 0, 0);
        wave_lds_sync();
    }
};

// Same contraction with an fp32 A operand in LDS and a B operand of type T:
// for bf16 the A values are rounded to bf16 on the fly (K multiple of 16).
__device__ __forceinline__ void mma_nt_f32a(f32x4& acc, const float* A, int lda, const bf16* B,
                                            int ldb, int K, int lane)
{
    const int row = lane & 15;
    for (int k0 = 0; k0 < K; k0 += 16) {
        const int kk = k0 + 4 * (lane >> 4);
        f32x4 af = *reinterpret_cast<const f32x4*>(A + row * lda + kk);
        bf16x4 a = bf16x4{static_cast<bf16>(af[0]), static_cast<bf16>(af[1]),
                          static_cast<bf16>(af[2]), static_cast<bf16>(af[3])};
        bf16x4 b = *reinterpret_cast<const bf16x4*>(B + row * ldb + kk);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
    }
}

__device__ __forceinline__ void mma_nt_f32a(f32x4& acc, const float* A, int lda, const float* B,
                                            int ldb, int K, int lane)
{
    mma_nt(acc, A, lda, B, ldb, K, lane);
}

// Store 4 consecutive values (a transposed accumulator column) as T.
__device__ __forceinline__ void store4(bf16* p, f32x4 v)
{
    *reinterpret_cast<bf16x4*>(p) = bf16x4{static_cast<bf16>(v[0]), static_cast<bf16>(v[1]),
                                           static_cast<bf16>(v[2]), static_cast<bf16>(v[3])};
}
__device__ __forceinline__ void store4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// ---------------------------------------------------------------------------
// 2x2 Moebius maps on homogeneous variance coordinates [n; d] (p = n / d).
// The per-token factor is M = [[a, w], [u a, 1 + u w]] (predict with decay
// a = alpha^2 and process noise w, then the information-scaled update with
// u = mu k^2 / r).  Products compose by LEFT multiplication in token order and
// are rescaled by 1 / max|entry| (all entries are >= 0, and the rescale keeps
// every ratio n / d), so fp32 never overflows.
// ---------------------------------------------------------------------------
struct Mob {
    float m00, m01, m10, m11;
};

__device__ __forceinline__ Mob mob_identity() { return Mob{1.f, 0.f, 0.f, 1.f}; }

// later o earlier  (apply `earlier` first)
__device__ __forceinline__ Mob mob_compose(const Mob& later, const Mob& earlier)
{
    Mob r;
    r.m00 = later.m00 * earlier.m00 + later.m01 * earlier.m10;
    r.m01 = later.m00 * earlier.m01 + later.m01 * earlier.m11;
    r.m10 = later.m10 * earlier.m00 + later.m11 * earlier.m10;
    r.m11 = later.m10 * earlier.m01 + later.m11 * earlier.m11;
    const float mx = fmaxf(fmaxf(r.m00, r.m01), fmaxf(r.m10, r.m11));
    const float s = rcp(mx);
    r.m00 *= s;
    r.m01 *= s;
    r.m10 *= s;
    r.m11 *= s;
    return r;
}

__device__ __forceinline__ float mob_apply(const Mob& m, float x)
{
    return (m.m00 * x + m.m01) * rcp(m.m10 * x + m.m11);
}

// DPP lane moves (GFX9 encodings).  `old` is returned for lanes whose source
// is outside the pattern, so passing the identity makes those lanes neutral.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_mov(float old, float src)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                           __builtin_bit_cast(int, src), CTRL, ROW_MASK, 0xf,
                                           false));
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ Mob mob_dpp(const Mob& src)
{
    const Mob id = mob_identity();
    return Mob{dpp_mov<CTRL, ROW_MASK>(id.m00, src.m00), dpp_mov<CTRL, ROW_MASK>(id.m01, src.m01),
               dpp_mov<CTRL, ROW_MASK>(id.m10, src.m10), dpp_mov<CTRL, ROW_MASK>(id.m11, src.m11)};
}

// Inclusive wave64 scan of Moebius maps in lane order: lane l ends with
// M_l o M_{l-1} o ... o M_0.  Six DPP steps: row_shr 1/2/4/8 inside each row
// of 16 lanes, then row_bcast 15 and row_bcast 31 across rows.
__device__ __forceinline__ Mob mob_wave_scan_inclusive(Mob x)
{
    x = mob_compose(x, mob_dpp<0x111, 0xf>(x));  // row_shr:1
    x = mob_compose(x, mob_dpp<0x112, 0xf>(x));  // row_shr:2
    x = mob_compose(x, mob_dpp<0x114, 0xf>(x));  // row_shr:4
    x = mob_compose(x, mob_dpp<0x118, 0xf>(x));  // row_shr:8
    x = mob_compose(x, mob_dpp<0x142, 0xa>(x));  // row_bcast:15 -> rows 1, 3
    x = mob_compose(x, mob_dpp<0x143, 0xc>(x));  // row_bcast:31 -> rows 2, 3
    return x;
}

// Exclusive version: lane l gets M_{l-1} o ... o M_0 (identity at lane 0).
__device__ __forceinline__ Mob mob_wave_shift_right(const Mob& x)
{
    return mob_dpp<0x138, 0xf>(x);  // wave_shr:1
}

}  // namespace kdn
