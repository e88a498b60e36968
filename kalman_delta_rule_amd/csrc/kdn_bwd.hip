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
// Three stages, all fp32 arithmetic whatever the io type (divisions in the
// gain recurrences through the hardware reciprocal, as in the forward):
//   A  gain forward recompute by the chunk-parallel Moebius gain scan
//      (kdn_gain.hip): kap_t, p_{t-1} and r + z_t (Isotropic: beta_t, b_{t-1},
//      mean alpha^2, |k|^2) for every token.
//   B  memory backward.  With dv a multiple of 64 in 16-token chunks on the
//      matrix cores (kdn_bwd_chunk.hip; for Diagonal with bf16 io its
//      chunk-start states come from the state-only forward walk, and few-head
//      long shapes split over the sequence, kdn_seqpar.hip).  Otherwise token
//      by token here: one 256-thread workgroup per (b,h) and 16-column
//      block of the value dimension (the columns of S evolve independently
//      given the gain).  A forward pass stores S every 16 tokens and every
//      token's innovations; then for each 16-token chunk, last first, the
//      chunk's 17 states are recomputed into registers (no reduction: the
//      innovations are known) and walked backwards.  dv is complete per column and
//      written here; the four row vectors that sum over all columns (dq, kapbar,
//      dk and dalpha of the memory) are written as per-block partials.
//   C  partial merge (dq and the summed row vectors; the chunked path's own
//      finishing kernel does this), then the variance
//      recurrence's adjoint as a chunked affine scan (summaries, carry,
//      replay), writing dk, dalpha, domega, dr and the initial variance's and
//      information scale's gradients.
// Each thread of B owns one row of S (one key channel) and 8 (d_k = 128) or 4
// (d_k = 64) columns, so row reductions stay in a lane pair or quad and the
// column reductions (delta in the forward pass, delbar in the reverse walk)
// cross the workgroup through LDS once per token.
#include "kdn_common.h"
#include "kdn_internal.h"
#include "kdn_ops.h"

namespace kdn {


// Lane exchanges in the vector ALU (no LDS round trip).  xor_lane<M>(x) is
// x of lane l ^ M, for M = 1, 2 (quad permutes) and 4, 8 (a row shift one way
// for the lanes whose bit M is clear, the other way for the rest, chosen by
// the bank mask: banks are the four 4-lane groups of a 16-lane row).
// add_xor<M>(x) = x + (x of lane l ^ M); M = 16 and 32 use gfx950's row-pair
// and half swaps of two registers holding x, after which each lane holds its
// own value in one register and its partner's in the other.  Every stage adds a pair commutatively, so a
// butterfly leaves bitwise-identical sums in all lanes of a group.
template <int CTRL, int BANK>
__device__ __forceinline__ float dpp_sel(float old, float src)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                 __builtin_bit_cast(int, src),
                                                                 CTRL, 0xF, BANK, false));
}

template <int M>
__device__ __forceinline__ float xor_lane(float x)
{
    if constexpr (M == 1)
        return dpp_sel<0xB1, 0xF>(x, x);  // quad_perm [1,0,3,2]
    else if constexpr (M == 2)
        return dpp_sel<0x4E, 0xF>(x, x);  // quad_perm [2,3,0,1]
    else if constexpr (M == 4)            // row_shl:4 on banks 0, 2; row_shr:4 on banks 1, 3
        return dpp_sel<0x114, 0xA>(dpp_sel<0x104, 0x5>(x, x), x);
    else                                  // row_shl:8 on banks 0, 1; row_shr:8 on banks 2, 3
        return dpp_sel<0x118, 0xC>(dpp_sel<0x108, 0x3>(x, x), x);
}

template <int M>
__device__ __forceinline__ float add_xor(float x)
{
    if constexpr (M <= 8) {
        return x + xor_lane<M>(x);
    } else {
        // The swap writes both of its registers; it is issued from inline
        // assembly because the compiler's builtin for it returns only the first
        // one here.  The s_nop padding keeps it clear of any VALU hazard, since
        // the compiler does not look inside the assembly.
        float a = x, b = x;
        if constexpr (M == 16)
            asm volatile("s_nop 4\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 4"
                         : "+v"(a), "+v"(b));
        else
            asm volatile("s_nop 4\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 4"
                         : "+v"(a), "+v"(b));
        return a + b;
    }
}

// Sum over the lanes whose index differs in bits log2(LO) .. 5 (LO = 1: the
// whole wave).
template <int LO>
__device__ __forceinline__ float sum_lanes_from(float x)
{
    if constexpr (LO <= 1)
        x = add_xor<1>(x);
    if constexpr (LO <= 2)
        x = add_xor<2>(x);
    if constexpr (LO <= 4)
        x = add_xor<4>(x);
    if constexpr (LO <= 8)
        x = add_xor<8>(x);
    if constexpr (LO <= 16)
        x = add_xor<16>(x);
    return add_xor<32>(x);
}

__device__ __forceinline__ float wave_sum(float x) { return sum_lanes_from<1>(x); }

// One reduce-scatter step over lane pairs l, l ^ M: of the first N values,
// the lane whose bit M is clear keeps the lower half and the other lane the
// upper half, each adding its partner's copy; v[0 .. N/2) hold the result.
template <int M, int N, int S>
__device__ __forceinline__ void rs_step(float (&v)[S], bool upper)
{
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        const float keep = upper ? v[i + N / 2] : v[i];
        const float send = upper ? v[i] : v[i + N / 2];
        v[i] = keep + xor_lane<M>(send);
    }
}

// ---------------------------------------------------------------------------
// A: gain forward recompute -- the chunk-parallel Moebius gain scan of
// kdn_gain.hip (summaries, carry, replay), asked for the backward's outputs
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// B: memory backward
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Direct global -> LDS copy of 16 (4) bytes per lane: lane l's bytes from
// its own global address land at LDS byte address lds + 16 l (4 l) (lds
// uniform).  Completion is tracked by vmcnt.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds)
{
    __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)(size_t)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, uint32_t lds)
{
    __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)(size_t)lds, 4, 0, 0);
}

__device__ __forceinline__ uint32_t lds_u32(const void* p)
{
    return (uint32_t)(size_t)(const lds_void_t*)p;
}

// A barrier that orders LDS only: global loads and stores stay in flight.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Every copy and store this wave issued has completed, then a barrier: after
// it, the whole workgroup's copies into LDS are visible.  The wait is the
// builtin (not inline assembly) so the compiler's own counter model sees that
// nothing is outstanding afterwards.
__device__ __forceinline__ void copies_landed_barrier()
{
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("s_barrier" ::: "memory");
}

// One 16-token chunk of inputs, staged in LDS.  Rows past a ragged chunk's
// end repeat its last row and are never read.
template <typename IO, bool ISO, int DK>
struct BwdStage {
    float al[BWD_L * DK];                  // alpha
    float kp[ISO ? BWD_L : BWD_L * DK];    // kappa (Diagonal) / beta (Isotropic)
    IO kk[BWD_L * DK];                     // k
    IO qq[BWD_L * DK];                     // q (reverse pass only)
    IO vv[BWD_L * BWD_COLS];               // v, this block's columns
    IO dd[BWD_L * BWD_COLS];               // dL/do, this block's columns (reverse only)
    float dl[BWD_L * BWD_COLS];            // innovations delta, this block's columns (reverse only)
    float ck[DK * BWD_COLS];               // the state at the chunk start (reverse only)
};

// Copies of one 16-token chunk into stage s: tok0 is the chunk's first token
// index in [B,T,H] order (tokens step by H), rows past `last` repeat row
// `last`.  Piece p of an array (16 bytes) is copied by thread p + off, whole
// waves active or idle, so each wave's LDS base is uniform.
struct StageSrc {
    const float* dlt;  // this (head, block)'s innovations from the chunk's first token
    const float* ck;   // this (head, block)'s state at the chunk start, [dk][16]
    const float* alpha;
    const float* kap;
    const float* gsc;
    const void* k;
    const void* q;
    const void* v;
    const void* go;
    int H, dv;
};

template <typename IO, bool ISO, int DK>
__device__ __forceinline__ void bwd_stage_copy(BwdStage<IO, ISO, DK>& s, StageSrc a,
                                               size_t tok0, int last, int blk, int tid,
                                               bool rev)
{
    constexpr int L = BWD_L, EK = 16 / (int)sizeof(IO);
    const int lane = tid & 63;
    const size_t H = (size_t)a.H, dv = (size_t)a.dv;
    // alpha (and Diagonal kappa): L * DK / 4 pieces
#pragma unroll
    for (int p0 = 0; p0 < L * DK / 4; p0 += 256) {
        const int p = p0 + tid;
        if (p < L * DK / 4) {
            const int e = p * 4, tau = min(e / DK, last);
            const size_t g = (tok0 + tau * H) * DK + e % DK;
            const uint32_t off = (uint32_t)(p - lane) * 16u;
            dma16(a.alpha + g, lds_u32(s.al) + off);
            if constexpr (!ISO)
                dma16(a.kap + g, lds_u32(s.kp) + off);
        }
    }
    if constexpr (ISO) {
        if (tid < L)  // first wave
            dma4(a.gsc + (tok0 + min(lane, last) * H) * 4, lds_u32(s.kp));
    }
    // k and q: L * DK / EK pieces
    const IO* kg = reinterpret_cast<const IO*>(a.k);
    const IO* qg = reinterpret_cast<const IO*>(a.q);
#pragma unroll
    for (int p0 = 0; p0 < L * DK / EK; p0 += 256) {
        const int p = p0 + tid;
        if (p < L * DK / EK) {
            const int e = p * EK, tau = min(e / DK, last);
            const size_t g = (tok0 + tau * H) * DK + e % DK;
            const uint32_t off = (uint32_t)(p - lane) * 16u;
            dma16(kg + g, lds_u32(s.kk) + off);
            if (rev)
                dma16(qg + g, lds_u32(s.qq) + off);
        }
    }
    // v and dL/do, this block's columns: L * 16 / EK pieces (32 or 64), by
    // the second and third waves
    constexpr int PV = L * BWD_COLS / EK;
    static_assert(PV <= 64, "one wave copies a chunk of v");
    const int pv = tid - 64, pd = tid - 128;
    if (pv >= 0 && pv < PV) {
        const int e = pv * EK, tau = min(e / BWD_COLS, last);
        const size_t g = (tok0 + tau * H) * dv + (size_t)blk * BWD_COLS + e % BWD_COLS;
        dma16(reinterpret_cast<const IO*>(a.v) + g, lds_u32(s.vv));
    }
    if (rev && pd >= 0 && pd < PV) {
        const int e = pd * EK, tau = min(e / BWD_COLS, last);
        const size_t g = (tok0 + tau * H) * dv + (size_t)blk * BWD_COLS + e % BWD_COLS;
        dma16(reinterpret_cast<const IO*>(a.go) + g, lds_u32(s.dd));
    }
    // the innovations the forward pass stored, 16 floats per token, contiguous
    // per (head, block): 64 pieces, by the fourth wave
    const int pl = tid - 192;
    if (rev && pl >= 0 && pl < L * BWD_COLS / 4) {
        const int e = pl * 4, tau = min(e / BWD_COLS, last);
        dma16(a.dlt + (size_t)tau * BWD_COLS + e % BWD_COLS, lds_u32(s.dl));
    }
    // the checkpoint, DK * 16 floats in the same [row][column] order
    if (rev) {
#pragma unroll
        for (int p0 = 0; p0 < DK * BWD_COLS / 4; p0 += 256) {
            const int p = p0 + tid;
            if (p < DK * BWD_COLS / 4)
                dma16(a.ck + (size_t)p * 4, lds_u32(s.ck) + (uint32_t)(p - lane) * 16u);
        }
    }
}

template <typename IO, bool ISO, int DK>
__global__ __launch_bounds__(256, 2) void kdn_bwd_mem_kernel(BwdArgs args)
{
    // kernel arguments copied to locals once: nothing below reads them through
    // a pointer
    const BwdArgs a = args;
    const StageSrc src{nullptr, nullptr, a.alpha, a.kap, a.gsc, a.k, a.q, a.v, a.go, a.H, a.dv};
    float* const part = a.part;
    float* const ckpt = a.ckpt;
    constexpr int TPR = 256 / DK;        // threads per row of S
    static_assert(TPR == 2 || TPR == 4, "row split");
    constexpr int CPT = BWD_COLS / TPR;  // columns per thread
    constexpr int L = BWD_L;
    typedef BwdStage<IO, ISO, DK> Stage;
    // Copies land in stL while the steps read stR; at each chunk boundary stL
    // is moved to stR.  Two distinct arrays let the compiler see that the
    // steps' LDS reads never depend on copies in flight, with one instance of
    // the step code (the kernel's loops stay small for the instruction cache).
    __shared__ __align__(16) Stage stL;
    __shared__ __align__(16) Stage stR;
    __shared__ float red[2][4][BWD_COLS];

    const int blk = blockIdx.x, nblk = gridDim.x, bh = blockIdx.y;
    const int H = a.H, T = a.T, dv = a.dv;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = tid / TPR, cp = tid % TPR;
    const int cb = cp * CPT;                // first column of this thread in the block
    const int col0 = blk * BWD_COLS + cb;   // ... in the value dimension
    const int nch = (T + L - 1) / L;
    const size_t ntok = (size_t)a.B * T * H;
    IO* dvg = reinterpret_cast<IO*>(a.gv);
    // this (head, block)'s innovations, 16 per token, stored by the forward pass
    float* const dlt_wg = a.dlt + ((size_t)bh * nblk + blk) * (size_t)T * BWD_COLS;
    float* const ck_wg = ckpt + ((size_t)bh * nblk + blk) * nch * (DK * BWD_COLS);
    float* ck = ckpt + ((size_t)bh * nblk + blk) * nch * (DK * BWD_COLS) + row * BWD_COLS + cb;
    auto tok_of = [&](int t) __attribute__((always_inline)) { return ((size_t)b * T + t) * H + h; };

    auto stage_copy = [&](Stage& st, int c, bool rev) __attribute__((always_inline)) {
        StageSrc sc = src;
        sc.dlt = dlt_wg + (size_t)c * L * BWD_COLS;
        sc.ck = ck_wg + (size_t)c * (DK * BWD_COLS);
        bwd_stage_copy<IO, ISO, DK>(st, sc, tok_of(c * L), min(L, T - c * L) - 1, blk, tid, rev);
    };

    int slot = 0;
    // sum over all rows of the block, per column; every thread gets the sums
    // of its CPT columns.  The two LDS slots alternate so the next call's
    // writes never meet this call's reads.
    auto col_sum = [&](float (&x)[CPT]) __attribute__((always_inline)) {
        // reduce-scatter over the row bits below 16 (each lane ends with one
        // of its CPT columns summed over 8 or 4 lanes), all-reduce over lane
        // bits 4 and 5, then across the four waves through LDS
        float v[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j)
            v[j] = x[j];
        int jl = 0;
        if constexpr (TPR == 2) {
            const bool b1 = (lane & 2) != 0;
            rs_step<2, 8>(v, b1);
            jl += b1 ? 4 : 0;
        }
        const bool b2 = (lane & 4) != 0, b3 = (lane & 8) != 0;
        rs_step<4, 4>(v, b2);
        rs_step<8, 2>(v, b3);
        jl += (b2 ? 2 : 0) + (b3 ? 1 : 0);
        const float r = add_xor<32>(add_xor<16>(v[0]));
        if (lane < 16)
            red[slot][wave][(lane % TPR) * CPT + jl] = r;
        lds_barrier();
#pragma unroll
        for (int j = 0; j < CPT; ++j)
            x[j] = red[slot][0][cb + j] + red[slot][1][cb + j] + red[slot][2][cb + j] +
                   red[slot][3][cb + j];
        slot ^= 1;
    };
    auto row_sum = [&](float x) __attribute__((always_inline)) {
        x = add_xor<1>(x);
        if constexpr (TPR == 4)
            x = add_xor<2>(x);
        return x;
    };
    auto gain = [&](const Stage& s, int tau, float kk) __attribute__((always_inline)) {
        if constexpr (ISO)
            return s.kp[tau] * kk;
        else
            return s.kp[tau * DK + row];
    };

    // ---- forward pass: the state at every chunk start --------------------
    float s[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
        s[j] = a.S0 ? a.S0[((size_t)bh * DK + row) * dv + col0 + j] : 0.f;
    // stL -> stR for the arrays a pass reads, 16 bytes per thread and step
    auto move_stage = [&](bool rev) __attribute__((always_inline)) {
        auto mv = [&](const void* src, void* dst, int bytes) __attribute__((always_inline)) {
            const uint4* s4 = reinterpret_cast<const uint4*>(src);
            uint4* d4 = reinterpret_cast<uint4*>(dst);
            for (int i = tid; i < bytes / 16; i += 256)
                d4[i] = s4[i];
        };
        mv(stL.al, stR.al, (int)sizeof(stL.al));
        mv(stL.kp, stR.kp, (int)sizeof(stL.kp));
        mv(stL.kk, stR.kk, (int)sizeof(stL.kk));
        mv(stL.vv, stR.vv, (int)sizeof(stL.vv));
        if (rev) {
            mv(stL.qq, stR.qq, (int)sizeof(stL.qq));
            mv(stL.dd, stR.dd, (int)sizeof(stL.dd));
            mv(stL.dl, stR.dl, (int)sizeof(stL.dl));
            mv(stL.ck, stR.ck, (int)sizeof(stL.ck));
        }
    };
    for (int c = 0; c < nch; ++c) {
        if (c == 0)
            stage_copy(stL, 0, false);
        copies_landed_barrier();  // chunk c in stL; chunk c - 1's readers done with stR
        move_stage(false);
        lds_barrier();            // stR holds chunk c; stL is free
        if (c + 1 < nch)
            stage_copy(stL, c + 1, false);
        const Stage& cur = stR;
#pragma unroll
        for (int j = 0; j < CPT; ++j)
            ck[(size_t)c * (DK * BWD_COLS) + j] = s[j];
        const int len = min(L, T - c * L);
        for (int tau = 0; tau < len; ++tau) {
            const float al = cur.al[tau * DK + row], kk = to_f32(cur.kk[tau * DK + row]);
            const float kap = gain(cur, tau, kk);
            float x[CPT];
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                s[j] *= al;
                x[j] = s[j] * kk;
            }
            col_sum(x);
            float del[CPT];
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                del[j] = to_f32(cur.vv[tau * BWD_COLS + cb + j]) - x[j];
                s[j] += kap * del[j];
            }
            if (row == 0) {  // every row holds the same innovations
                float* dst = dlt_wg + (size_t)(c * L + tau) * BWD_COLS + cb;
#pragma unroll
                for (int j = 0; j < CPT; j += 4)
                    *reinterpret_cast<float4*>(dst + j) = {del[j], del[j + 1], del[j + 2], del[j + 3]};
            }
        }
    }

    // ---- reverse pass -----------------------------------------------------
    float g[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
        g[j] = a.gS_T ? a.gS_T[((size_t)bh * DK + row) * dv + col0 + j] : 0.f;
    for (int c = nch - 1; c >= 0; --c) {
        if (c == nch - 1) {
            copies_landed_barrier();  // the forward pass's readers and writers are done
            stage_copy(stL, c, true);
        }
        copies_landed_barrier();  // chunk c (inputs, innovations, checkpoint) in stL
        move_stage(true);
        lds_barrier();
        const Stage& cur = stR;
        float st[L + 1][CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j)
            st[0][j] = cur.ck[row * BWD_COLS + cb + j];
        if (c > 0)
            stage_copy(stL, c - 1, true);
        const int t0 = c * L, len = min(L, T - t0);
        // recompute the chunk's states from the stored innovations
#pragma unroll
        for (int tau = 0; tau < L; ++tau) {
            if (tau < len) {
                const float al = cur.al[tau * DK + row], kk = to_f32(cur.kk[tau * DK + row]);
                const float kap = gain(cur, tau, kk);
#pragma unroll
                for (int j = 0; j < CPT; ++j)
                    st[tau + 1][j] = al * st[tau][j] + kap * cur.dl[tau * BWD_COLS + cb + j];
            }
            // one step's loads at a time: keeps the 17 states the only large
            // live set (the loop has no barrier to bound the scheduler)
            __builtin_amdgcn_sched_barrier(0);
        }
        // walk the chunk backwards
#pragma unroll
        for (int tau = L - 1; tau >= 0; --tau) {
            if (tau < len) {
                const size_t tok = tok_of(t0 + tau);
                const float al = cur.al[tau * DK + row], kk = to_f32(cur.kk[tau * DK + row]);
                const float qq = to_f32(cur.qq[tau * DK + row]);
                const float kap = gain(cur, tau, kk);
                float dov[CPT], y[CPT];
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    dov[j] = to_f32(cur.dd[tau * BWD_COLS + cb + j]);
                    g[j] = fmaf(qq, dov[j], g[j]);               // readout o = S^T q
                    sq = fmaf(st[tau + 1][j], dov[j], sq);      // dq = S do
                    sk = fmaf(g[j], cur.dl[tau * BWD_COLS + cb + j], sk);  // kapbar = G delta
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
                    float* pp = part + ((size_t)blk * ntok + tok) * DK + row;
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
// Sum of the per-block partials, in parallel over every (token, channel):
// writes dq and leaves kapbar, the memory's dk and its dalpha summed in the
// first block's slot of each.
template <typename IO, int DK>
__global__ __launch_bounds__(256) void kdn_bwd_merge_kernel(BwdArgs args, int nblk)
{
    const BwdArgs a = args;
    const size_t ntok = (size_t)a.B * a.T * a.H, n4 = ntok * DK / 4;
    const size_t i4 = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i4 >= n4)
        return;
    const size_t kstride4 = (size_t)nblk * n4;
    const float4* p = reinterpret_cast<const float4*>(a.part) + i4;
    float4 sum[4];
#pragma unroll
    for (int kd = 0; kd < 4; ++kd)
        sum[kd] = p[kd * kstride4];
    for (int bl = 1; bl < nblk; ++bl)
#pragma unroll
        for (int kd = 0; kd < 4; ++kd) {
            const float4 x = p[kd * kstride4 + (size_t)bl * n4];
            sum[kd].x += x.x;
            sum[kd].y += x.y;
            sum[kd].z += x.z;
            sum[kd].w += x.w;
        }
    IO* dq = reinterpret_cast<IO*>(a.gq) + i4 * 4;
    dq[0] = from_f32<IO>(sum[0].x);
    dq[1] = from_f32<IO>(sum[0].y);
    dq[2] = from_f32<IO>(sum[0].z);
    dq[3] = from_f32<IO>(sum[0].w);
    float4* w = reinterpret_cast<float4*>(a.part) + i4;
#pragma unroll
    for (int kd = 1; kd < 4; ++kd)
        w[kd * kstride4] = sum[kd];
}

// The variance recurrence's adjoint is affine in the carried gradient, per
// channel for Diagonal (pbar_{t-1} = A_t pbar_t + B_t, A_t = alpha^2 / den^2,
// B_t = alpha^2 (kapbar k / d + dbar k^2)) and per head for Isotropic
// (bbar_{t-1} = A_t bbar_t + B_t, A_t = a / den^2, B_t = a betabar r / e^2).
// Everything else a token needs is known beforehand (dbar = -sum kapbar kap
// / d and betabar = sum kapbar k do not depend on the carried gradient), so
// it runs as a chunked scan over GR_C-token chunks: summaries (A, B) per
// chunk and channel, a carry across chunks from the last, and a replay of
// each chunk from its carried gradient that writes every output.

// Per-token quantities of one chunk in LDS, one thread per channel.
template <int DK>
struct GrChunk {
    float red[GR_C][DK + 1];  // per-token, per-channel terms of a channel sum
    float tok[GR_C];          // dbar (Diagonal) / betabar (Isotropic) per token
};

template <typename IO, bool ISO, int DK>
__device__ __forceinline__ void gr_load(const BwdArgs& a, size_t kstride, size_t tok, int i,
                                        float& kb, float& kk, float& al, float& pp, float& om)
{
    const size_t e = tok * DK + i;
    kb = a.part[kstride + e];
    kk = to_f32(reinterpret_cast<const IO*>(a.k)[e]);
    al = a.alpha[e];
    if constexpr (!ISO) {
        pp = a.pprev[e];
        om = a.omega[e];
    }
}

// Fill g.tok with dbar or betabar for the chunk's nv tokens.
// The token loops of the gain backward take GT tokens at a time: every load
// of a batch is issued before any of its values is used, so a chunk waits
// for memory once per batch rather than once per token.
constexpr int GT = 8;

template <typename IO, bool ISO, int DK>
__device__ __forceinline__ void gr_token_sums(const BwdArgs& a, GrChunk<DK>& g, size_t kstride,
                                              size_t tok0, size_t tstride, int nv, int i)
{
    for (int tb = 0; tb < nv; tb += GT) {
        float kb[GT], kk[GT], al[GT], pp[GT], om[GT], dd[GT];
#pragma unroll
        for (int u = 0; u < GT; ++u) {
            const size_t tok = tok0 + min(tb + u, nv - 1) * tstride;
            pp[u] = om[u] = 0.f;
            gr_load<IO, ISO, DK>(a, kstride, tok, i, kb[u], kk[u], al[u], pp[u], om[u]);
            dd[u] = ISO ? 1.f : a.dd[tok];
        }
#pragma unroll
        for (int u = 0; u < GT; ++u) {
            const int t = tb + u;
            if (t < nv) {
                if constexpr (!ISO) {
                    const float ph = al[u] * al[u] * pp[u] + om[u];
                    g.red[t][i] = kb[u] * ph * kk[u] * rcp(dd[u]);  // kapbar kap
                } else {
                    g.red[t][i] = kb[u] * kk[u];
                }
            }
        }
    }
    __syncthreads();
    if (i < nv) {
        float sum = 0.f;
        for (int j = 0; j < DK; ++j)
            sum += g.red[i][j];
        const size_t tok = tok0 + i * tstride;
        g.tok[i] = ISO ? sum : -sum * rcp(a.dd[tok]);
    }
    __syncthreads();
}

// pass 1: each chunk's affine map from the gradient after its last token to
// the gradient before its first
template <typename IO, bool ISO, int DK>
__global__ __launch_bounds__(DK) void kdn_bwd_gr_summary_kernel(BwdArgs args, int nblk, int nchunks)
{
    const BwdArgs a = args;
    __shared__ GrChunk<DK> g;
    const int bh = blockIdx.x / nchunks, c = blockIdx.x % nchunks, i = threadIdx.x;
    const int H = a.H, T = a.T, b = bh / H, h = bh % H;
    const int t0 = c * GR_C, nv = min(GR_C, T - t0);
    const float mu = a.mu_h ? a.mu_h[h] : a.mu;
    const size_t kstride = (size_t)nblk * a.B * T * H * DK;
    const size_t tok0 = ((size_t)b * T + t0) * H + h, tstride = H;
    float A = 1.f, Bc = 0.f;
    if constexpr (!ISO) {
        // One pass over the chunk's data: the token sums' terms and, per
        // token, the map's pieces At = alpha^2 / den^2, B1 = alpha^2 kapbar k
        // / d and Ct = alpha^2 k^2 (Bt = B1 + dbar Ct once the sums are in).
        // The composite is A = prod_t At and B = sum_t Q_t Bt with Q_t the
        // product of At over the tokens before t, so it is formed in token
        // order: Q, sum_t Q_t B1 and the weights W_t = Q_t Ct run along, and
        // sum_t W_t dbar_t is added once the sums are in (one register per
        // token rather than three).
        float W[GR_C];
        float Q = 1.f, Bq = 0.f;
#pragma unroll
        for (int tb = 0; tb < GR_C; tb += GT) {
            float kb[GT], kk[GT], al[GT], pp[GT], om[GT], dd[GT], rt[GT];
#pragma unroll
            for (int u = 0; u < GT; ++u) {
                const size_t tok = tok0 + min(tb + u, nv - 1) * tstride;
                gr_load<IO, ISO, DK>(a, kstride, tok, i, kb[u], kk[u], al[u], pp[u], om[u]);
                dd[u] = a.dd[tok];
                rt[u] = a.r[tok];
            }
#pragma unroll
            for (int u = 0; u < GT; ++u) {
                const int t = tb + u;
                const float ph = al[u] * al[u] * pp[u] + om[u], id = rcp(dd[u]);
                if (t < nv)
                    g.red[t][i] = kb[u] * ph * kk[u] * id;  // kapbar kap
                const float den = 1.f + (mu / rt[u]) * kk[u] * kk[u] * ph;
                const float a2 = al[u] * al[u];
                W[t] = 0.f;
                if (t < nv) {
                    W[t] = Q * (a2 * (kk[u] * kk[u]));
                    Bq += Q * (a2 * (kb[u] * kk[u] * id));
                    Q *= a2 * rcp(den * den);
                }
            }
        }
        __syncthreads();
        if (i < nv) {
            float sum = 0.f;
            for (int j = 0; j < DK; ++j)
                sum += g.red[i][j];
            g.tok[i] = -sum * rcp(a.dd[tok0 + i * tstride]);
        }
        __syncthreads();
        A = Q;
        Bc = Bq;
#pragma unroll
        for (int t = 0; t < GR_C; ++t)
            if (t < nv)
                Bc += W[t] * g.tok[t];
    } else {
    gr_token_sums<IO, ISO, DK>(a, g, kstride, tok0, tstride, nv, i);
    for (int tb = nv - 1; tb >= 0; tb -= GT) {
        // the batch's loads (tokens tb, tb - 1, .., clamped at 0), then its maps
        float rt[GT], kb[GT], kk[GT], al[GT], pp[GT], om[GT], dd[GT];
        float4 gs[GT];
#pragma unroll
        for (int u = 0; u < GT; ++u) {
            const size_t tok = tok0 + max(tb - u, 0) * tstride;
            rt[u] = a.r[tok];
            if constexpr (!ISO) {
                gr_load<IO, ISO, DK>(a, kstride, tok, i, kb[u], kk[u], al[u], pp[u], om[u]);
                dd[u] = a.dd[tok];
            } else {
                gs[u] = *reinterpret_cast<const float4*>(a.gsc + tok * 4);
                om[u] = a.omega[tok];
            }
        }
#pragma unroll
        for (int u = 0; u < GT; ++u) {
            const int t = tb - u;
            if (t < 0)
                break;
            float At, Bt;
            if constexpr (!ISO) {
                const float ph = al[u] * al[u] * pp[u] + om[u];
                const float den = 1.f + (mu / rt[u]) * kk[u] * kk[u] * ph;
                const float inv2 = rcp(den * den);
                At = al[u] * al[u] * inv2;
                Bt = al[u] * al[u] * (kb[u] * kk[u] * rcp(dd[u]) + g.tok[t] * kk[u] * kk[u]);
            } else {
                const float bhat = gs[u].z * gs[u].y + om[u], n = gs[u].w;
                const float e = rt[u] + bhat * n;
                const float den = 1.f + mu * n / ((float)DK * rt[u]) * bhat;
                At = gs[u].z * rcp(den * den);
                Bt = gs[u].z * g.tok[t] * rt[u] * rcp(e * e);
            }
            A = At * A;
            Bc = At * Bc + Bt;
        }
    }
    }
    const size_t width = ISO ? 1 : DK;
    if (!ISO || i == 0) {
        const size_t o = (((size_t)bh * nchunks + c) * width + (ISO ? 0 : i)) * 2;
        a.gr_sum[o] = A;
        a.gr_sum[o + 1] = Bc;
    }
    if (i < nv)
        a.gr_tok[tok0 + i * tstride] = g.tok[i];
}

// pass 2: the gradient after every chunk's last token, from the last chunk;
// the initial variance's gradient at the end.  One lane per row ((b,h) and
// channel), up to GR_WAVES wavefronts per workgroup, each over its own
// contiguous run of chunks.  Every wave but the first composes its run's
// maps into one (g -> A g + B, the run's last chunk applied first); the
// waves exchange those through LDS, so that each applies the runs after its
// own to the final gradient; then every wave walks its run again, writing
// the gradient each chunk receives.  Two serial passes over nchunks / waves
// maps instead of one over nchunks.  Inside a run the maps are read GU chunks
// ahead into a second register set while the current GU are applied.
constexpr int GU = 16, GR_WAVES = 8;

// Walk chunks c_end - 1 down to c_begin of one row (maps and out point at the
// row's chunk 0, chunk c at c * width) from m = (A, B): m <- (A_c A, A_c B +
// B_c).  From (1, 0) that composes the run's maps; from (1, g) its second
// component is the carried gradient, stored (when STORE) as each chunk's
// before that chunk's map is applied.
template <bool STORE>
__device__ __forceinline__ float2 gr_run(const float2* maps, float* out, size_t width, int c_begin,
                                         int c_end, float2 m)
{
    float2 cur[GU], nxt[GU];
    auto fetch = [&](float2 (&dst)[GU], int top) {
#pragma unroll
        for (int u = 0; u < GU; ++u)
            dst[u] = top - u >= c_begin ? maps[(size_t)(top - u) * width] : make_float2(1.f, 0.f);
    };
    if (c_begin < c_end)
        fetch(cur, c_end - 1);
    for (int top = c_end - 1; top >= c_begin; top -= GU) {
        if (top - GU >= c_begin)
            fetch(nxt, top - GU);
#pragma unroll
        for (int u = 0; u < GU; ++u) {
            if (top - u >= c_begin) {
                if constexpr (STORE)
                    out[(size_t)(top - u) * width] = m.y;
                m = make_float2(cur[u].x * m.x, cur[u].x * m.y + cur[u].y);
            }
        }
#pragma unroll
        for (int u = 0; u < GU; ++u)
            cur[u] = nxt[u];
    }
    return m;
}

__global__ __launch_bounds__(64 * GR_WAVES) void kdn_bwd_gr_carry_kernel(BwdArgs args, int width,
                                                                        int nchunks)
{
    const BwdArgs a = args;
    __shared__ float2 run_map[GR_WAVES][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nwave = blockDim.x >> 6;
    const size_t rows = (size_t)a.B * a.H * width, r = (size_t)blockIdx.x * 64 + lane;
    const bool live = r < rows;
    const size_t row = live ? r : 0;  // lanes past the last row read row 0 and store nothing
    const size_t base = (row / width * nchunks) * width + row % width;
    const int per = (nchunks + nwave - 1) / nwave;
    const int c_begin = min(nchunks, wv * per), c_end = min(nchunks, c_begin + per);
    const float2* maps = reinterpret_cast<const float2*>(a.gr_sum) + base;
    const float2 id = make_float2(1.f, 0.f);
    run_map[wv][lane] = wv > 0 ? gr_run<false>(maps, nullptr, width, c_begin, c_end, id) : id;
    __syncthreads();
    float g = live && a.gvar_T ? a.gvar_T[row] : 0.f;
    for (int w2 = nwave - 1; w2 > wv; --w2) {
        const float2 m = run_map[w2][lane];
        g = m.x * g + m.y;
    }
    float2 e = id;
    if (live)
        e = gr_run<true>(maps, a.gr_carry + base, width, c_begin, c_end, make_float2(1.f, g));
    if (live && wv == 0 && a.gvar0)
        a.gvar0[row] = e.y;
}

// pass 3: replay every chunk from its carried gradient, writing dk, dalpha,
// domega, dr and a partial information-scale gradient per chunk
template <typename IO, bool ISO, int DK>
__global__ __launch_bounds__(DK) void kdn_bwd_gr_replay_kernel(BwdArgs args, int nblk, int nchunks)
{
    const BwdArgs a = args;
    __shared__ GrChunk<DK> g;
    __shared__ float smu[DK / 64];
    const int bh = blockIdx.x / nchunks, c = blockIdx.x % nchunks, i = threadIdx.x;
    const int H = a.H, T = a.T, b = bh / H, h = bh % H;
    const int t0 = c * GR_C, nv = min(GR_C, T - t0);
    const float mu = a.mu_h ? a.mu_h[h] : a.mu;
    const size_t kstride = (size_t)nblk * a.B * T * H * DK;
    const size_t tok0 = ((size_t)b * T + t0) * H + h, tstride = H;
    IO* dkg = reinterpret_cast<IO*>(a.gk);
    if (i < nv)
        g.tok[i] = a.gr_tok[tok0 + i * tstride];
    __syncthreads();
    const size_t width = ISO ? 1 : DK;
    float gbar = a.gr_carry[((size_t)bh * nchunks + c) * width + (ISO ? 0 : i)];
    float mub = 0.f;
    for (int tb = nv - 1; tb >= 0; tb -= GT) {
      // the batch's loads (tokens tb, tb - 1, .., clamped at 0), then its tokens
      float rt_[GT], kb_[GT], kk_[GT], al_[GT], pp_[GT], om_[GT], kmb_[GT], amb_[GT], dd_[GT];
      float4 gs_[GT];
#pragma unroll
      for (int u = 0; u < GT; ++u) {
          const size_t tok = tok0 + max(tb - u, 0) * tstride, e = tok * DK + i;
          rt_[u] = a.r[tok];
          pp_[u] = om_[u] = 0.f;
          gr_load<IO, ISO, DK>(a, kstride, tok, i, kb_[u], kk_[u], al_[u], pp_[u], om_[u]);
          kmb_[u] = a.part[2 * kstride + e];
          amb_[u] = a.part[3 * kstride + e];
          if constexpr (!ISO) {
              dd_[u] = a.dd[tok];
          } else {
              gs_[u] = *reinterpret_cast<const float4*>(a.gsc + tok * 4);
              om_[u] = a.omega[tok];
          }
      }
#pragma unroll
      for (int u = 0; u < GT; ++u) {
        const int t = tb - u;
        if (t < 0)
            break;
        const size_t tok = tok0 + t * tstride, e = tok * DK + i;
        const float rt = rt_[u], kb = kb_[u], kk = kk_[u], al = al_[u], pp = pp_[u], om = om_[u];
        const float kmb = kmb_[u], amb = amb_[u];
        if constexpr (!ISO) {
            const float d = dd_[u], dbar = g.tok[t];
            const float ph = al * al * pp + om;
            const float uu = (mu / rt) * kk * kk;
            const float den = 1.f + uu * ph, inv2 = rcp(den * den);
            const float ub = -gbar * ph * ph * inv2;
            const float phb = gbar * inv2 + kb * kk * rcp(d) + dbar * kk * kk;
            dkg[e] = from_f32<IO>(kmb + 2.f * ub * (mu / rt) * kk + kb * ph * rcp(d) +
                                  2.f * dbar * ph * kk);
            a.galpha[e] = amb + 2.f * phb * al * pp;
            a.gomega[e] = phb;
            g.red[t][i] = ub * uu;
            mub += ub * kk * kk / rt;
            gbar = phb * al * al;
        } else {
            const float4 gs = gs_[u];
            const float beta = gs.x, bprev = gs.y, am = gs.z, n = gs.w, betab = g.tok[t];
            const float bhat = am * bprev + om;
            const float ee = rt + bhat * n;
            const float uu = mu * n / ((float)DK * rt);
            const float den = 1.f + uu * bhat, inv2 = rcp(den * den);
            const float ub = -gbar * bhat * bhat * inv2;
            const float bhb = gbar * inv2 + betab * rt * rcp(ee * ee);
            const float nb = ub * mu / ((float)DK * rt) - betab * bhat * bhat * rcp(ee * ee);
            const float abar = bhb * bprev;
            dkg[e] = from_f32<IO>(kmb + beta * kb + 2.f * nb * kk);
            a.galpha[e] = amb + 2.f * abar * al / (float)DK;
            if (i == 0) {
                a.gomega[tok] = bhb;
                a.gr[tok] = -ub * uu / rt - betab * bhat * rcp(ee * ee);
                mub += ub * n / ((float)DK * rt);
            }
            gbar = bhb * am;
        }
      }
    }
    if constexpr (!ISO) {
        __syncthreads();
        if (i < nv) {
            float s2 = 0.f;
            for (int j = 0; j < DK; ++j)
                s2 += g.red[i][j];
            const size_t tok = tok0 + i * tstride;
            a.gr[tok] = g.tok[i] - s2 / a.r[tok];
        }
        mub = wave_sum(mub);
        if ((i & 63) == 0)
            smu[i >> 6] = mub;
        __syncthreads();
        if (i == 0) {
            float m = 0.f;
            for (int w = 0; w < DK / 64; ++w)
                m += smu[w];
            a.gr_mu[(size_t)bh * nchunks + c] = m;
        }
    } else {
        if (i == 0)
            a.gr_mu[(size_t)bh * nchunks + c] = mub;
    }
}

// pass 4: the information scale's gradient per (b,h), summed over chunks:
// one workgroup per (b,h), each thread a strided share of the chunks, then a
// fixed-order tree over the threads (deterministic)
__global__ __launch_bounds__(256) void kdn_bwd_gr_mu_kernel(BwdArgs args, int nchunks)
{
    const BwdArgs a = args;
    const size_t bh = blockIdx.x;
    const int t = threadIdx.x;
    __shared__ float part[256];
    float m = 0.f;
    for (int c = t; c < nchunks; c += 256)
        m += a.gr_mu[bh * nchunks + c];
    part[t] = m;
    __syncthreads();
    for (int n = 128; n > 0; n >>= 1) {
        if (t < n)
            part[t] += part[t + n];
        __syncthreads();
    }
    if (t == 0)
        a.gmu[bh] = part[0];
}

// ---------------------------------------------------------------------------
// workspace and launch
// ---------------------------------------------------------------------------
template <typename IO, bool ISO, int DK>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream)
{
    const bool chunked = bwd_chunked(DK, a.dv);
    const int bh = a.B * a.H, nblk = a.dv / (chunked ? BWD_CHUNK_COLS : BWD_COLS);
    if (a.T > 0) {
        const int nchunks = (a.T + 63) / 64;
        const size_t width = ISO ? 1 : (size_t)DK;
        GainArgs g{a.k, a.alpha, a.omega, a.r, a.var0, ISO ? nullptr : a.kap, nullptr, a.gscan,
                   a.gscan + (size_t)bh * 4 * width * nchunks, a.B, a.T, a.H, DK, a.mu};
        g.mu_h = a.mu_h;
        g.c0 = a.c0;
        g.pprev = a.pprev;
        g.dd = a.dd;
        g.gsc = a.gsc;
        hipError_t e = launch_gain_scan(g, ISO, sizeof(IO) == 2 ? 1 : 0, stream);
        if (e != hipSuccess)
            return e;
    }
    hipError_t e;
    if (chunked) {
        if (a.nseg) {
            e = launch_seqpar_bwd_mem(a, ISO, stream);
        } else if (!ISO && sizeof(IO) == 2 && a.T > 0) {
            // Diagonal with bf16 io: the chunk-start states from the forward
            // walk (state only, split-bf16 products, ~1e-5 relative), in place
            // of the chunk kernel's own fp32 forward pass
            FwdArgs w{};
            w.q = a.q;
            w.k = a.k;
            w.v = a.v;
            w.alpha = a.alpha;
            w.omega = a.omega;
            w.r = a.r;
            w.S0 = a.S0;
            w.var0 = a.var0;
            w.c0 = a.c0;
            w.mu = a.mu;
            w.mu_h = a.mu_h;
            w.S_T = a.walk_S;
            w.var_T = a.walk_p;
            w.B = a.B;
            w.T = a.T;
            w.H = a.H;
            w.dk = DK;
            w.dv = a.dv;
            w.split = true;
            w.state_only = 1;
            w.ckpt = a.ckpt;
            e = launch_walk_fwd(w, false, stream);
            if (e != hipSuccess)
                return e;
            BwdArgs ac = a;
            ac.ckpt_given = true;
            e = launch_bwd_chunk_mem(ac, ISO, 1, false, stream);
        } else {
            e = launch_bwd_chunk_mem(a, ISO, sizeof(IO) == 2 ? 1 : 0, false, stream);
        }
    } else {
        hipLaunchKernelGGL((kdn_bwd_mem_kernel<IO, ISO, DK>), dim3(nblk, bh), dim3(256), 0, stream,
                           a);
        e = hipGetLastError();
    }
    if (e != hipSuccess)
        return e;
    const size_t n4 = (size_t)a.B * a.T * a.H * DK / 4;
    if (n4 > 0 && !chunked) {  // the chunked path sums its blocks itself
        hipLaunchKernelGGL((kdn_bwd_merge_kernel<IO, DK>), dim3((unsigned)((n4 + 255) / 256)),
                           dim3(256), 0, stream, a, nblk);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const int ngc = (a.T + GR_C - 1) / GR_C, width = ISO ? 1 : DK;
    if (ngc > 0) {
        hipLaunchKernelGGL((kdn_bwd_gr_summary_kernel<IO, ISO, DK>), dim3(bh * ngc), dim3(DK), 0,
                           stream, a, nblk, ngc);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    // one wave per run of at least 64 chunks, up to GR_WAVES
    const int nwave = std::min(GR_WAVES, std::max(1, ngc / 64));
    hipLaunchKernelGGL(kdn_bwd_gr_carry_kernel, dim3((bh * width + 63) / 64), dim3(64 * nwave), 0,
                       stream, a, width, ngc);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (ngc > 0) {
        hipLaunchKernelGGL((kdn_bwd_gr_replay_kernel<IO, ISO, DK>), dim3(bh * ngc), dim3(DK), 0,
                           stream, a, nblk, ngc);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (a.gmu) {
        hipLaunchKernelGGL(kdn_bwd_gr_mu_kernel, dim3(bh), dim3(256), 0, stream, a, ngc);
        e = hipGetLastError();
    }
    return e;
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
