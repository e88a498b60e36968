// kdn_api.cpp -- host side of the C ABI declared in include/kdn.h:
// synchronous argument validation, regime choice and kernel launch.
// Nothing here allocates device memory or throws across the ABI.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "kdn.h"
#include "kdn_internal.h"
#include "kdn_ops.h"

namespace {

thread_local char g_msg[512] = "";

kdn_status fail(kdn_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
    va_end(ap);
    return st;
}

kdn_status ok()
{
    g_msg[0] = '\0';
    return KDN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kMaxElems = (size_t)1 << 31;

// true when the product of the (non-negative) factors stays below 2^31; each
// partial product is compared before the next multiplication, so no
// intermediate can wrap around
static bool below_2_31(std::initializer_list<size_t> factors)
{
    size_t p = 1;
    for (size_t f : factors) {
        if (f == 0)
            return true;
        if (f >= kMaxElems || p >= kMaxElems / f + 1)
            return false;
        p *= f;
        if (p >= kMaxElems)
            return false;
    }
    return true;
}

// Shape / dtype rules shared by the forward and step calls.
kdn_status check_common(int B, int T, int H, int dk, int dv, int io, float mu, bool chunked)
{
    if (io != KDN_F32 && io != KDN_BF16)
        return fail(KDN_ERR_INVALID_ARG, "io_dtype must be KDN_F32 (0) or KDN_BF16 (1), got %d", io);
    if (B < 1 || H < 1 || T < 0)
        return fail(KDN_ERR_INVALID_ARG, "need B >= 1, H >= 1, T >= 0 (got B=%d T=%d H=%d)", B, T, H);
    if (!(mu >= 0.f) || !std::isfinite(mu))
        return fail(KDN_ERR_INVALID_ARG, "mu must be finite and >= 0 (got %g)", (double)mu);
    if (chunked) {
        if (io == KDN_BF16) {
            if (dk != 64 && dk != 128)
                return fail(KDN_ERR_UNSUPPORTED, "bf16 forward supports dk in {64, 128}, got %d", dk);
            if (dv <= 0 || dv % 64 != 0 || dv > 256)
                return fail(KDN_ERR_UNSUPPORTED,
                            "bf16 forward supports dv a multiple of 64 up to 256, got %d", dv);
        } else {
            if (dk != 64)
                return fail(KDN_ERR_UNSUPPORTED, "fp32 forward supports dk = 64, got %d", dk);
            if (dv <= 0 || dv % 32 != 0 || dv > 256)
                return fail(KDN_ERR_UNSUPPORTED,
                            "fp32 forward supports dv a multiple of 32 up to 256, got %d", dv);
        }
    } else {
        if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128))
            return fail(KDN_ERR_UNSUPPORTED, "step supports dk, dv in {64, 128}, got %d, %d", dk, dv);
    }
    const size_t widest = (size_t)(dk > dv ? dk : dv);
    if (!below_2_31({(size_t)B, (size_t)(T > 0 ? T : 1), (size_t)H, widest}) ||
        !below_2_31({(size_t)B, (size_t)H, (size_t)dk, (size_t)dv}))
        return fail(KDN_ERR_UNSUPPORTED, "tensor sizes must stay below 2^31 elements");
    return KDN_OK;
}

#define KDN_REQUIRE(ptr, name)                                                   \
    do {                                                                         \
        if (!(ptr))                                                              \
            return fail(KDN_ERR_INVALID_ARG, "%s must not be NULL", name);        \
    } while (0)

#define KDN_ALIGNED(ptr, name)                                                   \
    do {                                                                         \
        if ((ptr) && !aligned16(ptr))                                            \
            return fail(KDN_ERR_INVALID_ARG, "%s must be 16-byte aligned", name); \
    } while (0)

#define KDN_ALIGNED_X(ptr, name)                                                 \
    do {                                                                         \
        if ((ptr) && (reinterpret_cast<uintptr_t>(ptr) & 3u))                    \
            return fail(KDN_ERR_INVALID_ARG, "%s must be 4-byte aligned", name);  \
    } while (0)

// The io dtype of a forward call and its contraction-precision flag:
// KDN_MATH_BF16 (bf16 io only) selects single bf16 products for Diagonal.
kdn_status split_io(int io_dtype, int& io, bool& math_bf16, bool& out_f32)
{
    math_bf16 = (io_dtype & KDN_MATH_BF16) != 0;
    out_f32 = (io_dtype & KDN_OUT_F32) != 0;
    io = io_dtype & ~(KDN_MATH_BF16 | KDN_OUT_F32);
    if (io != KDN_F32 && io != KDN_BF16)
        return fail(KDN_ERR_INVALID_ARG,
                    "io_dtype must be KDN_F32 (0) or KDN_BF16 (1), optionally with "
                    "KDN_MATH_BF16 (0x100) or KDN_OUT_F32 (0x200) for bf16, got %d", io_dtype);
    if ((math_bf16 || out_f32) && io != KDN_BF16)
        return fail(KDN_ERR_INVALID_ARG, "KDN_MATH_BF16 and KDN_OUT_F32 apply to bf16 io only");
    if (out_f32 && math_bf16)
        return fail(KDN_ERR_UNSUPPORTED, "KDN_OUT_F32 comes with the split-product contractions, "
                                         "not with KDN_MATH_BF16");
    return KDN_OK;
}

// Per-head options and the diagnostic output of the extended calls.
struct ExtOpts {
    const float* mu_h = nullptr;  // [H] or null
    const float* c0_h = nullptr;  // [H] or null
    float* beta_eff = nullptr;    // [B,T,H] / [B,H] or null
};

kdn_status check_ext(const ExtOpts& x, const void* var0, const void* r, const void* o,
                     const void* S_out, const void* var_out)
{
    if (x.c0_h && var0)
        return fail(KDN_ERR_INVALID_ARG, "give the initial variance either as var0 or as c0_h, not both");
    KDN_ALIGNED_X(x.mu_h, "mu_h");
    KDN_ALIGNED_X(x.c0_h, "c0_h");
    KDN_ALIGNED_X(x.beta_eff, "beta_eff");
    if (x.beta_eff && (x.beta_eff == r || x.beta_eff == o || x.beta_eff == S_out ||
                       x.beta_eff == var_out))
        return fail(KDN_ERR_INVALID_ARG, "beta_eff must not alias r, o, the state or the variances");
    return KDN_OK;
}

kdn_status fwd_impl(bool iso, int B, int T, int H, int dk, int dv, int io_dtype, float mu,
                    const void* q, const void* k, const void* v, const float* alpha,
                    const float* omega, const float* r, const float* S0, const float* var0,
                    void* o, float* S_T, float* var_T, void* workspace,
                    size_t workspace_bytes, void* stream, const ExtOpts& x = ExtOpts{},
                    const kdn::PrologueArgs* pro = nullptr)
{
    int io;
    bool math_bf16, out_f32;
    kdn_status st = split_io(io_dtype, io, math_bf16, out_f32);
    if (st != KDN_OK)
        return st;
    if (out_f32 && iso)
        return fail(KDN_ERR_UNSUPPORTED, "KDN_OUT_F32 is built for the Diagonal forward");
    st = check_common(B, T, H, dk, dv, io, mu, true);
    if (st != KDN_OK)
        return st;
    st = check_ext(x, var0, r, o, S_T, var_T);
    if (st != KDN_OK)
        return st;
    if (T > 0) {
        KDN_REQUIRE(q, "q");
        KDN_REQUIRE(k, "k");
        KDN_REQUIRE(v, "v");
        KDN_REQUIRE(alpha, "alpha");
        KDN_REQUIRE(omega, "omega");
        KDN_REQUIRE(r, "r");
        KDN_REQUIRE(o, "o");
    }
    KDN_REQUIRE(S_T, "S_T");
    KDN_REQUIRE(var_T, iso ? "b_T" : "p_T");
    KDN_ALIGNED(q, "q");
    KDN_ALIGNED(k, "k");
    KDN_ALIGNED(v, "v");
    KDN_ALIGNED(alpha, "alpha");
    if (!iso)
        KDN_ALIGNED(omega, "omega");
    KDN_ALIGNED(o, "o");
    KDN_ALIGNED(S0, "S0");
    KDN_ALIGNED(S_T, "S_T");
    if (!iso) {
        KDN_ALIGNED(var0, "p0");
        KDN_ALIGNED(var_T, "p_T");
    }
    // Every value-tile workgroup of a head (dv / 64 of them for bf16 io,
    // dv / 32 for fp32) reads the head's initial variances when it starts,
    // and only the first tile writes the final ones when it ends; nothing
    // orders a later tile's start after that write.  So the variances may
    // alias in place only where one workgroup walks each head.
    const int vtile = io == KDN_BF16 ? 64 : 32;
    if (var0 && var0 == var_T && dv > vtile)
        return fail(KDN_ERR_INVALID_ARG,
                    "%s may alias %s only when dv <= %d (one workgroup per head); give a "
                    "separate %s buffer", iso ? "b_T" : "p_T", iso ? "b0" : "p0", vtile,
                    iso ? "b_T" : "p_T");
    if (var0 && var0 != var_T) {
        // each variance is read at the start and written at the end, so a
        // partial overlap is never safe
        const size_t vb = (size_t)B * H * (iso ? 1 : dk) * sizeof(float);
        const char *a0 = (const char*)var0, *a1 = (const char*)var_T;
        if (a0 < a1 + vb && a1 < a0 + vb)
            return fail(KDN_ERR_INVALID_ARG, "%s must either equal %s or not overlap it",
                        iso ? "b_T" : "p_T", iso ? "b0" : "p0");
    }
    if (o && (o == q || o == k || o == v))
        return fail(KDN_ERR_INVALID_ARG, "o must not alias q, k or v");
    if (S0 && S0 != S_T) {
        const char* s0 = reinterpret_cast<const char*>(S0);
        const char* st_ = reinterpret_cast<const char*>(S_T);
        const size_t bytes = (size_t)B * H * dk * dv * sizeof(float);
        if (s0 < st_ + bytes && st_ < s0 + bytes)
            return fail(KDN_ERR_INVALID_ARG, "S_T must either equal S0 or not overlap it");
    }
    // the workspace is optional: with the size kdn_fwd_workspace_size names,
    // shapes with few heads and long sequences run sequence-parallel
    const int nseg = pro ? 0 : kdn::seqpar_segments(iso, B, T, H, dk, dv, io);
    const size_t sp_bytes =
        nseg ? kdn::seqpar_workspace_floats(iso, B, T, H, dk, dv, nseg) * sizeof(float) : 0;
    const bool seqpar = nseg && workspace && workspace_bytes >= sp_bytes;
    if (seqpar) {
        KDN_ALIGNED(workspace, "workspace");
        const char *w0 = (const char*)workspace, *w1 = w0 + sp_bytes;
        const size_t ntok = (size_t)B * T * H;
        const size_t nst = (size_t)B * H * dk * dv * sizeof(float);
        const size_t nvar = (size_t)B * H * (iso ? 1 : dk) * sizeof(float);
        const struct { const void* p; size_t n; const char* name; } bufs[] = {
            {q, ntok * dk * 2, "q"}, {k, ntok * dk * 2, "k"}, {v, ntok * dv * 2, "v"},
            {alpha, ntok * dk * 4, "alpha"}, {omega, ntok * (iso ? 1 : dk) * 4, "omega"},
            {r, ntok * 4, "r"}, {o, ntok * dv * (out_f32 ? 4 : 2), "o"}, {S0, nst, "S0"}, {S_T, nst, "S_T"},
            {var0, nvar, "var0"}, {var_T, nvar, "var_T"}, {x.mu_h, (size_t)H * 4, "mu_h"},
            {x.c0_h, (size_t)H * 4, "c0_h"}, {x.beta_eff, ntok * 4, "beta_eff"}};
        for (const auto& b : bufs) {
            const char* b0 = (const char*)b.p;
            if (b.p && w0 < b0 + b.n && b0 < w1)
                return fail(KDN_ERR_INVALID_ARG, "workspace must not overlap %s", b.name);
        }
    }

    kdn::FwdArgs a{q, k, v, alpha, omega, r, S0, var0, o, S_T, var_T, B, T, H, dk, dv, mu,
                   x.mu_h, x.c0_h, T > 0 ? x.beta_eff : nullptr};
    // the Diagonal bf16 walk runs split-operand products unless told otherwise
    a.split = !iso && io == KDN_BF16 && !math_bf16;
    a.o_f32 = out_f32;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    // From pre-activations, the bf16 walk reads a (and Diagonal w) itself and
    // forms alpha (and omega) on chip; the per-token gates (r, Isotropic
    // omega) and every gate of the fp32 path come from the gate pass, into
    // the workspace.
    const bool fused = pro && io == KDN_BF16 && !out_f32 && T > 0;
    const bool fuse_omega = fused && !iso;
    if (pro && T > 0) {
        kdn::PrologueArgs p = *pro;
        if (fused)
            p.n_alpha = 0;
        if (fuse_omega)
            p.n_omega = 0;
        hipError_t e = kdn::launch_gate_prologue(p, io, hs);
        if (e != hipSuccess)
            return fail(KDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
    if (fused) {
        a.a_pre = pro->a_pre;
        if (fuse_omega)
            a.w_pre = pro->w_pre;
    }
    hipError_t e = seqpar ? kdn::launch_seqpar_fwd(a, iso, nseg, static_cast<float*>(workspace), hs)
                   : io == KDN_BF16 ? kdn::launch_walk_fwd(a, iso, hs)
                                    : kdn::launch_chunk_fwd_f32(a, iso, hs);
    if (e != hipSuccess)
        return fail(KDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

size_t kdn_fwd_workspace_size(int variant, int B, int T, int H, int dk, int dv, int io_dtype)
{
    if (B < 0 || T < 0 || H <= 0 || (dk != 64 && dk != 128) || (dv != 64 && dv != 128) ||
        !below_2_31({(size_t)B, (size_t)(T > 0 ? T : 1), (size_t)H, (size_t)(dk > dv ? dk : dv)}))
        return 0;
    const bool iso = variant == KDN_ISO;
    const int nseg =
        kdn::seqpar_segments(iso, B, T, H, dk, dv, io_dtype & ~(KDN_MATH_BF16 | KDN_OUT_F32));
    // zero: the walk keeps every intermediate on chip; otherwise the
    // sequence-parallel path's segment states and carries
    return nseg ? kdn::seqpar_workspace_floats(iso, B, T, H, dk, dv, nseg) * sizeof(float) : 0;
}

kdn_status kdn_diag_fwd(int B, int T, int H, int dk, int dv, int io_dtype, float mu,
                        const void* q, const void* k, const void* v, const float* alpha,
                        const float* omega, const float* r, const float* S0, const float* p0,
                        void* o, float* S_T, float* p_T, void* workspace,
                        size_t workspace_bytes, void* stream)
{
    return fwd_impl(false, B, T, H, dk, dv, io_dtype, mu, q, k, v, alpha, omega, r, S0, p0, o,
                    S_T, p_T, workspace, workspace_bytes, stream);
}

kdn_status kdn_iso_fwd(int B, int T, int H, int dk, int dv, int io_dtype, float mu,
                       const void* q, const void* k, const void* v, const float* alpha,
                       const float* omega, const float* r, const float* S0, const float* b0,
                       void* o, float* S_T, float* b_T, void* workspace,
                       size_t workspace_bytes, void* stream)
{
    return fwd_impl(true, B, T, H, dk, dv, io_dtype, mu, q, k, v, alpha, omega, r, S0, b0, o,
                    S_T, b_T, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

kdn_status step_impl(int variant, int B, int H, int dk, int dv, int io_dtype, float mu,
                     const void* q, const void* k, const void* v, const float* alpha,
                     const float* omega, const float* r, float* S, float* var_state, void* o,
                     void* stream, const ExtOpts& x = ExtOpts{})
{
    if (variant != KDN_DIAG && variant != KDN_ISO)
        return fail(KDN_ERR_INVALID_ARG, "variant must be KDN_DIAG (0) or KDN_ISO (1), got %d",
                    variant);
    const bool iso = variant == KDN_ISO;
    kdn_status st = check_common(B, 1, H, dk, dv, io_dtype, mu, false);
    if (st != KDN_OK)
        return st;
    KDN_REQUIRE(q, "q");
    KDN_REQUIRE(k, "k");
    KDN_REQUIRE(v, "v");
    KDN_REQUIRE(alpha, "alpha");
    KDN_REQUIRE(omega, "omega");
    KDN_REQUIRE(r, "r");
    KDN_REQUIRE(S, "S");
    KDN_REQUIRE(var_state, "var_state");
    KDN_REQUIRE(o, "o");
    KDN_ALIGNED(S, "S");
    if (o == q || o == k || o == v)
        return fail(KDN_ERR_INVALID_ARG, "o must not alias q, k or v");
    st = check_ext(x, nullptr, r, o, S, var_state);
    if (st != KDN_OK)
        return st;
    kdn::StepArgs a{q, k, v, alpha, omega, r, S, var_state, o, B, H, dk, dv, mu, x.mu_h, x.beta_eff};
    hipError_t e = kdn::launch_step(a, iso, io_dtype, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(KDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

kdn_status kdn_step(int variant, int B, int H, int dk, int dv, int io_dtype, float mu,
                    const void* q, const void* k, const void* v, const float* alpha,
                    const float* omega, const float* r, float* S, float* var_state, void* o,
                    void* stream)
{
    return step_impl(variant, B, H, dk, dv, io_dtype, mu, q, k, v, alpha, omega, r, S, var_state,
                     o, stream);
}

kdn_status kdn_fwd_ex(int variant, int B, int T, int H, int dk, int dv, int io_dtype, float mu,
                      const float* mu_h, const void* q, const void* k, const void* v,
                      const float* alpha, const float* omega, const float* r, const float* S0,
                      const float* var0, const float* c0_h, void* o, float* S_T, float* var_T,
                      float* beta_eff, void* workspace, size_t workspace_bytes, void* stream)
{
    if (variant != KDN_DIAG && variant != KDN_ISO)
        return fail(KDN_ERR_INVALID_ARG, "variant must be KDN_DIAG (0) or KDN_ISO (1), got %d",
                    variant);
    ExtOpts x;
    x.mu_h = mu_h;
    x.c0_h = c0_h;
    x.beta_eff = beta_eff;
    return fwd_impl(variant == KDN_ISO, B, T, H, dk, dv, io_dtype, mu, q, k, v, alpha, omega, r,
                    S0, var0, o, S_T, var_T, workspace, workspace_bytes, stream, x);
}

kdn_status kdn_dense_fwd(int B, int T, int H, int dk, int dv, int io_dtype, const void* q,
                         const void* k, const void* v, const float* alpha, const float* omega,
                         const float* r, const float* S0, const float* P0, void* o, float* S_T,
                         float* P_T, float* beta_eff, void* stream)
{
    if (io_dtype != KDN_F32 && io_dtype != KDN_BF16)
        return fail(KDN_ERR_INVALID_ARG, "io_dtype must be KDN_F32 (0) or KDN_BF16 (1), got %d",
                    io_dtype);
    if (B < 1 || H < 1 || T < 0)
        return fail(KDN_ERR_INVALID_ARG, "need B >= 1, H >= 1, T >= 0 (got B=%d T=%d H=%d)", B, T, H);
    if (dk != 16 && dk != 32 && dk != 64)
        return fail(KDN_ERR_UNSUPPORTED, "dense filter supports dk in {16, 32, 64}, got %d", dk);
    if (dv != 16 && dv != 32 && dv != 64 && dv != 128)
        return fail(KDN_ERR_UNSUPPORTED, "dense filter supports dv in {16, 32, 64, 128}, got %d", dv);
    if (!below_2_31({(size_t)B, (size_t)(T > 0 ? T : 1), (size_t)H, (size_t)(dk > dv ? dk : dv)}))
        return fail(KDN_ERR_UNSUPPORTED, "tensor sizes must stay below 2^31 elements");
    if (T > 0) {
        KDN_REQUIRE(q, "q");
        KDN_REQUIRE(k, "k");
        KDN_REQUIRE(v, "v");
        KDN_REQUIRE(alpha, "alpha");
        KDN_REQUIRE(omega, "omega");
        KDN_REQUIRE(r, "r");
        KDN_REQUIRE(o, "o");
    }
    KDN_REQUIRE(S_T, "S_T");
    KDN_REQUIRE(P_T, "P_T");
    KDN_ALIGNED_X(S0, "S0");
    KDN_ALIGNED_X(P0, "P0");
    KDN_ALIGNED_X(S_T, "S_T");
    KDN_ALIGNED_X(P_T, "P_T");
    KDN_ALIGNED_X(beta_eff, "beta_eff");
    if (o && (o == q || o == k || o == v))
        return fail(KDN_ERR_INVALID_ARG, "o must not alias q, k or v");
    auto overlap = [](const void* x, const void* y, size_t bytes) {
        const char *a0 = (const char*)x, *a1 = (const char*)y;
        return x && y && x != y && a0 < a1 + bytes && a1 < a0 + bytes;
    };
    if (overlap(S0, S_T, (size_t)B * H * dk * dv * sizeof(float)))
        return fail(KDN_ERR_INVALID_ARG, "S_T must either equal S0 or not overlap it");
    if (overlap(P0, P_T, (size_t)B * H * dk * dk * sizeof(float)))
        return fail(KDN_ERR_INVALID_ARG, "P_T must either equal P0 or not overlap it");
    if (beta_eff && (beta_eff == r || (void*)beta_eff == o || beta_eff == S_T || beta_eff == P_T))
        return fail(KDN_ERR_INVALID_ARG, "beta_eff must not alias r, o, S_T or P_T");
    kdn::DenseArgs a{q, k, v, alpha, omega, r, S0, P0, o, S_T, P_T, T > 0 ? beta_eff : nullptr,
                     B, T, H, dk, dv};
    hipError_t e = kdn::launch_dense_fwd(a, io_dtype, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(KDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

static size_t round64f(size_t n) { return (n + 63) & ~(size_t)63; }

size_t kdn_fwd_preact_workspace_size(int variant, int B, int T, int H, int dk)
{
    if ((variant != KDN_DIAG && variant != KDN_ISO) || B < 1 || H < 1 || T < 0 || dk < 1 ||
        !below_2_31({(size_t)B, (size_t)(T > 0 ? T : 1), (size_t)H, (size_t)dk}))
        return 0;
    const size_t ntok = (size_t)B * T * H;
    return (round64f(ntok * dk) + round64f(variant == KDN_ISO ? ntok : ntok * dk) +
            round64f(ntok)) * sizeof(float);
}

kdn_status kdn_fwd_preact(int variant, int B, int T, int H, int dk, int dv, int io_dtype,
                          float mu, const float* mu_h, const void* q, const void* k,
                          const void* v, const void* a_pre, const void* w_pre, const void* r_pre,
                          float r_min, const float* S0, const float* var0, const float* c0_h,
                          void* o, float* S_T, float* var_T, float* beta_eff, void* workspace,
                          size_t workspace_bytes, void* stream)
{
    if (variant != KDN_DIAG && variant != KDN_ISO)
        return fail(KDN_ERR_INVALID_ARG, "variant must be KDN_DIAG (0) or KDN_ISO (1), got %d",
                    variant);
    int io;
    bool math_bf16, out_f32;
    kdn_status st = split_io(io_dtype, io, math_bf16, out_f32);
    if (st != KDN_OK)
        return st;
    if (B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1)
        return fail(KDN_ERR_INVALID_ARG, "need B >= 1, H >= 1, T >= 0 (got B=%d T=%d H=%d)", B, T, H);
    if (!(r_min > 0.f) || r_min > 3.0e38f)
        return fail(KDN_ERR_INVALID_ARG, "r_min must be finite and > 0 (got %g)", (double)r_min);
    const bool iso = variant == KDN_ISO;
    if (T > 0) {
        KDN_REQUIRE(a_pre, "a_pre");
        KDN_REQUIRE(w_pre, "w_pre");
        KDN_REQUIRE(r_pre, "r_pre");
    }
    KDN_ALIGNED(a_pre, "a_pre");
    KDN_ALIGNED(w_pre, "w_pre");
    KDN_ALIGNED(r_pre, "r_pre");
    const size_t need = kdn_fwd_preact_workspace_size(variant, B, T, H, dk);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(KDN_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                    workspace_bytes);
    KDN_ALIGNED(workspace, "workspace");
    // the workspace (which receives the gates) must be disjoint from every argument
    const size_t es = io == KDN_BF16 ? 2 : 4;
    const size_t ntok = (size_t)B * T * H, bh = (size_t)B * H;
    const size_t nw = iso ? ntok : ntok * dk, nvar = iso ? bh : bh * dk;
    struct Buf { const void* p; size_t n; const char* name; };
    const Buf bufs[] = {{q, ntok * dk * es, "q"}, {k, ntok * dk * es, "k"},
                        {v, ntok * dv * es, "v"}, {a_pre, ntok * dk * es, "a_pre"},
                        {w_pre, nw * es, "w_pre"}, {r_pre, ntok * es, "r_pre"},
                        {o, ntok * dv * (out_f32 ? 4 : es), "o"}, {S0, bh * dk * dv * 4, "S0"},
                        {S_T, bh * dk * dv * 4, "S_T"}, {var0, nvar * 4, "var0"},
                        {var_T, nvar * 4, "var_T"}, {beta_eff, ntok * 4, "beta_eff"},
                        {mu_h, (size_t)H * 4, "mu_h"}, {c0_h, (size_t)H * 4, "c0_h"}};
    if (workspace && need)
        for (const Buf& b : bufs) {
            const char *w0 = (const char*)workspace, *b0 = (const char*)b.p;
            if (b.p && b.n && w0 < b0 + b.n && b0 < w0 + need)
                return fail(KDN_ERR_INVALID_ARG, "workspace must not overlap %s", b.name);
        }
    float* alpha = static_cast<float*>(workspace);
    float* omega = alpha + round64f(ntok * dk);
    float* r = omega + round64f(nw);
    kdn::PrologueArgs pa{a_pre, w_pre, r_pre, alpha, omega, r, ntok * dk, nw, ntok, r_min};
    ExtOpts x;
    x.mu_h = mu_h;
    x.c0_h = c0_h;
    x.beta_eff = beta_eff;
    return fwd_impl(iso, B, T, H, dk, dv, io_dtype, mu, q, k, v, T > 0 ? alpha : nullptr,
                    T > 0 ? omega : nullptr, T > 0 ? r : nullptr, S0, var0, o, S_T, var_T, nullptr,
                    0, stream, x, &pa);
}

kdn_status kdn_gates_from_preact(int variant, int B, int T, int H, int dk, int io_dtype,
                                 const void* a_pre, const void* w_pre, const void* r_pre,
                                 float r_min, float* alpha, float* omega, float* r,
                                 void* stream)
{
    if (variant != KDN_DIAG && variant != KDN_ISO)
        return fail(KDN_ERR_INVALID_ARG, "variant must be KDN_DIAG (0) or KDN_ISO (1), got %d",
                    variant);
    if (io_dtype != KDN_F32 && io_dtype != KDN_BF16)
        return fail(KDN_ERR_INVALID_ARG, "io_dtype must be KDN_F32 (0) or KDN_BF16 (1), got %d",
                    io_dtype);
    if (B < 1 || H < 1 || T < 0 || dk < 1)
        return fail(KDN_ERR_INVALID_ARG, "need B >= 1, H >= 1, T >= 0, dk >= 1 (got B=%d T=%d H=%d dk=%d)",
                    B, T, H, dk);
    if (!below_2_31({(size_t)B, (size_t)(T > 0 ? T : 1), (size_t)H, (size_t)dk}))
        return fail(KDN_ERR_UNSUPPORTED, "tensor sizes must stay below 2^31 elements");
    if (!(r_min > 0.f) || r_min > 3.0e38f)
        return fail(KDN_ERR_INVALID_ARG, "r_min must be finite and > 0 (got %g)", (double)r_min);
    if (T == 0)
        return ok();
    KDN_REQUIRE(a_pre, "a_pre");
    KDN_REQUIRE(w_pre, "w_pre");
    KDN_REQUIRE(r_pre, "r_pre");
    KDN_REQUIRE(alpha, "alpha");
    KDN_REQUIRE(omega, "omega");
    KDN_REQUIRE(r, "r");
    KDN_ALIGNED(a_pre, "a_pre");
    KDN_ALIGNED(w_pre, "w_pre");
    KDN_ALIGNED(r_pre, "r_pre");
    KDN_ALIGNED(alpha, "alpha");
    KDN_ALIGNED(omega, "omega");
    KDN_ALIGNED(r, "r");
    const bool iso = variant == KDN_ISO;
    const size_t es = io_dtype == KDN_BF16 ? 2 : 4;
    const size_t ntok = (size_t)B * T * H, na = ntok * dk, nw = iso ? ntok : na;
    struct Buf { const void* p; size_t n; const char* name; };
    const Buf bufs[] = {{a_pre, na * es, "a_pre"}, {w_pre, nw * es, "w_pre"},
                        {r_pre, ntok * es, "r_pre"}, {alpha, na * 4, "alpha"},
                        {omega, nw * 4, "omega"}, {r, ntok * 4, "r"}};
    for (int x = 3; x < 6; ++x)
        for (int y = 0; y < 6; ++y) {
            if (x == y)
                continue;
            const char *a0 = (const char*)bufs[x].p, *b0 = (const char*)bufs[y].p;
            if (a0 < b0 + bufs[y].n && b0 < a0 + bufs[x].n)
                return fail(KDN_ERR_INVALID_ARG, "%s must not overlap %s", bufs[x].name,
                            bufs[y].name);
        }
    kdn::PrologueArgs pa{a_pre, w_pre, r_pre, alpha, omega, r, na, nw, ntok, r_min};
    hipError_t e = kdn::launch_gate_prologue(pa, io_dtype, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(KDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

size_t kdn_bwd_workspace_size(int variant, int B, int T, int H, int dk, int dv)
{
    if ((variant != KDN_DIAG && variant != KDN_ISO) || B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1 ||
        !below_2_31({(size_t)B, (size_t)(T > 0 ? T : 1), (size_t)H, (size_t)(dk > dv ? dk : dv)}))
        return 0;
    const bool iso = variant == KDN_ISO;
    const int nseg = kdn::bwd_segments(iso, B, T, H, dk, dv);
    return (kdn::bwd_workspace_floats(iso, B, T, H, dk, dv) +
            (nseg ? kdn::bwd_seg_workspace_floats(iso, B, T, H, dk, nseg) : 0)) *
           sizeof(float);
}

static kdn_status bwd_impl(int variant, int B, int T, int H, int dk, int dv, int io_dtype,
                           float mu, const float* mu_h, const void* q, const void* k,
                           const void* v, const float* alpha, const float* omega, const float* r,
                           const float* S0, const float* var0, const float* c0_h,
                           const void* d_o, const float* dS_T, const float* dvar_T, void* dq,
                           void* dk_out, void* dv_out, float* dalpha, float* domega, float* dr,
                           float* dS0, float* dvar0, float* dmu, void* workspace,
                           size_t workspace_bytes, void* stream,
                           const kdn::PrologueArgs* pro = nullptr)
{
    if (variant != KDN_DIAG && variant != KDN_ISO)
        return fail(KDN_ERR_INVALID_ARG, "variant must be KDN_DIAG (0) or KDN_ISO (1), got %d",
                    variant);
    if (io_dtype != KDN_F32 && io_dtype != KDN_BF16)
        return fail(KDN_ERR_INVALID_ARG, "io_dtype must be KDN_F32 (0) or KDN_BF16 (1), got %d",
                    io_dtype);
    if (B < 1 || H < 1 || T < 0)
        return fail(KDN_ERR_INVALID_ARG, "need B >= 1, H >= 1, T >= 0 (got B=%d T=%d H=%d)", B, T, H);
    if (!(mu >= 0.f) || mu > 3.0e38f)
        return fail(KDN_ERR_INVALID_ARG, "mu must be finite and >= 0 (got %g)", (double)mu);
    if (dk != 64 && dk != 128)
        return fail(KDN_ERR_UNSUPPORTED, "backward supports dk in {64, 128}, got %d", dk);
    if (dv < 16 || dv > 256 || dv % 16 != 0)
        return fail(KDN_ERR_UNSUPPORTED, "backward supports dv a multiple of 16 up to 256, got %d", dv);
    if (!below_2_31({(size_t)B, (size_t)(T > 0 ? T : 1), (size_t)H, (size_t)(dk > dv ? dk : dv)}))
        return fail(KDN_ERR_UNSUPPORTED, "tensor sizes must stay below 2^31 elements");
    const bool iso = variant == KDN_ISO;
    if (var0 && c0_h)
        return fail(KDN_ERR_INVALID_ARG, "give the initial variance either as var0 or as c0_h, not both");
    if (T > 0) {
        KDN_REQUIRE(q, "q");
        KDN_REQUIRE(k, "k");
        KDN_REQUIRE(v, "v");
        KDN_REQUIRE(alpha, "alpha");
        KDN_REQUIRE(omega, "omega");
        KDN_REQUIRE(r, "r");
        KDN_REQUIRE(d_o, "d_o");
        KDN_REQUIRE(dq, "dq");
        KDN_REQUIRE(dk_out, "dk");
        KDN_REQUIRE(dv_out, "dv");
        KDN_REQUIRE(dalpha, "dalpha");
        KDN_REQUIRE(domega, "domega");
        KDN_REQUIRE(dr, "dr");
    }
    const size_t es = io_dtype == KDN_BF16 ? 2 : 4;
    // inputs are staged with 16-byte copies
    KDN_ALIGNED(q, "q");
    KDN_ALIGNED(k, "k");
    KDN_ALIGNED(v, "v");
    KDN_ALIGNED(d_o, "d_o");
    KDN_ALIGNED(alpha, "alpha");
    const void* io_ptrs[] = {dq, dk_out, dv_out};
    const char* io_names[] = {"dq", "dk", "dv"};
    for (int i = 0; i < 3; ++i)
        if ((uintptr_t)io_ptrs[i] % es)
            return fail(KDN_ERR_INVALID_ARG, "%s must be aligned to its element size", io_names[i]);
    KDN_ALIGNED_X(omega, "omega");
    KDN_ALIGNED_X(r, "r");
    KDN_ALIGNED_X(S0, "S0");
    KDN_ALIGNED_X(var0, "var0");
    KDN_ALIGNED_X(c0_h, "c0_h");
    KDN_ALIGNED_X(mu_h, "mu_h");
    KDN_ALIGNED_X(dS_T, "dS_T");
    KDN_ALIGNED_X(dvar_T, "dvar_T");
    KDN_ALIGNED_X(dalpha, "dalpha");
    KDN_ALIGNED_X(domega, "domega");
    KDN_ALIGNED_X(dr, "dr");
    KDN_ALIGNED_X(dS0, "dS0");
    KDN_ALIGNED_X(dvar0, "dvar0");
    KDN_ALIGNED_X(dmu, "dmu");
    // every gradient output must be disjoint from every other buffer
    const size_t ntok = (size_t)B * T * H, bh = (size_t)B * H;
    const size_t nvar = iso ? bh : bh * dk;
    struct Buf { const void* p; size_t n; const char* name; bool out; };
    const Buf bufs[] = {
        {q, ntok * dk * es, "q", false}, {k, ntok * dk * es, "k", false},
        {v, ntok * dv * es, "v", false}, {alpha, ntok * dk * 4, "alpha", false},
        {omega, (iso ? ntok : ntok * dk) * 4, "omega", false}, {r, ntok * 4, "r", false},
        {S0, bh * dk * dv * 4, "S0", false}, {var0, nvar * 4, "var0", false},
        {c0_h, (size_t)H * 4, "c0_h", false}, {mu_h, (size_t)H * 4, "mu_h", false},
        {d_o, ntok * dv * es, "d_o", false}, {dS_T, bh * dk * dv * 4, "dS_T", false},
        {dvar_T, nvar * 4, "dvar_T", false}, {workspace, workspace_bytes, "workspace", false},
        {dq, ntok * dk * es, "dq", true}, {dk_out, ntok * dk * es, "dk", true},
        {dv_out, ntok * dv * es, "dv", true}, {dalpha, ntok * dk * 4, "dalpha", true},
        {domega, (iso ? ntok : ntok * dk) * 4, "domega", true}, {dr, ntok * 4, "dr", true},
        {dS0, bh * dk * dv * 4, "dS0", true}, {dvar0, nvar * 4, "dvar0", true},
        {dmu, bh * 4, "dmu", true}};
    const int nbufs = (int)(sizeof(bufs) / sizeof(bufs[0]));
    for (int i = 0; i < nbufs; ++i) {
        if (!bufs[i].out || !bufs[i].p || !bufs[i].n)
            continue;
        for (int j = 0; j < nbufs; ++j) {
            if (j == i || !bufs[j].p || !bufs[j].n)
                continue;
            const char *a0 = (const char*)bufs[i].p, *a1 = (const char*)bufs[j].p;
            if (a0 < a1 + bufs[j].n && a1 < a0 + bufs[i].n)
                return fail(KDN_ERR_INVALID_ARG, "%s must not overlap %s", bufs[i].name,
                            bufs[j].name);
        }
    }
    // the base workspace is required; the split over the sequence (bf16 io,
    // shapes that leave most compute units idle) runs when the workspace also
    // holds its planes
    const size_t need = kdn::bwd_workspace_floats(iso, B, T, H, dk, dv) * sizeof(float);
    if (workspace_bytes < need || (need && !workspace))
        return fail(KDN_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                    workspace_bytes);
    const int nseg = io_dtype == KDN_BF16 ? kdn::bwd_segments(iso, B, T, H, dk, dv) : 0;
    const size_t seg_bytes =
        nseg ? kdn::bwd_seg_workspace_floats(iso, B, T, H, dk, nseg) * sizeof(float) : 0;
    const bool split = nseg && workspace_bytes - need >= seg_bytes;
    if ((uintptr_t)workspace % 16)
        return fail(KDN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    kdn::BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.omega = omega; a.r = r;
    a.S0 = S0; a.var0 = var0; a.c0 = c0_h; a.mu_h = mu_h; a.mu = mu;
    a.go = d_o; a.gS_T = dS_T; a.gvar_T = dvar_T;
    a.gq = dq; a.gk = dk_out; a.gv = dv_out; a.galpha = dalpha; a.gomega = domega; a.gr = dr;
    a.gS0 = dS0; a.gvar0 = dvar0; a.gmu = dmu;
    a.B = B; a.T = T; a.H = H; a.dk = dk; a.dv = dv;
    kdn::bwd_carve_workspace(a, iso, static_cast<float*>(workspace));
    if (split) {
        a.nseg = nseg;
        a.segws = static_cast<float*>(workspace) + need / sizeof(float);
    }
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (pro && T > 0) {  // the gates from their pre-activations
        hipError_t e = kdn::launch_gate_prologue(*pro, io_dtype, hs);
        if (e != hipSuccess)
            return fail(KDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
    hipError_t e = kdn::launch_bwd(a, iso, io_dtype, hs);
    if (e == hipSuccess && pro && T > 0)  // and the chain rule back through them
        e = kdn::launch_gate_epilogue(*pro, dalpha, domega, dr, io_dtype, hs);
    if (e != hipSuccess)
        return fail(KDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

kdn_status kdn_bwd(int variant, int B, int T, int H, int dk, int dv, int io_dtype, float mu,
                   const float* mu_h, const void* q, const void* k, const void* v,
                   const float* alpha, const float* omega, const float* r, const float* S0,
                   const float* var0, const float* c0_h, const void* d_o, const float* dS_T,
                   const float* dvar_T, void* dq, void* dk_out, void* dv_out, float* dalpha,
                   float* domega, float* dr, float* dS0, float* dvar0, float* dmu,
                   void* workspace, size_t workspace_bytes, void* stream)
{
    return bwd_impl(variant, B, T, H, dk, dv, io_dtype, mu, mu_h, q, k, v, alpha, omega, r, S0,
                    var0, c0_h, d_o, dS_T, dvar_T, dq, dk_out, dv_out, dalpha, domega, dr, dS0,
                    dvar0, dmu, workspace, workspace_bytes, stream);
}

size_t kdn_bwd_preact_workspace_size(int variant, int B, int T, int H, int dk, int dv)
{
    if ((variant != KDN_DIAG && variant != KDN_ISO) || B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1)
        return 0;
    return kdn_fwd_preact_workspace_size(variant, B, T, H, dk) +
           kdn_bwd_workspace_size(variant, B, T, H, dk, dv);
}

kdn_status kdn_bwd_preact(int variant, int B, int T, int H, int dk, int dv, int io_dtype,
                          float mu, const float* mu_h, const void* q, const void* k,
                          const void* v, const void* a_pre, const void* w_pre, const void* r_pre,
                          float r_min, const float* S0, const float* var0, const float* c0_h,
                          const void* d_o, const float* dS_T, const float* dvar_T, void* dq,
                          void* dk_out, void* dv_out, float* da_pre, float* dw_pre, float* dr_pre,
                          float* dS0, float* dvar0, float* dmu, void* workspace,
                          size_t workspace_bytes, void* stream)
{
    if (variant != KDN_DIAG && variant != KDN_ISO)
        return fail(KDN_ERR_INVALID_ARG, "variant must be KDN_DIAG (0) or KDN_ISO (1), got %d",
                    variant);
    int io;
    bool math_bf16, out_f32;
    kdn_status st = split_io(io_dtype, io, math_bf16, out_f32);
    if (st != KDN_OK)
        return st;
    if (B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1)
        return fail(KDN_ERR_INVALID_ARG, "need B >= 1, H >= 1, T >= 0 (got B=%d T=%d H=%d)", B, T, H);
    if (!(r_min > 0.f) || r_min > 3.0e38f)
        return fail(KDN_ERR_INVALID_ARG, "r_min must be finite and > 0 (got %g)", (double)r_min);
    if (T > 0) {
        KDN_REQUIRE(a_pre, "a_pre");
        KDN_REQUIRE(w_pre, "w_pre");
        KDN_REQUIRE(r_pre, "r_pre");
    }
    KDN_ALIGNED(a_pre, "a_pre");
    KDN_ALIGNED(w_pre, "w_pre");
    KDN_ALIGNED(r_pre, "r_pre");
    const size_t gates = kdn_fwd_preact_workspace_size(variant, B, T, H, dk);
    const size_t need = kdn_bwd_preact_workspace_size(variant, B, T, H, dk, dv);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(KDN_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                    workspace_bytes);
    KDN_ALIGNED(workspace, "workspace");
    const bool iso = variant == KDN_ISO;
    const size_t es = io_dtype == KDN_BF16 ? 2 : 4;
    const size_t ntok = (size_t)B * T * H, nw = iso ? ntok : ntok * dk;
    // the pre-activations are inputs: no output or workspace may overlap them
    const struct { const void* p; size_t n; const char* name; } pres[] = {
        {a_pre, ntok * dk * es, "a_pre"}, {w_pre, nw * es, "w_pre"}, {r_pre, ntok * es, "r_pre"}};
    const struct { const void* p; size_t n; const char* name; } outs[] = {
        {workspace, need, "workspace"}, {dq, ntok * dk * es, "dq"}, {dk_out, ntok * dk * es, "dk"},
        {dv_out, ntok * dv * es, "dv"}, {da_pre, ntok * dk * 4, "da_pre"},
        {dw_pre, nw * 4, "dw_pre"}, {dr_pre, ntok * 4, "dr_pre"},
        {dS0, (size_t)B * H * dk * dv * 4, "dS0"}, {dvar0, (iso ? 1 : (size_t)dk) * B * H * 4, "dvar0"},
        {dmu, (size_t)B * H * 4, "dmu"}};
    for (const auto& o : outs)
        for (const auto& p : pres) {
            const char *a0 = (const char*)o.p, *b0 = (const char*)p.p;
            if (o.p && p.p && o.n && p.n && a0 < b0 + p.n && b0 < a0 + o.n)
                return fail(KDN_ERR_INVALID_ARG, "%s must not overlap %s", o.name, p.name);
        }
    float* alpha = static_cast<float*>(workspace);
    float* omega = alpha + round64f(ntok * dk);
    float* r = omega + round64f(nw);
    kdn::PrologueArgs pa{a_pre, w_pre, r_pre, alpha, omega, r, ntok * dk, nw, ntok, r_min};
    return bwd_impl(variant, B, T, H, dk, dv, io_dtype, mu, mu_h, q, k, v,
                    T > 0 ? alpha : nullptr, T > 0 ? omega : nullptr, T > 0 ? r : nullptr, S0,
                    var0, c0_h, d_o, dS_T, dvar_T, dq, dk_out, dv_out, da_pre, dw_pre, dr_pre,
                    dS0, dvar0, dmu, static_cast<char*>(workspace) + gates, workspace_bytes - gates,
                    stream, &pa);
}

kdn_status kdn_step_ex(int variant, int B, int H, int dk, int dv, int io_dtype, float mu,
                       const float* mu_h, const void* q, const void* k, const void* v,
                       const float* alpha, const float* omega, const float* r, float* S,
                       float* var_state, void* o, float* beta_eff, void* stream)
{
    ExtOpts x;
    x.mu_h = mu_h;
    x.beta_eff = beta_eff;
    return step_impl(variant, B, H, dk, dv, io_dtype, mu, q, k, v, alpha, omega, r, S, var_state,
                     o, stream, x);
}

size_t kdn_gain_workspace_size(int variant, int B, int T, int H, int dk)
{
    if (B < 1 || H < 1 || T < 0 || (dk != 64 && dk != 128) ||
        !below_2_31({(size_t)B, (size_t)(T > 0 ? T : 1), (size_t)H, (size_t)dk}))
        return 0;
    return kdn::gain_workspace_floats(variant == KDN_ISO, B, T, H, dk) * sizeof(float);
}

}  // extern "C"

namespace {

// Argument checks shared by the gain scan's two entry points.
kdn_status gain_check(int variant, int B, int T, int H, int dk, int io_dtype, float mu,
                      const void* k, const float* alpha, const float* omega, const float* r,
                      const float* var0, const float* var_T)
{
    if (variant != KDN_DIAG && variant != KDN_ISO)
        return fail(KDN_ERR_INVALID_ARG, "variant must be KDN_DIAG (0) or KDN_ISO (1), got %d",
                    variant);
    if (io_dtype != KDN_F32 && io_dtype != KDN_BF16)
        return fail(KDN_ERR_INVALID_ARG, "io_dtype must be KDN_F32 (0) or KDN_BF16 (1), got %d",
                    io_dtype);
    if (B < 1 || H < 1 || T < 0)
        return fail(KDN_ERR_INVALID_ARG, "need B >= 1, H >= 1, T >= 0");
    if (dk != 64 && dk != 128)
        return fail(KDN_ERR_UNSUPPORTED, "gain scan supports dk in {64, 128}, got %d", dk);
    if (!(mu >= 0.f) || !std::isfinite(mu))
        return fail(KDN_ERR_INVALID_ARG, "mu must be finite and >= 0");
    if (!below_2_31({(size_t)B, (size_t)(T > 0 ? T : 1), (size_t)H, (size_t)dk}))
        return fail(KDN_ERR_UNSUPPORTED, "tensor sizes must stay below 2^31 elements");
    if (T > 0) {
        KDN_REQUIRE(k, "k");
        KDN_REQUIRE(alpha, "alpha");
        KDN_REQUIRE(omega, "omega");
        KDN_REQUIRE(r, "r");
    }
    KDN_REQUIRE(var_T, "var_T");
    KDN_ALIGNED(alpha, "alpha");
    if (var0 && var0 == var_T)
        return fail(KDN_ERR_INVALID_ARG, "var_T must not alias var0");
    return KDN_OK;
}

kdn_status gain_launch(int variant, int B, int T, int H, int dk, int io_dtype, float mu,
                       const void* k, const float* alpha, const float* omega, const float* r,
                       const float* var0, float* kappa, float* var_T, float* ws, void* stream)
{
    const bool iso = variant == KDN_ISO;
    const size_t nchunks = (size_t)(T + 63) / 64;
    const size_t width = iso ? 1 : (size_t)dk;
    kdn::GainArgs a{k,     alpha, omega, r, var0, kappa, var_T, ws,
                    ws + (size_t)B * H * 4 * width * nchunks, B, T, H, dk, mu};
    hipError_t e = kdn::launch_gain_scan(a, iso, io_dtype, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(KDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

kdn_status kdn_gain_scan(int variant, int B, int T, int H, int dk, int io_dtype, float mu,
                         const void* k, const float* alpha, const float* omega, const float* r,
                         const float* var0, float* kappa, float* var_T, void* workspace,
                         size_t workspace_bytes, void* stream)
{
    kdn_status st = gain_check(variant, B, T, H, dk, io_dtype, mu, k, alpha, omega, r, var0, var_T);
    if (st != KDN_OK)
        return st;
    const size_t need = kdn_gain_workspace_size(variant, B, T, H, dk);
    if (workspace_bytes < need || !workspace)
        return fail(KDN_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                    workspace_bytes);
    if (!aligned16(workspace))
        return fail(KDN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    return gain_launch(variant, B, T, H, dk, io_dtype, mu, k, alpha, omega, r, var0, kappa, var_T,
                       static_cast<float*>(workspace), stream);
}

size_t kdn_gain_scan_static_max_bytes(void)
{
    return kdn::gain_static_scratch_floats() * sizeof(float);
}

kdn_status kdn_gain_scan_static(int variant, int B, int T, int H, int dk, int io_dtype, float mu,
                                const void* k, const float* alpha, const float* omega,
                                const float* r, const float* var0, float* kappa, float* var_T,
                                void* stream)
{
    kdn_status st = gain_check(variant, B, T, H, dk, io_dtype, mu, k, alpha, omega, r, var0, var_T);
    if (st != KDN_OK)
        return st;
    const size_t need = kdn_gain_workspace_size(variant, B, T, H, dk);
    const size_t have = kdn_gain_scan_static_max_bytes();
    if (need > have)
        return fail(KDN_ERR_WORKSPACE,
                    "this shape needs %zu bytes of scratch; the static scratch of "
                    "kdn_gain_scan_static holds %zu (use kdn_gain_scan with a workspace)",
                    need, have);
    float* ws = nullptr;
    hipError_t e = kdn::gain_static_scratch(&ws);
    if (e != hipSuccess)
        return fail(KDN_ERR_HIP, "static scratch lookup failed: %s", hipGetErrorString(e));
    return gain_launch(variant, B, T, H, dk, io_dtype, mu, k, alpha, omega, r, var0, kappa, var_T,
                       ws, stream);
}

const char* kdn_status_string(int status)
{
    switch (status) {
    case KDN_OK:
        return "KDN_OK";
    case KDN_ERR_INVALID_ARG:
        return "KDN_ERR_INVALID_ARG";
    case KDN_ERR_UNSUPPORTED:
        return "KDN_ERR_UNSUPPORTED";
    case KDN_ERR_WORKSPACE:
        return "KDN_ERR_WORKSPACE";
    case KDN_ERR_HIP:
        return "KDN_ERR_HIP";
    default:
        return "KDN_ERR_UNKNOWN";
    }
}

const char* kdn_last_error_message(void) { return g_msg; }

const char* kdn_version(void) { return "kdn-mi355x 0.1.0 gfx950"; }

}  // extern "C"
