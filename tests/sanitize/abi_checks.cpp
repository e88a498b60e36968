// The C ABI's host code (argument validation, aliasing rules, workspace
// planning) driven through every entry point with stand-in device addresses,
// built with the address and undefined-behaviour sanitizers against the
// launch stand-ins of launch_stubs.cpp.  Exits nonzero on the first failed
// expectation; the sanitizers abort on any memory or UB error.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "kdn.h"

extern int g_launches;

static int failures = 0;

#define EXPECT(cond)                                                              \
    do {                                                                          \
        if (!(cond)) {                                                            \
            std::printf("FAILED %s:%d: %s (last error: %s)\n", __FILE__, __LINE__, \
                        #cond, kdn_last_error_message());                         \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

static void* at(uint64_t a) { return reinterpret_cast<void*>(a); }
static float* fat(uint64_t a) { return reinterpret_cast<float*>(a); }
static bool said(const char* needle) { return std::strstr(kdn_last_error_message(), needle) != nullptr; }

static const uint64_t P = 1ull << 20;  // a 16-byte aligned stand-in address
static const uint64_t FAR = 1ull << 40;

struct Fwd {
    int variant = KDN_DIAG, B = 1, T = 64, H = 2, dk = 64, dv = 64, io = KDN_BF16;
    float mu = 64.f;
    uint64_t q = P, k = P, v = P, alpha = P, omega = P, r = P, S0 = 0, var0 = 0;
    uint64_t o = P + 4096, S_T = P + 8192, var_T = P + 16384, ws = 0;
    size_t ws_bytes = 0;
    kdn_status call() const
    {
        return (variant == KDN_DIAG ? kdn_diag_fwd : kdn_iso_fwd)(
            B, T, H, dk, dv, io, mu, at(q), at(k), at(v), fat(alpha), fat(omega), fat(r),
            fat(S0), fat(var0), at(o), fat(S_T), fat(var_T), at(ws), ws_bytes, nullptr);
    }
};

static void fwd_checks(int variant)
{
    Fwd f;
    f.variant = variant;
    auto bad = [&](Fwd g, kdn_status code, const char* needle) {
        const kdn_status st = g.call();
        if (st != code || !said(needle)) {
            std::printf("FAILED case '%s' (variant %d): status %d, last error: %s\n", needle,
                        variant, (int)st, kdn_last_error_message());
            ++failures;
        }
    };
    Fwd g = f;
    g.io = 2;
    bad(g, KDN_ERR_INVALID_ARG, "io_dtype");
    g = f; g.B = 0; bad(g, KDN_ERR_INVALID_ARG, "B >= 1");
    g = f; g.T = -1; bad(g, KDN_ERR_INVALID_ARG, "T >= 0");
    g = f; g.mu = NAN; bad(g, KDN_ERR_INVALID_ARG, "mu");
    g = f; g.dk = 96; bad(g, KDN_ERR_UNSUPPORTED, "dk");
    g = f; g.dv = 512; bad(g, KDN_ERR_UNSUPPORTED, "dv");
    g = f; g.q = 0; bad(g, KDN_ERR_INVALID_ARG, "q must not be NULL");
    g = f; g.r = 0; bad(g, KDN_ERR_INVALID_ARG, "r must not be NULL");
    g = f; g.q = P + 4; bad(g, KDN_ERR_INVALID_ARG, "aligned");
    g = f; g.o = P; bad(g, KDN_ERR_INVALID_ARG, "alias");
    g = f; g.S0 = P + 8192 + 64; bad(g, KDN_ERR_INVALID_ARG, "overlap");
    g = f; g.io = 0x100; bad(g, KDN_ERR_INVALID_ARG, "bf16 io only");
    g = f; g.io = 0x401; bad(g, KDN_ERR_INVALID_ARG, "io_dtype");
    g = f; g.dv = 128; g.var0 = g.var_T; bad(g, KDN_ERR_INVALID_ARG, "only when dv <= 64");
    // sizes whose element counts pass 2^31: refused before any arithmetic wraps
    g = f; g.B = 1 << 14; g.T = 1 << 14; g.H = 16; bad(g, KDN_ERR_UNSUPPORTED, "2^31");
    g = f; g.B = 1 << 30; g.T = 1 << 30; g.H = 1 << 30; bad(g, KDN_ERR_UNSUPPORTED, "2^31");
    // valid: reaches the launcher
    int before = g_launches;
    EXPECT(f.call() == KDN_ERR_HIP);
    EXPECT(g_launches == before + 1);
    g = f; g.T = 0; EXPECT(g.call() == KDN_ERR_HIP || g.call() == KDN_OK);
    // split over the sequence, with and without its workspace
    g = f; g.T = 8192; g.dk = g.dv = 128;
    g.q = g.k = g.v = g.alpha = g.omega = g.r = FAR;
    g.o = FAR + (1ull << 32); g.S_T = FAR + (2ull << 32); g.var_T = FAR + (3ull << 32);
    g.ws_bytes = kdn_fwd_workspace_size(variant, 1, 8192, 2, 128, 128, KDN_BF16);
    EXPECT(g.ws_bytes > 0);
    g.ws = FAR + (4ull << 32);
    EXPECT(g.call() == KDN_ERR_HIP);
    g.ws = FAR + 64;  // overlapping q
    EXPECT(g.call() == KDN_ERR_INVALID_ARG);
}

static void other_checks()
{
    // decode
    EXPECT(kdn_step(KDN_DIAG, 4, 2, 128, 128, KDN_BF16, 128.f, at(P), at(P), at(P), fat(P), fat(P),
                    fat(P), fat(P + 8192), fat(P + (1 << 22)), at(P + (1 << 23)), nullptr) == KDN_ERR_HIP);
    EXPECT(kdn_step(KDN_DIAG, 4, 2, 96, 128, KDN_BF16, 128.f, at(P), at(P), at(P), fat(P), fat(P),
                    fat(P), fat(P + 8192), fat(P + (1 << 22)), at(P + (1 << 23)), nullptr) == KDN_ERR_UNSUPPORTED);
    EXPECT(kdn_step(KDN_ISO, 4, 2, 128, 128, KDN_BF16, 128.f, at(P), at(P), at(P), fat(P), fat(P),
                    fat(P), nullptr, fat(P + (1 << 22)), at(P + (1 << 23)), nullptr) == KDN_ERR_INVALID_ARG);
    // gain scan
    const size_t gws = kdn_gain_workspace_size(KDN_DIAG, 1, 128, 2, 64);
    EXPECT(gws == (size_t)1 * 2 * 2 * 64 * 5 * 4);
    EXPECT(kdn_gain_scan(KDN_DIAG, 1, 128, 2, 64, KDN_BF16, 64.f, at(P), fat(P), fat(P), fat(P), nullptr,
                         fat(FAR), fat(FAR + (1 << 24)), at(FAR + (1 << 26)), gws - 1, nullptr) == KDN_ERR_WORKSPACE);
    EXPECT(kdn_gain_scan(KDN_DIAG, 1, 128, 2, 64, KDN_BF16, 64.f, at(P), fat(P), fat(P), fat(P), nullptr,
                         fat(FAR), fat(FAR + (1 << 24)), at(FAR + (1 << 26)), gws, nullptr) == KDN_ERR_HIP);
    EXPECT(kdn_gain_scan(KDN_DIAG, 1, 128, 2, 64, KDN_BF16, 64.f, at(P), fat(P), fat(P), fat(P), nullptr,
                         fat(FAR), nullptr, at(FAR + (1 << 26)), gws, nullptr) == KDN_ERR_INVALID_ARG);
    // the allocation-free gain scan: a shape beyond its static scratch is refused
    EXPECT(kdn_gain_scan_static_max_bytes() == ((size_t)8 << 20) * 4);
    EXPECT(kdn_gain_scan_static(KDN_DIAG, 1, 65536, 16, 128, KDN_BF16, 128.f, at(P), fat(P), fat(P),
                                fat(P), nullptr, nullptr, fat(FAR), nullptr) == KDN_ERR_WORKSPACE);
    EXPECT(kdn_gain_scan_static(KDN_DIAG, 1, 128, 2, 64, KDN_BF16, 64.f, at(P), fat(P), fat(P), fat(P),
                                nullptr, fat(FAR), fat(FAR + (1 << 24)), nullptr) == KDN_ERR_HIP);
    // backward: workspace too small, then enough
    const size_t bws = kdn_bwd_workspace_size(KDN_DIAG, 1, 64, 2, 64, 64);
    EXPECT(bws > 0);
    uint64_t out = FAR;
    auto next = [&]() { out += 1ull << 28; return out; };
    const uint64_t dq = next(), dk = next(), dv = next(), da = next(), dw = next(), dr = next();
    const uint64_t ws = next();
    EXPECT(kdn_bwd(KDN_DIAG, 1, 64, 2, 64, 64, KDN_BF16, 64.f, nullptr, at(P), at(P), at(P), fat(P), fat(P),
                   fat(P), nullptr, nullptr, nullptr, at(P), nullptr, nullptr, at(dq), at(dk), at(dv),
                   fat(da), fat(dw), fat(dr), nullptr, nullptr, nullptr, at(ws), bws - 1, nullptr) == KDN_ERR_WORKSPACE);
    EXPECT(kdn_bwd(KDN_DIAG, 1, 64, 2, 64, 64, KDN_BF16, 64.f, nullptr, at(P), at(P), at(P), fat(P), fat(P),
                   fat(P), nullptr, nullptr, nullptr, at(P), nullptr, nullptr, at(dq), at(dk), at(dv),
                   fat(da), fat(dw), fat(dr), nullptr, nullptr, nullptr, at(ws), bws, nullptr) == KDN_ERR_HIP);
    // a shape the backward splits over the sequence (2 segments of 1024
    // tokens): its full workspace, and one byte short of it (the same call
    // without the split), both reach the launch
    const size_t sws = kdn_bwd_workspace_size(KDN_DIAG, 1, 2048, 2, 64, 64);
    EXPECT(sws > kdn_bwd_workspace_size(KDN_ISO, 1, 2048, 2, 64, 64));
    const size_t wbs[2] = {sws, sws - 1};
    for (const size_t wb : wbs)
        EXPECT(kdn_bwd(KDN_DIAG, 1, 2048, 2, 64, 64, KDN_BF16, 64.f, nullptr, at(P), at(P), at(P), fat(P),
                       fat(P), fat(P), nullptr, nullptr, nullptr, at(P), nullptr, nullptr, at(dq), at(dk),
                       at(dv), fat(da), fat(dw), fat(dr), fat(ws), nullptr, nullptr, at(ws + (1ull << 27)),
                       wb, nullptr) == KDN_ERR_HIP);
    // forward from pre-activations
    const size_t pws = kdn_fwd_preact_workspace_size(KDN_DIAG, 1, 64, 2, 64);
    EXPECT(kdn_fwd_preact(KDN_DIAG, 1, 64, 2, 64, 64, KDN_BF16, 64.f, nullptr, at(P), at(P), at(P), at(P),
                          at(P), at(P), 0.f, nullptr, nullptr, nullptr, at(dq), fat(dk), fat(dv), nullptr,
                          at(ws), pws, nullptr) == KDN_ERR_INVALID_ARG);
    EXPECT(kdn_fwd_preact(KDN_DIAG, 1, 64, 2, 64, 64, KDN_BF16, 64.f, nullptr, at(P), at(P), at(P), at(P),
                          at(P), at(P), 0.01f, nullptr, nullptr, nullptr, at(dq), fat(dk), fat(dv), nullptr,
                          at(ws), pws, nullptr) == KDN_ERR_HIP);
    // the gates alone
    EXPECT(kdn_gates_from_preact(KDN_DIAG, 1, 64, 2, 64, KDN_BF16, at(P), at(P), at(P), -1.f, fat(dq),
                                 fat(dk), fat(dv), nullptr) == KDN_ERR_INVALID_ARG);
    EXPECT(kdn_gates_from_preact(KDN_ISO, 1, 64, 2, 64, KDN_BF16, at(P), at(P), at(P), 0.01f, fat(dq),
                                 fat(dq + 64), fat(dv), nullptr) == KDN_ERR_INVALID_ARG && said("overlap"));
    EXPECT(kdn_gates_from_preact(KDN_ISO, 1 << 30, 1 << 30, 1 << 30, 64, KDN_BF16, at(P), at(P), at(P),
                                 0.01f, fat(dq), fat(dk), fat(dv), nullptr) == KDN_ERR_UNSUPPORTED);
    EXPECT(kdn_gates_from_preact(KDN_DIAG, 1, 64, 2, 64, KDN_BF16, at(P), at(P + 65536), at(P + 131072),
                                 0.01f, fat(dq), fat(dk), fat(dv), nullptr) == KDN_ERR_HIP);
    // dense filter
    EXPECT(kdn_dense_fwd(1, 64, 2, 96, 64, KDN_BF16, at(P), at(P), at(P), fat(P), fat(P), fat(P), nullptr,
                         nullptr, at(dq), fat(dk), fat(dv), nullptr, nullptr) == KDN_ERR_UNSUPPORTED);
    EXPECT(kdn_dense_fwd(1, 64, 2, 64, 64, KDN_BF16, at(P), at(P), at(P), fat(P), fat(P), fat(P), nullptr,
                         nullptr, at(dq), fat(dk), fat(dv), nullptr, nullptr) == KDN_ERR_HIP);
    // status strings and version
    EXPECT(std::strcmp(kdn_status_string(KDN_ERR_HIP), "KDN_ERR_HIP") == 0);
    EXPECT(std::strcmp(kdn_status_string(7), "KDN_ERR_UNKNOWN") == 0);
    EXPECT(kdn_version() != nullptr && std::strlen(kdn_version()) > 0);
    // workspace sizes of shapes past every limit: 0, no wrap-around
    EXPECT(kdn_fwd_workspace_size(KDN_DIAG, 1 << 30, 1 << 30, 1 << 30, 128, 128, KDN_BF16) == 0);
    EXPECT(kdn_gain_workspace_size(KDN_DIAG, 1, 128, 2, 96) == 0);
    EXPECT(kdn_gain_workspace_size(KDN_DIAG, 1 << 30, 1 << 30, 1 << 30, 128) == 0);
    EXPECT(kdn_bwd_workspace_size(KDN_DIAG, 1 << 30, 1 << 30, 1 << 30, 128, 128) == 0);
    EXPECT(kdn_fwd_preact_workspace_size(KDN_DIAG, 1 << 30, 1 << 30, 1 << 30, 128) == 0);
    EXPECT(kdn_bwd_preact_workspace_size(KDN_ISO, 1 << 16, 1 << 16, 1, 128, 128) == 0);
}

int main()
{
    fwd_checks(KDN_DIAG);
    fwd_checks(KDN_ISO);
    other_checks();
    if (failures) {
        std::printf("%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("all checks passed (%d launches reached)\n", g_launches);
    return 0;
}
