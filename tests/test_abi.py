"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/kdn.h declares, and rejects invalid arguments synchronously
(before any launch) with the documented status codes.

The invalid-argument cases pass stand-in pointer values; they are skipped
when a GPU is visible, so that a validation gap can never turn into a launch
on fake addresses.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kdn.h")


@pytest.fixture(scope="module")
def L():
    from kalman_delta_rule_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from kalman_delta_rule_amd import build
        build.build_library()
    return _lib.lib()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kdn_[a-z_]+)\s*\(", src)))


def test_header_declares_the_three_calls():
    names = _declared_functions()
    for n in ("kdn_diag_fwd", "kdn_iso_fwd", "kdn_step"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    from kalman_delta_rule_amd import _lib
    names = _declared_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(L, n), "libkdn.so does not export %s" % n
    assert set(_lib.EXPORTED) == set(names)


def test_version_and_status_strings(L):
    assert L.kdn_version().decode().startswith("kdn-mi355x")
    assert L.kdn_status_string(0) == b"KDN_OK"
    assert L.kdn_status_string(-1) == b"KDN_ERR_INVALID_ARG"
    assert L.kdn_status_string(-2) == b"KDN_ERR_UNSUPPORTED"
    assert L.kdn_status_string(-3) == b"KDN_ERR_WORKSPACE"
    assert L.kdn_status_string(-4) == b"KDN_ERR_HIP"
    assert L.kdn_status_string(7) == b"KDN_ERR_UNKNOWN"


def test_workspace_sizes(L):
    assert L.kdn_fwd_workspace_size(0, 8, 4096, 16, 128, 128, 1) == 0
    # few heads, long sequence: 8 segments; gain scan + 2 variance planes + 4 state
    # planes (the walk that forms M takes v = 0 without reading it: no zero copy)
    gain, pin, st = 16 * 1024 * 128 * 5, 8 * 16 * 128, 8 * 16 * 128 * 128
    assert L.kdn_fwd_workspace_size(0, 1, 65536, 16, 128, 128, 1) == (gain + 2 * pin + 4 * st) * 4
    gain, pin = 16 * 1024 * 5, 8 * 16
    assert L.kdn_fwd_workspace_size(1, 1, 65536, 16, 128, 128, 1) == (gain + 2 * pin + 4 * st) * 4
    assert L.kdn_fwd_workspace_size(0, 1, 65536, 16, 128, 128, 0) == 0   # fp32 io: serial
    assert L.kdn_fwd_workspace_size(0, 1, 65536, 16, 128, 64, 1) == 0    # dk != dv
    assert L.kdn_fwd_workspace_size(0, 1, 2048, 16, 128, 128, 1) == 0    # segments too short
    # gain scan: 4 summary planes + carries per chunk and channel
    assert L.kdn_gain_workspace_size(0, 1, 128, 2, 64) == 1 * 2 * 2 * 64 * 5 * 4
    assert L.kdn_gain_workspace_size(1, 1, 128, 2, 64) == 1 * 2 * 2 * 1 * 5 * 4
    assert L.kdn_gain_workspace_size(0, 1, 128, 2, 96) == 0


# ---------------------------------------------------------------------------
# validation: every case below has exactly one invalid argument
# ---------------------------------------------------------------------------
cpu_only = pytest.mark.skipif(
    __import__("torch").cuda.is_available(),
    reason="stand-in pointers are only used where no GPU is visible")

P = 1 << 20      # a 16-byte-aligned stand-in address
MIS = P + 4      # misaligned


def _fwd_call(L, variant="diag", **kw):
    args = dict(B=1, T=64, H=2, dk=64, dv=64, io=1, mu=64.0, q=P, k=P, v=P, alpha=P, omega=P,
                r=P, S0=None, var0=None, o=P + 4096, S_T=P + 8192, var_T=P + 16384, ws=None,
                ws_bytes=0, stream=None)
    args.update(kw)
    fn = L.kdn_diag_fwd if variant == "diag" else L.kdn_iso_fwd
    a = args
    return fn(a["B"], a["T"], a["H"], a["dk"], a["dv"], a["io"], a["mu"], a["q"], a["k"], a["v"],
              a["alpha"], a["omega"], a["r"], a["S0"], a["var0"], a["o"], a["S_T"], a["var_T"],
              a["ws"], a["ws_bytes"], a["stream"])


@cpu_only
@pytest.mark.parametrize("variant", ["diag", "iso"])
@pytest.mark.parametrize("bad,code,needle", [
    (dict(io=2), -1, "io_dtype"),
    (dict(B=0), -1, "B >= 1"),
    (dict(H=0), -1, "H >= 1"),
    (dict(T=-1), -1, "T >= 0"),
    (dict(mu=-1.0), -1, "mu"),
    (dict(mu=float("nan")), -1, "mu"),
    (dict(dk=96), -2, "dk"),
    (dict(dv=96), -2, "dv"),
    (dict(dv=512), -2, "dv"),
    (dict(io=0, dk=128), -2, "fp32 forward supports dk"),
    (dict(q=None), -1, "q must not be NULL"),
    (dict(k=None), -1, "k must not be NULL"),
    (dict(v=None), -1, "v must not be NULL"),
    (dict(alpha=None), -1, "alpha"),
    (dict(omega=None), -1, "omega"),
    (dict(r=None), -1, "r must not be NULL"),
    (dict(o=None), -1, "o must not be NULL"),
    (dict(S_T=None), -1, "S_T"),
    (dict(var_T=None), -1, "_T must not be NULL"),
    (dict(q=MIS), -1, "aligned"),
    (dict(S_T=MIS), -1, "aligned"),
    (dict(o=P), -1, "alias"),
    (dict(S0=P + 8192 + 64), -1, "overlap"),
    (dict(B=1 << 14, T=1 << 14, H=16), -2, "2^31"),
])
def test_fwd_validation(L, variant, bad, code, needle):
    st = _fwd_call(L, variant, **bad)
    assert st == code
    assert needle in L.kdn_last_error_message().decode()


@cpu_only
@pytest.mark.parametrize("variant", ["diag", "iso"])
@pytest.mark.parametrize("bad,code,needle", [
    (dict(io=0x100), -1, "bf16 io only"),            # KDN_MATH_BF16 with fp32 io
    (dict(io=0x200), -1, "bf16 io only"),            # KDN_OUT_F32 with fp32 io
    (dict(io=0x301), -2, "KDN_OUT_F32 comes with"),  # both flags
    (dict(io=0x401), -1, "io_dtype"),                # an unknown flag
])
def test_fwd_precision_flag_validation(L, variant, bad, code, needle):
    st = _fwd_call(L, variant, **bad)
    assert st == code
    assert needle in L.kdn_last_error_message().decode()


@cpu_only
def test_fwd_out_f32_is_diagonal_only(L):
    assert _fwd_call(L, "iso", io=0x201) == -2
    assert "Diagonal" in L.kdn_last_error_message().decode()


@cpu_only
def test_fwd_out_f32_widens_the_output_overlap_check(L):
    # split over the sequence with its workspace: with fp32 o the workspace
    # must clear the twice larger output
    shape = dict(B=1, T=8192, H=2, dk=128, dv=128)
    need = L.kdn_fwd_workspace_size(0, 1, 8192, 2, 128, 128, 0x201)
    assert need == L.kdn_fwd_workspace_size(0, 1, 8192, 2, 128, 128, 1) > 0
    far = 1 << 40
    o = far + (1 << 32)
    obytes_bf16 = 8192 * 2 * 128 * 2
    kw = dict(shape, q=far, k=far, v=far, alpha=far, omega=far, r=far, o=o,
              S_T=far + (2 << 32), var_T=far + (3 << 32), ws_bytes=need)
    # just past where a bf16 o would end, inside the fp32 o
    assert _fwd_call(L, "diag", io=0x201, ws=o + obytes_bf16, **kw) == -1
    assert "workspace must not overlap o" in L.kdn_last_error_message().decode()


@cpu_only
@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_fwd_variance_in_place_needs_one_tile(L, variant):
    # exact aliasing of the variances is refused when several value-tile
    # workgroups read them (dv > 64 for bf16, dv > 32 for fp32)
    assert _fwd_call(L, variant, dv=128, var0=P + 16384) == -1
    assert "only when dv <= 64" in L.kdn_last_error_message().decode()
    assert _fwd_call(L, variant, io=0, dv=64, var0=P + 16384) == -1
    assert "only when dv <= 32" in L.kdn_last_error_message().decode()


@cpu_only
@pytest.mark.parametrize("variant,offset", [("diag", 16), ("iso", 4)])
def test_fwd_variance_partial_overlap(L, variant, offset):
    # exact aliasing of the initial and final variances is allowed, a partial
    # overlap is not
    assert _fwd_call(L, variant, var0=P + 16384 + offset) == -1
    assert "overlap" in L.kdn_last_error_message().decode()


@cpu_only
@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_fwd_sequence_parallel_workspace_overlap(L, variant):
    # a shape the library splits over the sequence, given its workspace
    shape = dict(B=1, T=8192, H=2, dk=128, dv=128)
    need = L.kdn_fwd_workspace_size(0 if variant == "diag" else 1, 1, 8192, 2, 128, 128, 1)
    assert need > 0
    far = 1 << 40
    kw = dict(shape, q=far, k=far, v=far, alpha=far, omega=far, r=far, o=far + (1 << 32),
              S_T=far + (2 << 32), var_T=far + (3 << 32), ws_bytes=need)
    assert _fwd_call(L, variant, ws=far + 64, **kw) == -1
    assert "workspace must not overlap q" in L.kdn_last_error_message().decode()
    assert _fwd_call(L, variant, ws=far + (2 << 32) - 64, **kw) == -1
    assert "workspace must not overlap S_T" in L.kdn_last_error_message().decode()
    assert _fwd_call(L, variant, ws=far + 4, **kw) == -1
    assert "aligned" in L.kdn_last_error_message().decode()


@cpu_only
def test_step_validation(L):
    def step(**kw):
        a = dict(var=0, B=4, H=2, dk=128, dv=128, io=1, mu=128.0, q=P, k=P, v=P, alpha=P,
                 omega=P, r=P, S=P + 4096, vs=P + 8192, o=P + 16384)
        a.update(kw)
        return L.kdn_step(a["var"], a["B"], a["H"], a["dk"], a["dv"], a["io"], a["mu"], a["q"],
                          a["k"], a["v"], a["alpha"], a["omega"], a["r"], a["S"], a["vs"], a["o"],
                          None)
    assert step(var=3) == -1
    assert step(dk=32) == -2
    assert step(dv=256) == -2
    assert step(S=None) == -1
    assert step(vs=None) == -1
    assert step(S=MIS) == -1
    assert step(o=P) == -1
    assert step(io=5) == -1


@cpu_only
def test_gain_scan_validation(L):
    def gs(**kw):
        a = dict(var=0, B=1, T=64, H=2, dk=64, io=1, mu=64.0, k=P, alpha=P, omega=P, r=P,
                 var0=None, kappa=None, var_T=P + 4096, ws=P + 8192, wsb=1 << 20)
        a.update(kw)
        return L.kdn_gain_scan(a["var"], a["B"], a["T"], a["H"], a["dk"], a["io"], a["mu"], a["k"],
                               a["alpha"], a["omega"], a["r"], a["var0"], a["kappa"], a["var_T"],
                               a["ws"], a["wsb"], None)
    assert gs(var=2) == -1
    assert gs(dk=32) == -2
    assert gs(wsb=16) == -3
    assert gs(ws=None) == -3
    assert gs(var_T=None) == -1
    assert gs(alpha=MIS) == -1
    assert gs(var0=P + 4096) == -1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from kalman_delta_rule_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(_lib.KdnLibraryMissing):
        _lib.lib()


def _fwd_ex_call(L, **kw):
    a = dict(variant=0, B=1, T=64, H=2, dk=64, dv=64, io=1, mu=64.0, mu_h=None, q=P, k=P, v=P,
             alpha=P, omega=P, r=P, S0=None, var0=None, c0_h=None, o=P + 4096, S_T=P + 8192,
             var_T=P + 16384, beta=None, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return L.kdn_fwd_ex(a["variant"], a["B"], a["T"], a["H"], a["dk"], a["dv"], a["io"], a["mu"],
                        a["mu_h"], a["q"], a["k"], a["v"], a["alpha"], a["omega"], a["r"],
                        a["S0"], a["var0"], a["c0_h"], a["o"], a["S_T"], a["var_T"], a["beta"],
                        a["ws"], a["ws_bytes"], a["stream"])


@cpu_only
@pytest.mark.parametrize("bad,code,needle", [
    (dict(variant=2), -1, "variant"),
    (dict(var0=P + 32768, c0_h=P + 65536), -1, "either as var0 or as c0_h"),
    (dict(mu_h=P + 2), -1, "mu_h must be 4-byte aligned"),
    (dict(c0_h=P + 1), -1, "c0_h must be 4-byte aligned"),
    (dict(beta=P + 3), -1, "beta_eff must be 4-byte aligned"),
    (dict(beta=P), -1, "beta_eff must not alias"),
    (dict(beta=P + 4096), -1, "beta_eff must not alias"),
    (dict(dk=96), -2, "dk"),
])
def test_fwd_ex_validation(L, bad, code, needle):
    assert _fwd_ex_call(L, **bad) == code
    assert needle in L.kdn_last_error_message().decode()


@cpu_only
def test_step_ex_validation(L):
    def step(**kw):
        a = dict(var=0, B=4, H=2, dk=128, dv=128, io=1, mu=128.0, mu_h=None, q=P, k=P, v=P,
                 alpha=P, omega=P, r=P, S=P + 4096, vs=P + 8192, o=P + 16384, beta=None)
        a.update(kw)
        return L.kdn_step_ex(a["var"], a["B"], a["H"], a["dk"], a["dv"], a["io"], a["mu"],
                             a["mu_h"], a["q"], a["k"], a["v"], a["alpha"], a["omega"], a["r"],
                             a["S"], a["vs"], a["o"], a["beta"], None)
    assert step(var=5) == -1 and "variant" in L.kdn_last_error_message().decode()
    assert step(beta=P + 8192) == -1 and "beta_eff" in L.kdn_last_error_message().decode()
    assert step(mu_h=P + 1) == -1 and "mu_h" in L.kdn_last_error_message().decode()
    assert step(dv=96) == -2


@cpu_only
def test_dense_fwd_validation(L):
    def dense(**kw):
        a = dict(B=1, T=32, H=2, dk=32, dv=64, io=0, q=P, k=P, v=P, alpha=P, omega=P, r=P,
                 S0=None, P0=None, o=P + 4096, S_T=P + 8192, P_T=P + 65536, beta=None)
        a.update(kw)
        return L.kdn_dense_fwd(a["B"], a["T"], a["H"], a["dk"], a["dv"], a["io"], a["q"], a["k"],
                               a["v"], a["alpha"], a["omega"], a["r"], a["S0"], a["P0"], a["o"],
                               a["S_T"], a["P_T"], a["beta"], None)
    msg = lambda: L.kdn_last_error_message().decode()
    assert dense(dk=128) == -2 and "dk" in msg()
    assert dense(dv=96) == -2 and "dv" in msg()
    assert dense(io=3) == -1 and "io_dtype" in msg()
    assert dense(T=-1) == -1
    assert dense(q=None) == -1 and "q must not be NULL" in msg()
    assert dense(P_T=None) == -1 and "P_T" in msg()
    assert dense(P0=P + 65536 + 64) == -1 and "P_T must either equal P0" in msg()
    assert dense(S0=P + 8192 + 4) == -1 and "S_T must either equal S0" in msg()
    assert dense(o=P) == -1 and "alias" in msg()
    assert dense(beta=P + 4096) == -1 and "beta_eff" in msg()
    assert dense(S_T=P + 2) == -1 and "aligned" in msg()


def test_bwd_validation(L):
    G = 1 << 28  # every buffer in its own region, far apart
    names = ["q", "k", "v", "alpha", "omega", "r", "S0", "var0", "c0", "d_o", "dS_T", "dvar_T",
             "dq", "gk", "gv", "dalpha", "domega", "dr", "dS0", "dvar0", "dmu", "ws"]
    base = {n: P + (i + 1) * G for i, n in enumerate(names)}

    def bwd(**kw):
        a = dict(variant=0, B=1, T=40, H=2, dk=128, dv=64, io=1, mu=128.0, mu_h=None)
        a.update({n: base[n] for n in names})
        a.update(S0=None, var0=None, c0=None, dS_T=None, dvar_T=None)
        a.update(kw)
        ws_bytes = a.pop("ws_bytes", L.kdn_bwd_workspace_size(a["variant"], a["B"], a["T"],
                                                              a["H"], a["dk"], a["dv"]))
        return L.kdn_bwd(a["variant"], a["B"], a["T"], a["H"], a["dk"], a["dv"], a["io"], a["mu"],
                         a["mu_h"], a["q"], a["k"], a["v"], a["alpha"], a["omega"], a["r"],
                         a["S0"], a["var0"], a["c0"], a["d_o"], a["dS_T"], a["dvar_T"], a["dq"],
                         a["gk"], a["gv"], a["dalpha"], a["domega"], a["dr"], a["dS0"],
                         a["dvar0"], a["dmu"], a["ws"], ws_bytes, None)
    msg = lambda: L.kdn_last_error_message().decode()
    assert bwd(variant=2) == -1 and "variant" in msg()
    assert bwd(io=2) == -1 and "io_dtype" in msg()
    assert bwd(dk=32) == -2 and "dk" in msg()
    assert bwd(dv=40) == -2 and "dv" in msg()
    assert bwd(dv=272) == -2
    assert bwd(mu=-1.0) == -1 and "mu" in msg()
    assert bwd(q=None) == -1 and "q must not be NULL" in msg()
    assert bwd(d_o=None) == -1 and "d_o" in msg()
    assert bwd(dalpha=None) == -1 and "dalpha" in msg()
    assert bwd(var0=base["var0"], c0=base["c0"]) == -1 and "either" in msg()
    assert bwd(dq=base["dq"] + 1) == -1 and "aligned" in msg()
    assert bwd(alpha=base["alpha"] + 4) == -1 and "16-byte" in msg()
    assert bwd(d_o=base["d_o"] + 8) == -1 and "16-byte" in msg()
    assert bwd(dr=base["dr"] + 2) == -1 and "aligned" in msg()
    assert bwd(dq=base["q"]) == -1 and "dq must not overlap q" in msg()
    assert bwd(dS0=base["ws"] + 64) == -1 and "overlap" in msg()
    assert bwd(dv=64, dmu=base["dalpha"] + 4) == -1 and "overlap" in msg()
    assert bwd(ws_bytes=16) == -3 and "workspace" in msg()
    assert bwd(ws=base["ws"] + 4) == -1 and "16-byte" in msg()
    # workspace: gain pieces, the gain scan's summaries and carries, the state
    # every 16th token, 4 partial row sums per value-column block (64 columns
    # for the chunked memory backward, dv a multiple of 64; 16 columns and
    # every token's innovations for the token-serial one)
    B, T, H, dk = 2, 40, 3, 128
    ntok, nch = B * T * H, 3
    r64 = lambda n: (n + 63) // 64 * 64
    for dv in (64, 128, 32, 48):
        chunked = dv % 64 == 0
        nblk = dv // (64 if chunked else 16)
        common = (r64(B * H * nch * dk * dv) + (0 if chunked else r64(ntok * dv))
                  + r64(4 * nblk * ntok * dk))
        scan = lambda width: r64(B * H * 1 * width * 5)  # the gain scan: one 64-token chunk
        # the gain backward's scan over 32-token chunks (two here): (A, B) and
        # carry per chunk and width, a scalar per token, an information-scale
        # part per chunk
        grad = lambda width: (r64(B * H * 2 * width * 2) + r64(B * H * 2 * width) + r64(ntok)
                              + r64(B * H * 2))
        # Diagonal chunked: the checkpoint walk's final state and variance
        walk = r64(B * H * dk * dv) + r64(B * H * dk) if chunked else 0
        diag = 2 * r64(ntok * dk) + r64(ntok) + scan(dk) + grad(dk) + common + walk
        iso = r64(ntok * 4) + scan(1) + grad(1) + common
        assert L.kdn_bwd_workspace_size(0, B, T, H, dk, dv) == 4 * diag, dv
        assert L.kdn_bwd_workspace_size(1, B, T, H, dk, dv) == 4 * iso, dv
    assert L.kdn_bwd_workspace_size(0, B, 0, H, dk, 64) == 0
    # the backward split over the sequence (Diagonal, d_k = d_v, few heads,
    # long T) adds two variance planes and six state planes of the segments
    # (config 3's shape: 8 segments; T = 2048 with 16 or 64 heads: 2)
    def base(iso, B, T, H, dk, dv):
        ntok, nch, ngc, ngr = B * T * H, (T + 15) // 16, (T + 63) // 64, (T + 31) // 32
        width = 1 if iso else dk
        pieces = r64(ntok * 4) if iso else 2 * r64(ntok * dk) + r64(ntok)
        walk = 0 if iso else r64(B * H * dk * dv) + r64(B * H * dk)
        return (pieces + r64(B * H * ngc * width * 5) + r64(B * H * ngr * width * 2)
                + r64(B * H * ngr * width) + r64(ntok) + r64(B * H * ngr)
                + r64(B * H * nch * dk * dv) + r64(4 * (dv // 64) * ntok * dk) + walk)
    for (B, T, H, d, S) in ((1, 65536, 16, 128, 8), (1, 2048, 16, 128, 2), (4, 2048, 16, 128, 2),
                            (1, 8192, 1, 64, 8), (1, 4096, 2, 64, 4)):
        seg = 2 * r64(B * S * H * d) + 6 * r64(B * S * H * d * d)
        assert L.kdn_bwd_workspace_size(0, B, T, H, d, d) == 4 * (base(False, B, T, H, d, d) + seg)
        assert L.kdn_bwd_workspace_size(1, B, T, H, d, d) == 4 * base(True, B, T, H, d, d)
    # not split: the grid already fills the chip, segments would be shorter
    # than 1024 tokens, or T does not divide
    for (B, T, H, d) in ((8, 4096, 16, 128), (1, 1024, 2, 128), (1, 4160, 2, 128)):
        assert L.kdn_bwd_workspace_size(0, B, T, H, d, d) == 4 * base(False, B, T, H, d, d)


def test_fwd_preact_validation(L):
    G = 1 << 28
    names = ["q", "k", "v", "a", "w", "r", "o", "S_T", "var_T", "ws"]
    base = {n: P + (i + 1) * G for i, n in enumerate(names)}

    def pre(**kw):
        a = dict(variant=0, B=1, T=40, H=2, dk=128, dv=128, io=1, mu=128.0, r_min=0.01)
        a.update({n: base[n] for n in names})
        a.update(kw)
        ws_bytes = a.pop("ws_bytes", L.kdn_fwd_preact_workspace_size(a["variant"], a["B"], a["T"],
                                                                     a["H"], a["dk"]))
        return L.kdn_fwd_preact(a["variant"], a["B"], a["T"], a["H"], a["dk"], a["dv"], a["io"],
                                a["mu"], None, a["q"], a["k"], a["v"], a["a"], a["w"], a["r"],
                                a["r_min"], None, None, None, a["o"], a["S_T"], a["var_T"], None,
                                a["ws"], ws_bytes, None)
    msg = lambda: L.kdn_last_error_message().decode()
    assert pre(variant=3) == -1 and "variant" in msg()
    assert pre(r_min=0.0) == -1 and "r_min" in msg()
    assert pre(r_min=float("nan")) == -1 and "r_min" in msg()
    assert pre(a=None) == -1 and "a_pre must not be NULL" in msg()
    assert pre(r=base["r"] + 2) == -1 and "r_pre must be 16-byte aligned" in msg()
    assert pre(ws_bytes=64) == -3 and "workspace" in msg()
    assert pre(ws=base["o"] + 256) == -1 and "workspace must not overlap o" in msg()
    assert pre(ws=base["ws"] + 4) == -1 and "workspace" in msg()
    # the forward's own checks still apply after the prologue's
    assert pre(dk=96) == -2 and "dk" in msg()
    ntok = 1 * 40 * 2
    r64 = lambda n: (n + 63) // 64 * 64
    assert L.kdn_fwd_preact_workspace_size(0, 1, 40, 2, 128) == 4 * (2 * r64(ntok * 128) + r64(ntok))
    assert L.kdn_fwd_preact_workspace_size(1, 1, 40, 2, 128) == 4 * (r64(ntok * 128) + 2 * r64(ntok))


@cpu_only
def test_gates_from_preact_validation(L):
    G = 1 << 28
    names = ["a", "w", "r", "alpha", "omega", "rr"]
    base = {n: P + (i + 1) * G for i, n in enumerate(names)}

    def gp(**kw):
        a = dict(variant=0, B=1, T=40, H=2, dk=128, io=1, r_min=0.01)
        a.update({n: base[n] for n in names})
        a.update(kw)
        return L.kdn_gates_from_preact(a["variant"], a["B"], a["T"], a["H"], a["dk"], a["io"],
                                       a["a"], a["w"], a["r"], a["r_min"], a["alpha"],
                                       a["omega"], a["rr"], None)
    msg = lambda: L.kdn_last_error_message().decode()
    assert gp(variant=2) == -1 and "variant" in msg()
    assert gp(io=1 | 0x100) == -1 and "io_dtype" in msg()
    assert gp(r_min=0.0) == -1 and "r_min" in msg()
    assert gp(dk=0) == -1
    assert gp(a=None) == -1 and "a_pre must not be NULL" in msg()
    assert gp(omega=None) == -1 and "omega must not be NULL" in msg()
    assert gp(alpha=base["alpha"] + 8) == -1 and "alpha must be 16-byte aligned" in msg()
    # alpha [1,40,2,128] fp32 is 40 KiB: an omega 16 KiB after it overlaps
    assert gp(omega=base["alpha"] + 16384) == -1 and "overlap" in msg()
    assert gp(rr=base["a"] + 64) == -1 and "r must not overlap a_pre" in msg()
    # nothing to do, nothing read
    assert gp(T=0, a=None, w=None, r=None, alpha=None, omega=None, rr=None) == 0


def test_bwd_preact_validation(L):
    G = 1 << 28
    names = ["q", "k", "v", "a", "w", "r", "d_o", "dq", "gk", "gv", "da", "dw", "dr", "ws"]
    base = {n: P + (i + 1) * G for i, n in enumerate(names)}

    def bp(**kw):
        a = dict(variant=0, B=1, T=40, H=2, dk=128, dv=64, io=1, mu=128.0, r_min=0.01)
        a.update({n: base[n] for n in names})
        a.update(kw)
        ws_bytes = a.pop("ws_bytes", L.kdn_bwd_preact_workspace_size(a["variant"], a["B"], a["T"],
                                                                     a["H"], a["dk"], a["dv"]))
        return L.kdn_bwd_preact(a["variant"], a["B"], a["T"], a["H"], a["dk"], a["dv"], a["io"],
                                a["mu"], None, a["q"], a["k"], a["v"], a["a"], a["w"], a["r"],
                                a["r_min"], None, None, None, a["d_o"], None, None, a["dq"],
                                a["gk"], a["gv"], a["da"], a["dw"], a["dr"], None, None, None,
                                a["ws"], ws_bytes, None)
    msg = lambda: L.kdn_last_error_message().decode()
    assert bp(r_min=-1.0) == -1 and "r_min" in msg()
    assert bp(w=None) == -1 and "w_pre must not be NULL" in msg()
    assert bp(ws_bytes=32) == -3 and "workspace" in msg()
    assert bp(da=base["a"] + 64) == -1 and "da_pre must not overlap a_pre" in msg()
    assert bp(dq=base["w"]) == -1 and "overlap" in msg()
    # the backward's own checks apply to the rest
    assert bp(dv=40) == -2 and "dv" in msg()
    assert (L.kdn_bwd_preact_workspace_size(0, 1, 40, 2, 128, 64)
            == L.kdn_fwd_preact_workspace_size(0, 1, 40, 2, 128)
            + L.kdn_bwd_workspace_size(0, 1, 40, 2, 128, 64))


@cpu_only
def test_gain_scan_static_validation(L):
    # the allocation-free gain scan checks like kdn_gain_scan, then rejects a
    # shape whose scratch exceeds its static array, before any launch
    assert L.kdn_gain_scan_static_max_bytes() == 32 << 20
    ok = dict(variant=0, B=1, T=65536, H=16, dk=128, io=1, mu=128.0)

    def call(**kw):
        a = dict(ok, **kw)
        return L.kdn_gain_scan_static(a["variant"], a["B"], a["T"], a["H"], a["dk"], a["io"],
                                      a["mu"], P, P, P, P, None, None, P + 4096, None)
    assert call() == -3
    assert "static scratch" in L.kdn_last_error_message().decode()
    assert call(variant=2) == -1
    assert call(dk=96) == -2
    assert call(io=2) == -1
    assert call(mu=-1.0) == -1
