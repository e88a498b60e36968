"""GPU parity of the sequence-parallel bf16 forward: shapes with few heads and
long sequences, given the workspace kdn_fwd_workspace_size names, run as S
independent segments (three walks and a per-head combine of the segments'
affine maps).  Against the fp64 oracle (every element) and against the serial
walk, which the same call runs without the workspace.
"""
import numpy as np
import pytest
import torch

from kalman_delta_rule_amd import api, inputs
from kdn_testutil import TOL, compare_heads, host, oracle_heads, rel_l2, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a HIP GPU")
    torch.cuda.init()


def _split(variant, B, T, H, dk, dv):
    return api.kdn_fwd_workspace_size(variant, B, T, H, dk, dv, torch.bfloat16) > 0


def _run(variant, d, seqpar, mu=None, S0=None, var0=None, mu_h=None, c0_h=None, beta=False):
    o, S, var, b = api.kdn_fwd_ex(variant, d["q"], d["k"], d["v"], d["alpha"], d["omega"],
                                  d["r"], S0=S0, var0=var0, mu=mu, mu_h=mu_h, c0_h=c0_h,
                                  want_beta_eff=beta, sequence_parallel=seqpar)
    torch.cuda.synchronize()
    return o, S, var, b


def _alpha(regime, shape, rng):
    if regime == "one":       # no decay: the segments' affine parts N dwarf their linear parts M
        return np.ones(shape, np.float32)
    if regime == "slow":
        return (1.0 / (1.0 + np.exp(-rng.normal(6.0, 0.5, shape)))).astype(np.float32)
    return None               # the workload's own decays


def _compare(ora, variant, inp, mu=None, S0=None, var0=None, tag=""):
    B, T, H, dk = inp["k"].shape
    dv = inp["v"].shape[-1]
    assert _split(variant, B, T, H, dk, dv)
    d = to_dev(inp, "bf16")
    S0d = None if S0 is None else torch.from_numpy(S0).cuda()
    v0d = None if var0 is None else torch.from_numpy(var0).cuda()
    o, S, var, _ = _run(variant, d, True, mu=mu, S0=S0d, var0=v0d)
    heads = [(b, h) for b in range(B) for h in range(H)]
    res = oracle_heads(ora, variant, inp, heads, mu=mu, S0=S0, var0=var0)
    err = compare_heads(res, host(o), host(S), host(var), heads)
    # the serial walk on the same inputs
    o1, S1, var1, _ = _run(variant, d, False, mu=mu, S0=S0d, var0=v0d)
    d_ser = {"o": rel_l2(host(o).ravel(), host(o1).ravel()),
             "S": rel_l2(host(S).ravel(), host(S1).ravel()),
             "var": rel_l2(np.ravel(host(var)), np.ravel(host(var1)))}
    err1 = compare_heads(res, host(o1), host(S1), host(var1), heads)
    print("%s %s oracle %s serial-vs-oracle %s split-vs-serial %s" % (tag, variant, err, err1,
                                                                     d_ser), flush=True)
    tol = TOL["bf16"]
    assert err["o"] <= tol and err["S"] <= tol and err["var"] <= tol, err
    assert d_ser["o"] <= tol and d_ser["S"] <= tol and d_ser["var"] <= 1e-4, d_ser


@pytest.mark.timeout(300)
@pytest.mark.parametrize("variant", ["diag", "iso"])
@pytest.mark.parametrize("shape", [(1, 8192, 2, 128), (1, 4096, 1, 64), (2, 8192, 1, 64)],
                         ids=lambda s: "B%dT%dH%dd%d" % s)
def test_seqpar_matches_oracle(ora, variant, shape):
    B, T, H, d = shape
    w = inputs.Workload("t", variant, "bf16", B, H, T, d, d, seed=900 + T // 64 + d)
    _compare(ora, variant, inputs.make_fwd_inputs(w), tag=str(shape))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("variant", ["diag", "iso"])
@pytest.mark.parametrize("regime", ["one", "slow"])
def test_seqpar_decay_regimes(ora, variant, regime):
    B, T, H, d = 1, 8192, 1, 128
    w = inputs.Workload("t", variant, "bf16", B, H, T, d, d, seed=930)
    inp = inputs.make_fwd_inputs(w)
    inp["alpha"] = _alpha(regime, inp["alpha"].shape, np.random.default_rng(931))
    _compare(ora, variant, inp, tag=regime)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_seqpar_initial_state_and_mu(ora, variant):
    B, T, H, d = 1, 4096, 2, 64
    w = inputs.Workload("t", variant, "bf16", B, H, T, d, d, seed=940)
    inp = inputs.make_fwd_inputs(w)
    rng = np.random.default_rng(941)
    S0 = rng.standard_normal((B, H, d, d)).astype(np.float32)
    var0 = rng.uniform(0.1, 2.0, (B, H, d) if variant == "diag" else (B, H)).astype(np.float32)
    for mu in (0.0, 300.0):
        _compare(ora, variant, inp, mu=mu, S0=S0, var0=var0, tag="mu=%g" % mu)


@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_seqpar_per_head_options_match_serial(variant):
    B, T, H, d = 1, 8192, 2, 128
    w = inputs.Workload("t", variant, "bf16", B, H, T, d, d, seed=950)
    dd = to_dev(inputs.make_fwd_inputs(w), "bf16")
    mu_h = torch.tensor([3.0, 200.0], device="cuda")
    c0_h = torch.tensor([0.5, 4.0], device="cuda")
    a = _run(variant, dd, True, mu_h=mu_h, c0_h=c0_h, beta=True)
    b = _run(variant, dd, False, mu_h=mu_h, c0_h=c0_h, beta=True)
    errs = [rel_l2(host(x).ravel(), host(y).ravel()) for x, y in zip(a, b)]
    print(variant, "o S var beta", errs, flush=True)
    assert errs[0] <= 2e-2 and errs[1] <= 2e-2 and errs[2] <= 1e-4 and errs[3] <= 1e-4, errs


def test_seqpar_in_place_state():
    # S_T may equal S0 on the split path too (the variances in place only
    # with one workgroup per head, which d = 128 is not)
    B, T, H, d = 1, 8192, 2, 128
    w = inputs.Workload("t", "diag", "bf16", B, H, T, d, d, seed=960)
    dd = to_dev(inputs.make_fwd_inputs(w), "bf16")
    g = torch.Generator(device="cpu").manual_seed(961)
    S0 = torch.randn((B, H, d, d), generator=g).cuda()
    p0 = (torch.rand((B, H, d), generator=g) + 0.5).cuda()
    o, S, p, _ = _run("diag", dd, True, S0=S0.clone(), var0=p0.clone())
    S_in, p_in = S0.clone(), p0.clone()
    o2, S2, p2, _ = api.kdn_fwd_ex("diag", dd["q"], dd["k"], dd["v"], dd["alpha"], dd["omega"],
                                   dd["r"], S0=S_in, var0=p_in, S_T=S_in)
    torch.cuda.synchronize()
    assert S2.data_ptr() == S_in.data_ptr()
    assert torch.equal(o, o2) and torch.equal(S, S2) and torch.equal(p, p2)


def test_short_workspace_runs_the_serial_walk():
    # a workspace one byte short of kdn_fwd_workspace_size is ignored: the call
    # equals the serial walk (same kernels, bit for bit); the full size splits
    from kalman_delta_rule_amd import _lib
    L = _lib.lib()
    B, T, H, d = 1, 8192, 2, 128
    w = inputs.Workload("t", "diag", "bf16", B, H, T, d, d, seed=970)
    inp = inputs.make_fwd_inputs(w)
    # slow decay keeps each segment's linear part M away from zero (with the
    # workload's decays it underflows within a segment, and the split then
    # reproduces the serial state bit for bit)
    inp["alpha"] = _alpha("slow", inp["alpha"].shape, np.random.default_rng(971))
    dd = to_dev(inp, "bf16")
    need = api.kdn_fwd_workspace_size("diag", B, T, H, d, d, torch.bfloat16)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ser = _run("diag", dd, False)

    def call(nbytes):
        o = torch.empty((B, T, H, d), dtype=torch.bfloat16, device="cuda")
        S = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda")
        p = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
        st = L.kdn_diag_fwd(B, T, H, d, d, 1, float(d), dd["q"].data_ptr(), dd["k"].data_ptr(),
                            dd["v"].data_ptr(), dd["alpha"].data_ptr(), dd["omega"].data_ptr(),
                            dd["r"].data_ptr(), None, None, o.data_ptr(), S.data_ptr(),
                            p.data_ptr(), ws.data_ptr(), nbytes,
                            torch.cuda.current_stream().cuda_stream)
        _lib.check(st)
        torch.cuda.synchronize()
        return o, S, p

    short = call(need - 1)
    assert all(torch.equal(x, y) for x, y in zip(short, ser[:3]))
    full = call(need)
    spl = _run("diag", dd, True)
    assert all(torch.equal(x, y) for x, y in zip(full, spl[:3]))
    assert not torch.equal(full[1], ser[1])   # the split path really ran


@pytest.mark.timeout(600)
def test_seqpar_config3_shape_iso_slow_decay(ora):
    """Isotropic at the long-sequence shape (B1 H16 T65536 d128) with slow
    decays, so that the segments' linear parts M carry the combine: whole
    tensors against the oracle."""
    w = inputs.workload(3)
    inp = inputs.make_fwd_inputs(w, "iso")
    inp["alpha"] = _alpha("slow", inp["alpha"].shape, np.random.default_rng(3201))
    B, T, H, dk = inp["k"].shape
    assert _split("iso", B, T, H, dk, inp["v"].shape[-1])
    ref = ora.iso_fwd(*(inp[n] for n in ("q", "k", "v", "alpha", "omega", "r")))
    d = to_dev(inp, "bf16")
    o, S, b, _ = _run("iso", d, True)
    from kdn_testutil import compare_whole
    err, worst = compare_whole(ref, host(o), host(S), host(b))
    print(w.name, "iso slow decay, split over the sequence: rel-L2", err, "worst (b,h)", worst,
          flush=True)
    assert max(err.values()) <= TOL["bf16"] and max(worst.values()) <= TOL["bf16"], (err, worst)
