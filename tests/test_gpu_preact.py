"""GPU parity of the forward from gate pre-activations (kdn_fwd_preact; KDN
reading notes, method part §8: alpha = sigmoid(a), omega = softplus(w),
r = r_min + softplus(rho), r_min = 0.01) against the oracle's gate prologue
followed by the oracle forward, on identical seeded pre-activations.  Bar as
for the forward: relative L2 <= 1e-4 (fp32 io) or <= 2e-2 (bf16 io) on o,
S_T, the variances and beta_eff."""
import numpy as np
import pytest
import torch

from kalman_delta_rule_amd import api, inputs
from kdn_testutil import TOL, host, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a HIP GPU")
    torch.cuda.init()


def _dev(x, io):
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    return {n: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda() for n, a in x.items()}


CASES = [
    # (variant, io, B, T, H, dk, dv)
    ("diag", "bf16", 2, 150, 3, 128, 128),
    ("iso", "bf16", 1, 97, 2, 128, 128),
    ("diag", "bf16", 1, 70, 2, 64, 64),
    ("diag", "f32", 2, 75, 3, 64, 64),
    ("iso", "f32", 1, 61, 2, 64, 32),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-%s-B%dT%dH%ddk%ddv%d" % c)
def test_preact_forward_matches_oracle(ora, case):
    variant, io, B, T, H, dk, dv = case
    w = inputs.Workload("t", variant, io, B, H, T, dk, dv, seed=700 + T)
    x = inputs.make_preact_inputs(w)
    mu_h = np.array([1.0, 40.0, 128.0][:H], dtype=np.float32) if variant == "diag" else None
    d = _dev(x, io)
    o, S, var, beta = api.kdn_fwd_preact(
        variant, d["q"], d["k"], d["v"], d["a_pre"], d["w_pre"], d["r_pre"], r_min=0.01,
        mu_h=None if mu_h is None else torch.from_numpy(mu_h).cuda(), want_beta_eff=True)
    torch.cuda.synchronize()
    g = ora.gate_prologue(x["a_pre"], x["w_pre"], x["r_pre"], r_min=0.01)
    fn = ora.diag_fwd if variant == "diag" else ora.iso_fwd
    ref = fn(x["q"], x["k"], x["v"], g["alpha"], g["omega"], g["r"],
             mu_h=None if mu_h is None else mu_h.astype(np.float64), return_beta_eff=True)
    rv = ref["p"] if variant == "diag" else ref["b"]
    err = {"o": rel_l2(host(o), ref["o"]), "S": rel_l2(host(S), ref["S"]),
           "var": rel_l2(host(var), rv), "beta_eff": rel_l2(host(beta), ref["beta_eff"])}
    print("preact %s errors %s" % (case, err), flush=True)
    assert max(err.values()) <= TOL[io], err


def test_preact_equals_forward_on_the_same_gates():
    # the gates computed by torch and fed to the plain forward give the
    # result of the call that computes them from the pre-activations
    w = inputs.Workload("t", "diag", "bf16", 1, 2, 64, 128, 128, seed=731)
    x = inputs.make_preact_inputs(w)
    d = _dev(x, "bf16")
    o1, S1, p1, _ = api.kdn_fwd_preact("diag", d["q"], d["k"], d["v"], d["a_pre"], d["w_pre"],
                                       d["r_pre"], r_min=0.05)
    a = torch.sigmoid(d["a_pre"].float())
    om = torch.nn.functional.softplus(d["w_pre"].float())
    r = 0.05 + torch.nn.functional.softplus(d["r_pre"].float())
    o2, S2, p2 = api.kdn_diag_fwd(d["q"], d["k"], d["v"], a.contiguous(), om.contiguous(),
                                  r.contiguous())
    torch.cuda.synchronize()
    # the prologue's exp / log are the hardware ones (~1 ulp from torch's),
    # so the fp32 state and variances agree to ~1e-6 while the bf16 output
    # can round the other way here and there
    assert rel_l2(host(S1), host(S2)) < 1e-5 and rel_l2(host(p1), host(p2)) < 1e-5
    assert rel_l2(host(o1), host(o2)) < 2e-3


FUSED_CASES = [
    # (variant, math, B, T, H, dk, dv): the bf16 forward forms alpha (and
    # Diagonal omega) from the pre-activations on chip
    ("diag", None, 2, 150, 3, 128, 128),
    ("diag", "bf16", 2, 150, 3, 128, 128),
    ("iso", None, 1, 97, 2, 128, 256),
    ("diag", None, 1, 70, 2, 64, 64),
    ("diag", "bf16", 1, 33, 2, 64, 128),
    ("iso", None, 2, 50, 1, 64, 64),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "%s-%s-B%dT%dH%ddk%ddv%d" % c)
def test_fused_preact_equals_forward_on_its_gates(case):
    """kdn_fwd_preact (pre-activations read by the walk) against kdn_fwd_ex on
    the gates kdn_gates_from_preact returns: equal bit for bit, with per-head
    mu, an initial state and variance, and beta_eff."""
    variant, math, B, T, H, dk, dv = case
    w = inputs.Workload("t", variant, "bf16", B, H, T, dk, dv, seed=770 + T + dk)
    x = inputs.make_preact_inputs(w)
    d = _dev(x, "bf16")
    rng = np.random.default_rng(771)
    mu_h = torch.from_numpy(rng.uniform(1.0, 150.0, H).astype(np.float32)).cuda()
    S0 = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32)).cuda()
    vs = (B, H) if variant == "iso" else (B, H, dk)
    var0 = torch.from_numpy(rng.uniform(0.1, 2.0, vs).astype(np.float32)).cuda()
    fused = api.kdn_fwd_preact(variant, d["q"], d["k"], d["v"], d["a_pre"], d["w_pre"],
                               d["r_pre"], r_min=0.03, S0=S0, var0=var0, mu_h=mu_h,
                               want_beta_eff=True, math=math)
    al, om, r = api.kdn_gates_from_preact(variant, d["a_pre"], d["w_pre"], d["r_pre"], r_min=0.03)
    ref = api.kdn_fwd_ex(variant, d["q"], d["k"], d["v"], al, om, r, S0=S0, var0=var0, mu_h=mu_h,
                         want_beta_eff=True, math=math)
    torch.cuda.synchronize()
    for name, a_, b_ in zip(("o", "S_T", "var_T", "beta_eff"), fused, ref):
        assert torch.equal(a_, b_), (name, rel_l2(host(a_).ravel(), host(b_).ravel()))


def test_gates_from_preact_match_oracle(ora):
    """The gates on their own against the oracle's fp64 prologue: ~1 ulp
    hardware exp2 / log2 / rcp, so a few fp32 ulps relative."""
    for variant, io in (("diag", "bf16"), ("iso", "bf16"), ("diag", "f32")):
        w = inputs.Workload("t", variant, io, 2, 3, 45, 64, 64, seed=780)
        x = inputs.make_preact_inputs(w)
        x["a_pre"] = x["a_pre"] * 8.0   # saturating sigmoids and large softplus arguments too
        x["w_pre"] = x["w_pre"] * 8.0
        if io == "bf16":
            x = {n: inputs.round_bf16(a) for n, a in x.items()}
        d = _dev(x, io)
        g = api.kdn_gates_from_preact(variant, d["a_pre"], d["w_pre"], d["r_pre"], r_min=0.02)
        torch.cuda.synchronize()
        ref = ora.gate_prologue(x["a_pre"], x["w_pre"], x["r_pre"], r_min=0.02)
        for name, got in zip(("alpha", "omega", "r"), g):
            want = np.asarray(ref[name], dtype=np.float64)
            rel = np.abs(host(got).astype(np.float64) - want) / np.maximum(np.abs(want), 1e-30)
            print(variant, io, name, "max rel err %.2e" % rel.max(), flush=True)
            assert rel.max() < 4e-6, (variant, io, name, rel.max())


def test_preact_empty_sequence_gives_initial_state():
    B, H, dk, dv = 2, 2, 128, 64
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    S0 = torch.randn(B, H, dk, dv, device="cuda")
    o, S, var, _ = api.kdn_fwd_preact("diag", z(B, 0, H, dk), z(B, 0, H, dk), z(B, 0, H, dv),
                                      z(B, 0, H, dk), z(B, 0, H, dk), z(B, 0, H), S0=S0)
    torch.cuda.synchronize()
    assert torch.equal(S, S0) and torch.equal(var, torch.ones_like(var))


@pytest.mark.timeout(400)
def test_preact_config2_full_sampled(ora):
    # the launch configuration bench.py --preact times, sampled heads against
    # the oracle prologue + forward on each head's own slice
    from kdn_testutil import sample_heads
    w = inputs.workload(2)
    x = inputs.make_preact_inputs(w)
    d = _dev(x, w.io)
    o, S, var, _ = api.kdn_fwd_preact(w.variant, d["q"], d["k"], d["v"], d["a_pre"], d["w_pre"],
                                      d["r_pre"], r_min=0.01)
    # the whole tensors equal the forward on the gates the gate pass forms
    g = api.kdn_gates_from_preact(w.variant, d["a_pre"], d["w_pre"], d["r_pre"], r_min=0.01)
    o2, S2, var2, _ = api.kdn_fwd_ex(w.variant, d["q"], d["k"], d["v"], *g)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S, S2) and torch.equal(var, var2)
    del g, o2, S2, var2
    heads = sample_heads(w.B, w.H, 4, seed=202)
    sl = lambda a, b, h: np.ascontiguousarray(a[b:b + 1, :, h:h + 1])
    oh, Sh, vh = host(o), host(S), host(var)
    eo, es, ev = [], [], []
    for (b, h) in heads:
        g = ora.gate_prologue(sl(x["a_pre"], b, h), sl(x["w_pre"], b, h), sl(x["r_pre"], b, h),
                              r_min=0.01)
        ref = ora.diag_fwd(sl(x["q"], b, h), sl(x["k"], b, h), sl(x["v"], b, h), g["alpha"],
                           g["omega"], g["r"])
        eo.append((oh[b, :, h].ravel(), ref["o"].ravel()))
        es.append((Sh[b, h].ravel(), ref["S"].ravel()))
        ev.append((vh[b, h].ravel(), ref["p"].ravel()))
    err = {n: rel_l2(np.concatenate([a for a, _ in pr]), np.concatenate([r for _, r in pr]))
           for n, pr in (("o", eo), ("S", es), ("var", ev))}
    print("preact %s heads=%s errors %s" % (w.name, heads, err), flush=True)
    assert max(err.values()) <= TOL[w.io], err


@pytest.mark.parametrize("case", [("diag", "f32", 1, 37, 2, 64, 32), ("iso", "bf16", 1, 70, 2, 128, 64),
                                  ("diag", "bf16", 2, 50, 2, 128, 128)],
                         ids=lambda c: "%s-%s-B%dT%dH%ddk%ddv%d" % c)
def test_bwd_preact_matches_oracle(ora, case):
    variant, io, B, T, H, dk, dv = case
    w = inputs.Workload("t", variant, io, B, H, T, dk, dv, seed=760 + T)
    x = inputs.make_preact_inputs(w)
    do = np.random.default_rng(761).standard_normal((B, T, H, dv)).astype(np.float32)
    x["do"] = inputs.round_bf16(do) if io == "bf16" else do
    d = _dev(x, io)
    g = api.kdn_bwd_preact(variant, d["q"], d["k"], d["v"], d["a_pre"], d["w_pre"], d["r_pre"],
                           d["do"], r_min=0.02)
    torch.cuda.synchronize()
    ref = ora.bwd_preact(variant, x["q"], x["k"], x["v"], x["a_pre"], x["w_pre"], x["r_pre"],
                         x["do"], r_min=0.02)
    err = {n: rel_l2(host(g[n]), ref[n]) for n in ("dq", "dk", "dv", "da_pre", "dw_pre", "dr_pre",
                                                   "dS0", "dvar0", "dmu")}
    print("bwd_preact %s errors %s" % (case, {k_: "%.2e" % v_ for k_, v_ in err.items()}),
          flush=True)
    assert max(err.values()) <= TOL[io], err


@pytest.mark.parametrize("variant,io,dk", [("diag", "bf16", 128), ("iso", "bf16", 128),
                                           ("diag", "f32", 64)],
                         ids=lambda x: str(x))
def test_preact_very_negative_gates(ora, variant, io, dk):
    """a_pre in [-12, -5] in every fourth channel (alpha from 6e-6 to 7e-3:
    16-token chunk products down to about 1e-84, past fp32's span) and
    a_pre = -200 (alpha exactly 0 after the sigmoid saturates) at a tenth of
    its tokens.  The forward's strong-decay rule raises alphas below 2^-14 to
    2^-14 in chunks that fp32 cannot span, a relative perturbation of at most
    6.1e-5 of a state row per raised token: fp32-equivalent paths are held
    to 2e-4 here, the single-product bf16 paths to their usual bar."""
    B, T, H, dv = 1, 200, 2, dk
    w = inputs.Workload("t", variant, io, B, H, T, dk, dv, seed=741)
    x = inputs.make_preact_inputs(w)
    rng = np.random.default_rng(742)
    sel = (np.arange(dk) % 4 == 3)[None, None, None, :]
    neg = rng.uniform(-12.0, -5.0, x["a_pre"].shape)
    neg = np.where(rng.random(x["a_pre"].shape) < 0.1, -200.0, neg)
    x["a_pre"] = np.where(sel, neg, x["a_pre"]).astype(np.float32)
    if io == "bf16":   # the values the device sees
        x["a_pre"] = inputs.round_bf16(x["a_pre"])
    d = _dev(x, io)
    split = io == "bf16" and variant == "diag"
    o, S, var, _ = api.kdn_fwd_preact(variant, d["q"], d["k"], d["v"], d["a_pre"], d["w_pre"],
                                      d["r_pre"], r_min=0.01)
    torch.cuda.synchronize()
    g = ora.gate_prologue(x["a_pre"], x["w_pre"], x["r_pre"], r_min=0.01)
    fn = ora.diag_fwd if variant == "diag" else ora.iso_fwd
    ref = fn(x["q"], x["k"], x["v"], g["alpha"], g["omega"], g["r"])
    rv = ref["p"] if variant == "diag" else ref["b"]
    err = {"S": rel_l2(host(S), ref["S"]), "var": rel_l2(host(var), rv),
           "o": rel_l2(host(o), ref["o"])}
    print("very negative a_pre", variant, io, err, flush=True)
    assert all(np.isfinite(host(t)).all() for t in (o, S, var))
    tol = 2e-4 if (io == "f32" or split) else TOL[io]
    assert err["S"] <= tol and err["var"] <= tol, err
    # o in bf16 carries its own rounding
    assert err["o"] <= (TOL["bf16"] if io == "bf16" else tol), err
