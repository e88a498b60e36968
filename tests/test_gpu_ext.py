"""GPU parity of the extended calls: per-head information scale mu_h and
initial covariance c0_h (KDN reading notes, method part §8, trained per-head
parameters) and the effective write strength beta_eff = z / (r + z) (method
part §2), through kdn_fwd_ex / kdn_step_ex against the fp64 oracle on
identical seeded inputs.  Bar as for the forward: relative L2 <= 1e-4 (fp32
q/k/v) or <= 2e-2 (bf16 q/k/v) on o, S_T, the variances and beta_eff.
"""
import numpy as np
import pytest
import torch

from kalman_delta_rule_amd import api, inputs
from kdn_testutil import TOL, host, rel_l2, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a HIP GPU")
    torch.cuda.init()


def _oracle_fwd(ora, variant, inp, mu_h, c0_h):
    args = [inp[n] for n in ("q", "k", "v", "alpha", "omega", "r")]
    fn = ora.diag_fwd if variant == "diag" else ora.iso_fwd
    out = fn(*args, mu_h=mu_h, c0_h=c0_h, return_beta_eff=True)
    out["var"] = out["p"] if variant == "diag" else out["b"]
    return out


SHAPES = [
    # (io, B, T, H, dk, dv)
    ("bf16", 2, 150, 3, 128, 128),
    ("bf16", 1, 97, 3, 64, 64),
    ("f32", 2, 75, 3, 64, 64),
]


@pytest.mark.parametrize("variant", ["diag", "iso"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%s-B%dT%dH%ddk%ddv%d" % s)
def test_fwd_ex_per_head_and_beta_eff(ora, variant, shape):
    io, B, T, H, dk, dv = shape
    w = inputs.Workload("t", variant, io, B, H, T, dk, dv, seed=301 + T)
    inp = inputs.make_fwd_inputs(w)
    mu_h = np.array([1.0, 11.3, 2.0 * dk][:H], dtype=np.float32)
    c0_h = np.array([0.4, 2.5, 1.0][:H], dtype=np.float32)
    d = to_dev(inp, io)
    o, S, var, beta = api.kdn_fwd_ex(
        variant, d["q"], d["k"], d["v"], d["alpha"], d["omega"], d["r"],
        mu_h=torch.from_numpy(mu_h).cuda(), c0_h=torch.from_numpy(c0_h).cuda(),
        want_beta_eff=True)
    torch.cuda.synchronize()
    ref = _oracle_fwd(ora, variant, inp, mu_h.astype(np.float64), c0_h.astype(np.float64))
    err = {"o": rel_l2(host(o), ref["o"]), "S": rel_l2(host(S), ref["S"]),
           "var": rel_l2(host(var), ref["var"]), "beta_eff": rel_l2(host(beta), ref["beta_eff"])}
    print("fwd_ex %s %s errors %s" % (variant, shape, err), flush=True)
    assert max(err.values()) <= TOL[io], err
    bh = host(beta)
    assert (bh >= 0).all() and (bh < 1).all()


@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_fwd_ex_without_options_is_the_plain_forward(variant):
    w = inputs.Workload("t", variant, "bf16", 1, 2, 90, 128, 128, seed=311)
    d = to_dev(inputs.make_fwd_inputs(w), "bf16")
    fn = api.kdn_diag_fwd if variant == "diag" else api.kdn_iso_fwd
    a = fn(d["q"], d["k"], d["v"], d["alpha"], d["omega"], d["r"])
    b = api.kdn_fwd_ex(variant, d["q"], d["k"], d["v"], d["alpha"], d["omega"], d["r"])
    torch.cuda.synchronize()
    for x, y in zip(a, b[:3]):
        assert torch.equal(x, y)
    assert b[3] is None


@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_fwd_ex_empty_sequence_gives_c0(variant):
    B, H, dk, dv = 2, 3, 128, 128
    z = lambda *s: torch.zeros(s, dtype=torch.float32, device="cuda")
    q = torch.zeros((B, 0, H, dk), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((B, 0, H, dv), dtype=torch.bfloat16, device="cuda")
    om = z(B, 0, H, dk) if variant == "diag" else z(B, 0, H)
    c0 = torch.tensor([0.5, 1.5, 3.0], device="cuda")
    o, S, var, beta = api.kdn_fwd_ex(variant, q, q, v, z(B, 0, H, dk), om, z(B, 0, H),
                                     c0_h=c0, want_beta_eff=True)
    torch.cuda.synchronize()
    want = c0[None, :, None].expand(B, H, dk) if variant == "diag" else c0[None, :].expand(B, H)
    assert torch.equal(var, want) and torch.equal(S, torch.zeros_like(S))
    assert beta.shape == (B, 0, H)


@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_step_ex_per_head_mu_and_beta_eff(ora, variant):
    B, H, dk, dv = 4, 3, 128, 128
    rng = np.random.default_rng(321)
    w = inputs.Workload("t", variant, "bf16", B, H, 1, dk, dv, seed=322)
    inp = inputs.make_fwd_inputs(w)
    S0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    var0 = rng.uniform(0.2, 2.0, (B, H, dk) if variant == "diag" else (B, H)).astype(np.float32)
    mu_h = np.array([1.0, 30.0, 300.0], dtype=np.float32)
    d = to_dev(inp, "bf16")
    one = lambda t: t[:, 0].contiguous()
    S = torch.from_numpy(S0).cuda()
    var = torch.from_numpy(var0).cuda()
    beta = torch.empty((B, H), dtype=torch.float32, device="cuda")
    o = api.kdn_step(variant, one(d["q"]), one(d["k"]), one(d["v"]), one(d["alpha"]),
                     one(d["omega"]), one(d["r"]), S, var,
                     mu_h=torch.from_numpy(mu_h).cuda(), beta_eff=beta)
    torch.cuda.synchronize()
    t0 = lambda x: np.asarray(x)[:, 0]
    ref = ora.step(variant, t0(inp["q"]), t0(inp["k"]), t0(inp["v"]), t0(inp["alpha"]),
                   t0(inp["omega"]), t0(inp["r"]), S0.astype(np.float64),
                   var0.astype(np.float64), mu_h=mu_h.astype(np.float64))
    err = {"o": rel_l2(host(o), ref["o"]), "S": rel_l2(host(S), ref["S"]),
           "var": rel_l2(host(var), ref["var"]), "beta_eff": rel_l2(host(beta), ref["beta_eff"])}
    print("step_ex %s errors %s" % (variant, err), flush=True)
    assert max(err.values()) <= TOL["bf16"], err
