"""GPU parity of the exact dense-covariance Kalman memory (kdn_dense_fwd,
KDN reading notes, method part §2, Eq. (12)-(17), with D_t = diag(alpha_t),
Omega_t = diag(omega_t)) against the oracle's dense filter -- itself pinned
to the printed collision table and to batch Bayesian regression -- run head
by head on identical inputs.  Bar: relative L2 <= 1e-4 (fp32 q/k/v) or
<= 2e-2 (bf16 q/k/v) on o, S_T, P_T and beta_eff.
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


def _spd(rng, B, H, dk):
    A = rng.standard_normal((B, H, dk, dk)) / np.sqrt(dk)
    return (A @ np.swapaxes(A, -1, -2) + 0.3 * np.eye(dk)).astype(np.float32)


def _oracle(ora, inp, S0, P0):
    B, T, H, dk = inp["k"].shape
    dv = inp["v"].shape[-1]
    o = np.zeros((B, T, H, dv))
    S = np.zeros((B, H, dk, dv))
    P = np.zeros((B, H, dk, dk))
    beta = np.zeros((B, T, H))
    for b in range(B):
        for h in range(H):
            sl = lambda n: np.asarray(inp[n][b, :, h], dtype=np.float64)
            D = np.stack([np.diag(a) for a in sl("alpha")])
            Om = np.stack([np.diag(w) for w in sl("omega")])
            out = ora.dense_kf(sl("k"), sl("v"), sl("q"), D, Om, sl("r"),
                               S0[b, h].astype(np.float64), P0[b, h].astype(np.float64))
            o[b, :, h] = out["o"]
            S[b, h] = out["S"]
            P[b, h] = out["P"]
            beta[b, :, h] = out["z"] / (sl("r") + out["z"])
    return o, S, P, beta


SHAPES = [
    # (io, B, T, H, dk, dv)
    ("f32", 2, 120, 2, 16, 32),
    ("f32", 1, 80, 2, 32, 128),
    ("f32", 1, 60, 1, 64, 64),
    ("f32", 1, 40, 3, 64, 16),
    ("bf16", 2, 100, 2, 64, 128),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%s-B%dT%dH%ddk%ddv%d" % s)
def test_dense_matches_oracle(ora, shape):
    io, B, T, H, dk, dv = shape
    w = inputs.Workload("t", "diag", io, B, H, T, dk, dv, seed=401 + T + dk)
    inp = inputs.make_fwd_inputs(w)
    rng = np.random.default_rng(402 + dk)
    S0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    P0 = _spd(rng, B, H, dk)
    d = to_dev(inp, io)
    o, S, P, beta = api.kdn_dense_fwd(d["q"], d["k"], d["v"], d["alpha"], d["omega"], d["r"],
                                      S0=torch.from_numpy(S0).cuda(),
                                      P0=torch.from_numpy(P0).cuda(), want_beta_eff=True)
    torch.cuda.synchronize()
    ro, rS, rP, rb = _oracle(ora, inp, S0, P0)
    err = {"o": rel_l2(host(o), ro), "S": rel_l2(host(S), rS), "P": rel_l2(host(P), rP),
           "beta_eff": rel_l2(host(beta), rb)}
    print("dense %s errors %s" % (shape, err), flush=True)
    assert max(err.values()) <= TOL[io], err


def test_dense_axis_aligned_keys_equal_diagonal_forward():
    # axis-aligned keys keep the exact posterior diagonal, so the dense filter
    # and the Diagonal forward at mu = 1 compute the same thing
    B, T, H, dk, dv = 1, 90, 2, 64, 64
    rng = np.random.default_rng(411)
    w = inputs.Workload("t", "diag", "f32", B, H, T, dk, dv, seed=412)
    inp = inputs.make_fwd_inputs(w)
    k = np.zeros((B, T, H, dk), np.float32)
    idx = rng.integers(0, dk, (B, T, H))
    np.put_along_axis(k, idx[..., None], (0.3 + 2 * rng.random((B, T, H, 1))).astype(np.float32),
                      axis=-1)
    inp["k"] = k
    p0 = (0.2 + rng.random((B, H, dk))).astype(np.float32)
    P0 = np.zeros((B, H, dk, dk), np.float32)
    for b in range(B):
        for h in range(H):
            P0[b, h] = np.diag(p0[b, h])
    d = to_dev(inp, "f32")
    od, Sd, Pd, _ = api.kdn_dense_fwd(d["q"], d["k"], d["v"], d["alpha"], d["omega"], d["r"],
                                      P0=torch.from_numpy(P0).cuda())
    of, Sf, pf = api.kdn_diag_fwd(d["q"], d["k"], d["v"], d["alpha"], d["omega"], d["r"],
                                  p0=torch.from_numpy(p0).cuda(), mu=1.0)
    torch.cuda.synchronize()
    assert rel_l2(host(od), host(of)) < 1e-4
    assert rel_l2(host(Sd), host(Sf)) < 1e-4
    assert rel_l2(np.diagonal(host(Pd), axis1=-2, axis2=-1), host(pf)) < 1e-4
    off = host(Pd) - np.stack([np.stack([np.diag(np.diag(x)) for x in y]) for y in host(Pd)])
    assert np.abs(off).max() < 1e-6


def test_dense_empty_sequence_passes_state_through():
    B, H, dk, dv = 2, 2, 32, 64
    z = lambda *s: torch.zeros(s, dtype=torch.float32, device="cuda")
    S0 = torch.randn(B, H, dk, dv, device="cuda")
    P0 = torch.eye(dk, device="cuda").expand(B, H, dk, dk).contiguous() * 0.7
    o, S, P, beta = api.kdn_dense_fwd(z(B, 0, H, dk), z(B, 0, H, dk), z(B, 0, H, dv),
                                      z(B, 0, H, dk), z(B, 0, H, dk), z(B, 0, H),
                                      S0=S0, P0=P0, want_beta_eff=True)
    torch.cuda.synchronize()
    assert torch.equal(S, S0) and torch.equal(P, P0) and o.shape == (B, 0, H, dv)
