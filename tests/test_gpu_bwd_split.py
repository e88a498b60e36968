"""GPU parity of the backward split over the sequence (Diagonal, bf16 io,
shapes whose serial grid leaves most compute units idle) against the oracle's
backward, and against the same call without the split.

Over a span of tokens the state recurrence is affine, S_out = M S_in + N
(KDN reading notes, method part §2 and §6), so its reverse carries the state
adjoint as dS_in = M^T dS_out + (the span's own outputs): the call runs each
segment of the sequence as a batch row, from its entry state (forward walks
and a combine) and the adjoint entering it from the right (an adjoint-only
reverse pass and a combine from the last segment).  Every gradient is
compared whole against the oracle at the bf16 bar, and against the serial
call (a workspace one byte short of kdn_bwd_workspace_size) at 1e-3.  The
slow-decay cases keep M far from zero over a segment, so the combine
carries the result; there the two calls must differ bitwise.
"""
import numpy as np
import pytest
import torch

from kalman_delta_rule_amd import api, _lib
from kdn_testutil import TOL, rel_l2
import test_gpu_bwd as tb

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dalpha", "domega", "dr", "dS0", "dvar0", "dmu")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a HIP GPU")
    torch.cuda.init()


def _call(x, ws_bytes=None, mu=None, mu_h=None, c0_h=None):
    d = tb._dev(x, "bf16")
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    need = int(_lib.lib().kdn_bwd_workspace_size(0, B, T, H, dk, dv))
    ws = torch.empty(need if ws_bytes is None else ws_bytes(need), dtype=torch.uint8,
                     device="cuda")
    g = api.kdn_bwd("diag", d["q"], d["k"], d["v"], d["alpha"], d["omega"], d["r"], d["do"],
                    S0=d.get("S0"), var0=d.get("var0"), mu=mu,
                    mu_h=None if mu_h is None else torch.from_numpy(mu_h).cuda(),
                    c0_h=None if c0_h is None else torch.from_numpy(c0_h).cuda(),
                    dS_T=d.get("dS_T"), dvar_T=d.get("dvar_T"), workspace=ws)
    torch.cuda.synchronize()
    return {n: g[n].float().cpu().numpy() for n in NAMES}


CASES = [
    # (B, T, H, d, segments, slow decay, initial state and final gradients)
    (1, 2048, 2, 128, 2, False, True),
    (1, 4096, 2, 64, 4, True, True),
    (1, 8192, 1, 64, 8, True, True),
    (2, 8192, 1, 128, 8, True, False),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dT%dH%dd%d-S%d-slow%d-state%d" % c)
def test_bwd_split_matches_oracle_and_serial(ora, case):
    B, T, H, d, S, slow, full = case
    print("bwd split case %s" % (case,), flush=True)
    x = tb._case("diag", "bf16", B, T, H, d, d, seed=900 + T + d + B, full_state=full)
    if slow:
        rng = np.random.default_rng(901)
        x["alpha"] = (1.0 / (1.0 + np.exp(-rng.normal(6.0, 0.5, x["alpha"].shape)))).astype(
            np.float32)
    g = _call(x)
    ser = _call(x, ws_bytes=lambda n: n - 1)
    ref = tb._oracle(ora, "diag", x)
    err = {n: rel_l2(g[n], ref[n]) for n in NAMES}
    err_ser = {n: rel_l2(ser[n], ref[n]) for n in NAMES}
    diff = {n: rel_l2(g[n], ser[n]) for n in NAMES}
    print("  split vs oracle %s" % {n: "%.1e" % e for n, e in err.items()}, flush=True)
    print("  serial vs oracle %s" % {n: "%.1e" % e for n, e in err_ser.items()}, flush=True)
    print("  split vs serial %s" % {n: "%.1e" % e for n, e in diff.items()}, flush=True)
    assert max(err.values()) <= TOL["bf16"], err
    assert max(diff.values()) <= 1e-3, diff
    if slow:
        assert any(not np.array_equal(g[n], ser[n]) for n in NAMES)


def test_bwd_split_per_head_mu_c0(ora):
    B, T, H, d = 1, 4096, 2, 64
    x = tb._case("diag", "bf16", B, T, H, d, d, seed=931, full_state=False)
    mu_h = np.array([2.0, 40.0], dtype=np.float32)
    c0_h = np.array([0.5, 2.0], dtype=np.float32)
    g = _call(x, mu_h=mu_h, c0_h=c0_h)
    ser = _call(x, ws_bytes=lambda n: n - 1, mu_h=mu_h, c0_h=c0_h)
    ref = tb._oracle(ora, "diag", x, mu_h=mu_h, c0_h=c0_h)
    err = {n: rel_l2(g[n], ref[n]) for n in NAMES}
    diff = {n: rel_l2(g[n], ser[n]) for n in NAMES}
    print("bwd split mu_h c0_h: vs oracle %s, vs serial %s" % (
        {n: "%.1e" % e for n, e in err.items()}, {n: "%.1e" % e for n, e in diff.items()}),
        flush=True)
    assert max(err.values()) <= TOL["bf16"], err
    assert max(diff.values()) <= 1e-3, diff
