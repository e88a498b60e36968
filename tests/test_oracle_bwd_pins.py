"""Pins of the oracle's backward pass (``oracle.bwd``).

The KDN reading notes train with the scanned recurrence (method part §8) but
print no gradient formulas, so the oracle's reverse-mode derivative is
derived.  It is pinned here to things it does not share code with:

* central finite differences of the oracle forward (``diag_fwd`` /
  ``iso_fwd``) for every input, the initial state and variance, the
  information scale and the per-head initial covariance, on tiny problems
  with several batch rows and heads, for a loss that touches o, S_T and the
  final variance;
* a closed form at T = 1 from a zero state, where o = (q . kappa) v.
"""
import numpy as np
import pytest


def _problem(variant, B=2, T=6, H=2, dk=3, dv=2, seed=0):
    rng = np.random.default_rng(seed)
    x = {
        "q": rng.standard_normal((B, T, H, dk)),
        "k": rng.standard_normal((B, T, H, dk)),
        "v": rng.standard_normal((B, T, H, dv)),
        "alpha": rng.uniform(0.5, 1.0, (B, T, H, dk)),
        "omega": rng.uniform(0.05, 0.5, (B, T, H) if variant == "iso" else (B, T, H, dk)),
        "r": rng.uniform(0.5, 2.0, (B, T, H)),
        "S0": rng.standard_normal((B, H, dk, dv)),
        "var0": rng.uniform(0.2, 1.5, (B, H) if variant == "iso" else (B, H, dk)),
    }
    w = {
        "do": rng.standard_normal((B, T, H, dv)),
        "dS_T": rng.standard_normal((B, H, dk, dv)),
        "dvar_T": rng.standard_normal(x["var0"].shape),
    }
    return x, w


def _loss(ora, variant, x, w, mu, mu_h=None, c0_h=None):
    fn = ora.diag_fwd if variant == "diag" else ora.iso_fwd
    var_key = "p0" if variant == "diag" else "b0"
    out = fn(x["q"], x["k"], x["v"], x["alpha"], x["omega"], x["r"], S0=x["S0"],
             mu=mu, mu_h=mu_h, c0_h=c0_h, **{var_key: x["var0"]})
    var = out["p"] if variant == "diag" else out["b"]
    return (np.sum(out["o"] * w["do"]) + np.sum(out["S"] * w["dS_T"])
            + np.sum(var * w["dvar_T"]))


def _fd(f, x, eps=1e-6):
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        old = x[idx]
        x[idx] = old + eps
        lp = f()
        x[idx] = old - eps
        lm = f()
        x[idx] = old
        g[idx] = (lp - lm) / (2 * eps)
    return g


def _close(an, fd):
    scale = max(np.abs(fd).max(), 1e-3)
    return np.abs(an - fd).max() <= 1e-6 * scale


@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_bwd_matches_finite_differences(ora, variant):
    x, w = _problem(variant)
    mu = 2.7
    g = ora.bwd(variant, x["q"], x["k"], x["v"], x["alpha"], x["omega"], x["r"], w["do"],
                S0=x["S0"], var0=x["var0"], mu=mu, dS_T=w["dS_T"], dvar_T=w["dvar_T"])
    f = lambda: _loss(ora, variant, x, w, mu)
    names = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "omega": "domega",
             "r": "dr", "S0": "dS0", "var0": "dvar0"}
    for n, gn in names.items():
        fd = _fd(f, x[n])
        assert _close(g[gn], fd), (variant, n, np.abs(g[gn] - fd).max())
    # the information scale: dL/dmu sums every (b,h)'s derivative
    mu_arr = np.array([mu])
    fd_mu = _fd(lambda: _loss(ora, variant, x, w, float(mu_arr[0])), mu_arr)
    assert _close(np.array([g["dmu"].sum()]), fd_mu)


@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_bwd_per_head_mu_and_c0(ora, variant):
    x, w = _problem(variant, seed=1)
    del x["var0"]
    w["dvar_T"] = np.random.default_rng(2).standard_normal((2, 2) if variant == "iso" else (2, 2, 3))
    mu_h = np.array([0.7, 5.0])
    c0_h = np.array([0.4, 1.9])
    var_key = "p0" if variant == "diag" else "b0"

    def loss():
        fn = ora.diag_fwd if variant == "diag" else ora.iso_fwd
        out = fn(x["q"], x["k"], x["v"], x["alpha"], x["omega"], x["r"], S0=x["S0"],
                 mu_h=mu_h, c0_h=c0_h, **{var_key: None})
        var = out["p"] if variant == "diag" else out["b"]
        return (np.sum(out["o"] * w["do"]) + np.sum(out["S"] * w["dS_T"])
                + np.sum(var * w["dvar_T"]))

    g = ora.bwd(variant, x["q"], x["k"], x["v"], x["alpha"], x["omega"], x["r"], w["do"],
                S0=x["S0"], mu_h=mu_h, c0_h=c0_h, dS_T=w["dS_T"], dvar_T=w["dvar_T"])
    assert _close(g["dmu"].sum(axis=0), _fd(loss, mu_h))
    dc0 = g["dvar0"].sum(axis=0) if variant == "iso" else g["dvar0"].sum(axis=(0, 2))
    assert _close(dc0, _fd(loss, c0_h))
    assert _close(g["dk"], _fd(loss, x["k"]))


@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_bwd_single_token_closed_form(ora, variant):
    # T = 1 from S = 0: delta = v, S_1 = kappa v^T, o = (q . kappa) v, so
    # dL/dv = (q . kappa) do and dL/dq = kappa (v . do) for L = sum(do * o)
    rng = np.random.default_rng(5)
    B, H, dk, dv = 1, 1, 4, 3
    q, k = rng.standard_normal((2, B, 1, H, dk))
    v, do = rng.standard_normal((2, B, 1, H, dv))
    alpha = rng.uniform(0.6, 1.0, (B, 1, H, dk))
    omega = rng.uniform(0.1, 0.4, (B, 1, H) if variant == "iso" else (B, 1, H, dk))
    r = np.full((B, 1, H), 0.8)
    fn = ora.diag_fwd if variant == "diag" else ora.iso_fwd
    kap = fn(q, k, v, alpha, omega, r, return_gain=True)
    kappa = kap["kappa"] if variant == "diag" else kap["beta"][..., None] * k
    g = ora.bwd(variant, q, k, v, alpha, omega, r, do)
    qk = float(np.sum(q * kappa))
    np.testing.assert_allclose(g["dv"], qk * do, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g["dq"], kappa * float(np.sum(v * do)), rtol=1e-12, atol=1e-14)
    # and through the decay, dL/dS0 = diag(alpha) (q - (q . kappa) k) do^T
    a0, q0, k0, d0 = alpha[0, 0, 0], q[0, 0, 0], k[0, 0, 0], do[0, 0, 0]
    np.testing.assert_allclose(g["dS0"][0, 0], a0[:, None] * np.outer(q0 - qk * k0, d0),
                               rtol=1e-12, atol=1e-14)


def test_bwd_empty_sequence_passes_adjoints_through(ora):
    B, H, dk, dv = 2, 2, 3, 2
    z = lambda *s: np.zeros(s)
    rng = np.random.default_rng(9)
    dS_T = rng.standard_normal((B, H, dk, dv))
    dp_T = rng.standard_normal((B, H, dk))
    g = ora.bwd("diag", z(B, 0, H, dk), z(B, 0, H, dk), z(B, 0, H, dv), z(B, 0, H, dk),
                z(B, 0, H, dk), z(B, 0, H), z(B, 0, H, dv), dS_T=dS_T, dvar_T=dp_T)
    assert np.array_equal(g["dS0"], dS_T) and np.array_equal(g["dvar0"], dp_T)
