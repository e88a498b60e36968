"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these tests touches the GPU.  Each pin checks the oracle against
something other than itself: printed worked-example values (tests/golden),
closed forms, an exact dense Kalman filter that is itself pinned (printed
collision table + batch Bayesian regression), the textbook delta rule, and
invariants the notes state.  Sizes use d_k != d_v so a transposed state
fails loudly.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_inputs(rng, B, T, H, dk, dv, variant="diag"):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    alpha = 1.0 / (1.0 + np.exp(-(2.0 + 0.5 * rng.standard_normal((B, T, H, dk)))))
    wshape = (B, T, H, dk) if variant == "diag" else (B, T, H)
    omega = np.log1p(np.exp(rng.standard_normal(wshape)))
    r = np.log1p(np.exp(rng.standard_normal((B, T, H))))
    return q, k, v, alpha, omega, r


# ---------------------------------------------------------------------------
# Dense Kalman filter: pinned to the printed collision table and to batch
# Bayesian linear regression, so it can serve as the reference below.
# ---------------------------------------------------------------------------
def _collision_run(ora, cfg, reset):
    D, m, rho = cfg["D"], cfg["m"], cfg["rho"]
    r2, l2 = cfg["r2"], cfg["l2"]
    e = np.eye(D)
    keys = [e[0], rho * e[0] + np.sqrt(1 - rho ** 2) * e[1], e[2], e[3], e[4], e[5]]
    vals = np.eye(m)
    order = [0, 1, 2, 3, 4, 5] * 2 + [1] * 40 + [0] * 60
    T = len(order)
    K = np.array([keys[i] for i in order])
    V = np.array([vals[i] for i in order])
    Q = np.tile(keys[1], (T, 1))
    r = np.full(T, r2)
    if not reset:
        Dm = np.tile(np.eye(D), (T, 1, 1))
        Om = np.tile(l2 * np.eye(D), (T, 1, 1))
        out = ora.dense_kf(K, V, Q, Dm, Om, r, np.zeros((D, m)),
                           cfg["P0_scale"] * np.eye(D))
        gain = out["z"] / (r + out["z"])
        y = out["o"]
    else:
        # reset control: the predicted covariance is set to l2*I every step,
        # i.e. the delta rule with eta = l2 / (r2 + l2 |k|^2)
        beta = l2 / (r2 + l2 * np.sum(K * K, axis=1))
        out = ora.gated_delta_rule(K, V, Q, np.ones((T, D)), beta, np.zeros((D, m)))
        gain = beta * np.sum(K * K, axis=1)
        y = out["o"]
    pAB = np.exp(y[:, 1]) / (np.exp(y[:, 0]) + np.exp(y[:, 1]))
    return pAB, gain


def test_dense_kf_collision_table(ora):
    g = _golden("bl_collision_example.json")
    cfg, pr = g["setup"], g["printed"]
    tol = 0.5 * 10.0 ** (-g["printed_decimals"]) + 1e-12
    pAB, gain = _collision_run(ora, cfg, reset=False)
    assert abs(pAB[51] - pr["bl_pAB_t52"]) <= tol
    assert abs(pAB[111] - pr["bl_pAB_t112"]) <= tol
    assert abs((2 * pAB[111] - 1) - pr["bl_delta_t112"]) <= 2 * tol
    assert abs(gain[52] - pr["bl_gain_t53"]) <= tol
    assert abs(gain[111] - pr["bl_gain_longrun"]) <= tol
    pAB_r, gain_r = _collision_run(ora, cfg, reset=True)
    assert abs(pAB_r[51] - pr["reset_pAB_t52"]) <= tol
    assert abs(pAB_r[111] - pr["reset_pAB_t112"]) <= tol
    assert abs((2 * pAB_r[111] - 1) - pr["reset_delta_t112"]) <= 2 * tol
    assert np.allclose(gain_r, pr["reset_gain"], atol=1e-15)


def test_dense_kf_steady_state_gain_closed_form(ora):
    # BL notes §2.5: x_{t+1} = r2 x/(r2 + x) + l2 has fixed point
    # x_inf = (l2 + sqrt(l2^2 + 4 r2 l2))/2 and g_inf = x_inf/(r2 + x_inf).
    g = _golden("bl_collision_example.json")
    for r2, l2 in [(0.05, 0.05), (0.3, 0.02), (1.0, 2.0)]:
        x_inf = (l2 + np.sqrt(l2 ** 2 + 4 * r2 * l2)) / 2
        g_inf = x_inf / (r2 + x_inf)
        T = 400
        k = np.tile([1.0, 0.0, 0.0], (T, 1))
        out = ora.dense_kf(k, np.ones((T, 2)), k, np.tile(np.eye(3), (T, 1, 1)),
                           np.tile(l2 * np.eye(3), (T, 1, 1)), np.full(T, r2),
                           np.zeros((3, 2)), np.eye(3))
        gain = out["z"] / (r2 + out["z"])
        assert abs(gain[-1] - g_inf) < 1e-12
    assert abs(g["printed"]["g_inf_closed_form_r2_l2_0.05"]
               - (0.05 + np.sqrt(0.05 ** 2 + 4 * 0.05 ** 2)) / 2
               / (0.05 + (0.05 + np.sqrt(0.05 ** 2 + 4 * 0.05 ** 2)) / 2)) < 5e-7


def test_dense_kf_equals_batch_bayesian_regression(ora):
    # With D = I and Omega = 0 the filter's posterior is the batch posterior of
    # Bayesian linear regression: P_T = (P0^-1 + sum k k^T / r)^-1 and
    # S_T = P_T (P0^-1 S0 + sum k v^T / r).
    rng = np.random.default_rng(1)
    T, dk, dv = 30, 5, 3
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    r = 0.2 + rng.random(T)
    A = rng.standard_normal((dk, dk))
    P0 = A @ A.T + 0.5 * np.eye(dk)
    S0 = rng.standard_normal((dk, dv))
    out = ora.dense_kf(k, v, k, np.tile(np.eye(dk), (T, 1, 1)), np.zeros((T, dk, dk)),
                       r, S0, P0)
    prec = np.linalg.inv(P0) + (k.T / r) @ k
    P_T = np.linalg.inv(prec)
    S_T = P_T @ (np.linalg.inv(P0) @ S0 + (k.T / r) @ v)
    assert np.allclose(out["P"], P_T, rtol=1e-10, atol=1e-12)
    assert np.allclose(out["S"], S_T, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# P-a: scalar teaching values (KDN notes §2)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_scalar_teaching_values(ora, variant):
    g = _golden("kdn_teaching_examples.json")
    one = np.ones((1, 1, 1, 1))
    for case in g["scalar_gain"]["cases"]:
        tol = 0.5 * 10.0 ** (-case["printed_decimals"])
        # alpha = 1, omega = 0, p0 = phat  =>  predicted variance = phat
        if variant == "diag":
            out = ora.diag_fwd(one, one, one, one, 0 * one, np.ones((1, 1, 1)),
                               p0=np.full((1, 1, 1), case["phat"]), mu=1.0, return_gain=True)
            gain = out["kappa"][0, 0, 0, 0]
        else:
            out = ora.iso_fwd(one, one, one, one, np.zeros((1, 1, 1)), np.ones((1, 1, 1)),
                              b0=np.full((1, 1), case["phat"]), mu=1.0, return_gain=True)
            gain = out["beta"][0, 0, 0]
        assert abs(gain - case["gain"]) <= tol
    n_max = g["repeated_observation"]["n_max"]
    T = n_max
    ones = np.ones((1, T, 1, 1))
    for n in (1, 2, 7, n_max):
        if variant == "diag":
            out = ora.diag_fwd(ones[:, :n], ones[:, :n], ones[:, :n], ones[:, :n],
                               0 * ones[:, :n], np.ones((1, n, 1)), mu=1.0)
            p = out["p"][0, 0, 0]
        else:
            out = ora.iso_fwd(ones[:, :n], ones[:, :n], ones[:, :n], ones[:, :n],
                              np.zeros((1, n, 1)), np.ones((1, n, 1)), mu=1.0)
            p = out["b"][0, 0]
        assert abs(p - 1.0 / (n + 1)) < 1e-14


# ---------------------------------------------------------------------------
# P-b: uniform-energy example (KDN notes §5, Appendix B)
# ---------------------------------------------------------------------------
def test_uniform_energy_example(ora):
    g = _golden("kdn_teaching_examples.json")["uniform_energy"]
    m, p, r = g["m"], g["p"], g["r"]
    tol = 0.5 * 10.0 ** (-g["printed_decimals"])
    k = np.full((1, 1, 1, m), np.sqrt(1.0 / m))
    ones = np.ones((1, 1, 1, m))
    for mu, expect in ((1.0, g["V_proj_mu1"]), (float(m), g["V_proj_mu128"])):
        out = ora.diag_fwd(ones, k, np.ones((1, 1, 1, 2)), ones, 0 * ones,
                           np.full((1, 1, 1), r), p0=np.full((1, 1, m), p), mu=mu)
        V = float(np.sum(k[0, 0, 0] ** 2 * out["p"][0, 0]))
        assert abs(V - expect) <= tol
    # exact dense directional variance k^T P* k from the dense filter
    kk = k[0, 0]
    out = ora.dense_kf(kk, np.ones((1, 2)), kk, np.eye(m)[None], np.zeros((1, m, m)),
                       np.array([r]), np.zeros((m, 2)), p * np.eye(m))
    assert abs(float(kk[0] @ out["P"] @ kk[0]) - g["V_exact"]) <= tol


# ---------------------------------------------------------------------------
# P-c / P-e: one step against the dense filter (KDN notes §4, §7)
# ---------------------------------------------------------------------------
def test_diag_one_step_matches_dense_posterior(ora):
    rng = np.random.default_rng(2)
    dk, dv = 7, 4
    for trial in range(5):
        q, k, v, alpha, omega, r = _rand_inputs(rng, 1, 1, 1, dk, dv)
        k = k * (0.5 + 2 * rng.random())      # arbitrary key norm
        p0 = 0.1 + rng.random((1, 1, dk))
        S0 = rng.standard_normal((1, 1, dk, dv))
        out = ora.diag_fwd(q, k, v, alpha, omega, r, S0=S0, p0=p0, mu=1.0)
        D = np.diag(alpha[0, 0, 0])[None]
        Om = np.diag(omega[0, 0, 0])[None]
        den = ora.dense_kf(k[0, :, 0], v[0, :, 0], q[0, :, 0], D, Om, r[0, :, 0],
                           S0[0, 0], np.diag(p0[0, 0]))
        # mean: exact one-step posterior mean
        assert np.allclose(out["S"][0, 0], den["S"], rtol=1e-12, atol=1e-13)
        assert np.allclose(out["o"][0, 0, 0], den["o"][0], rtol=1e-12, atol=1e-13)
        # variance: p_i = 1 / (P*^{-1})_ii  (reverse-KL diagonal projection)
        prec = np.linalg.inv(den["P"])
        assert np.allclose(out["p"][0, 0], 1.0 / np.diag(prec), rtol=1e-10)
        # and it is NOT the diagonal of P* (unless k is axis-aligned)
        assert not np.allclose(out["p"][0, 0], np.diag(den["P"]), rtol=1e-6)


def test_iso_one_step_projections(ora):
    rng = np.random.default_rng(3)
    dk, dv = 6, 5
    for trial in range(5):
        q, k, v, alpha, omega, r = _rand_inputs(rng, 1, 1, 1, dk, dv, "iso")
        k = k * (0.5 + 2 * rng.random())
        b0 = 0.1 + rng.random((1, 1))
        S0 = rng.standard_normal((1, 1, dk, dv))
        out = ora.iso_fwd(q, k, v, alpha, omega, r, S0=S0, b0=b0, mu=1.0, return_gain=True)
        D = np.diag(alpha[0, 0, 0])[None]
        Om = (omega[0, 0, 0] * np.eye(dk))[None]
        den = ora.dense_kf(k[0, :, 0], v[0, :, 0], q[0, :, 0], D, Om, r[0, :, 0],
                           S0[0, 0], b0[0, 0] * np.eye(dk))
        # predict: trace (Frobenius-nearest isotropic) projection of P^
        assert abs(out["bhat"][0, 0, 0] - np.trace(den["Phat"][0]) / dk) < 1e-13
        # update: harmonic mean of the posterior eigenvalues of the projected
        # prior's exact posterior  (P* = (b^^-1 I + k k^T / r)^-1)
        bh = out["bhat"][0, 0, 0]
        kk = k[0, 0, 0]
        Pstar = np.linalg.inv(np.eye(dk) / bh + np.outer(kk, kk) / r[0, 0, 0])
        assert abs(out["b"][0, 0] - dk / np.trace(np.linalg.inv(Pstar))) < 1e-12
        # mean: exact KF mean under the isotropic predicted prior
        den_iso = ora.dense_kf(k[0, :, 0], v[0, :, 0], q[0, :, 0], D, np.zeros((1, dk, dk)),
                               r[0, :, 0], S0[0, 0], bh * np.linalg.inv(D[0] @ D[0]))
        assert np.allclose(out["S"][0, 0], den_iso["S"], rtol=1e-11, atol=1e-12)
    # mu = d_k and |k| = 1  =>  u = 1/r: b = b^/(1 + b^/r)
    q, k, v, alpha, omega, r = _rand_inputs(rng, 1, 1, 1, dk, dv, "iso")
    out = ora.iso_fwd(q, k, v, alpha, omega, r, mu=float(dk), return_gain=True)
    bh = out["bhat"][0, 0, 0]
    assert abs(out["b"][0, 0] - bh / (1 + bh / r[0, 0, 0])) < 1e-14


# ---------------------------------------------------------------------------
# P-d / P-f: multi-step equivalences with the dense filter
# ---------------------------------------------------------------------------
def test_diag_axis_aligned_keys_equal_dense_kf(ora):
    # With axis-aligned keys the exact posterior stays diagonal, so the
    # diagonal projection is exact at every step (mu = 1).
    rng = np.random.default_rng(4)
    T, dk, dv = 60, 4, 3
    q, _, v, alpha, omega, r = _rand_inputs(rng, 1, T, 1, dk, dv)
    k = np.zeros((1, T, 1, dk))
    idx = rng.integers(0, dk, T)
    k[0, np.arange(T), 0, idx] = 0.3 + 2 * rng.random(T)
    p0 = 0.2 + rng.random((1, 1, dk))
    S0 = rng.standard_normal((1, 1, dk, dv))
    out = ora.diag_fwd(q, k, v, alpha, omega, r, S0=S0, p0=p0, mu=1.0, return_gain=True)
    D = np.stack([np.diag(a) for a in alpha[0, :, 0]])
    Om = np.stack([np.diag(w) for w in omega[0, :, 0]])
    den = ora.dense_kf(k[0, :, 0], v[0, :, 0], q[0, :, 0], D, Om, r[0, :, 0],
                       S0[0, 0], np.diag(p0[0, 0]))
    assert np.allclose(out["o"][0, :, 0], den["o"], rtol=1e-11, atol=1e-12)
    assert np.allclose(out["S"][0, 0], den["S"], rtol=1e-11, atol=1e-12)
    assert np.allclose(out["kappa"][0, :, 0], den["kappa"], rtol=1e-11, atol=1e-13)
    assert np.allclose(out["p"][0, 0], np.diag(den["P"]), rtol=1e-11)
    assert np.allclose(den["P"], np.diag(np.diag(den["P"])), atol=1e-14)


@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_scalar_case_equals_scalar_kf(ora, variant):
    rng = np.random.default_rng(5)
    T, dv = 80, 3
    q, k, v, alpha, omega, r = _rand_inputs(rng, 1, T, 1, 1, dv, variant)
    k = k * (0.2 + 2 * rng.random((1, T, 1, 1)))
    S0 = rng.standard_normal((1, 1, 1, dv))
    w = omega if variant == "diag" else omega[..., None]
    den = ora.dense_kf(k[0, :, 0], v[0, :, 0], q[0, :, 0], alpha[0, :, 0, :, None],
                       w[0, :, 0, :, None], r[0, :, 0], S0[0, 0], np.eye(1) * 0.7)
    if variant == "diag":
        out = ora.diag_fwd(q, k, v, alpha, omega, r, S0=S0,
                           p0=np.full((1, 1, 1), 0.7), mu=1.0)
        var = out["p"][0, 0, 0]
    else:
        out = ora.iso_fwd(q, k, v, alpha, omega, r, S0=S0, b0=np.full((1, 1), 0.7), mu=1.0)
        var = out["b"][0, 0]
    assert np.allclose(out["o"][0, :, 0], den["o"], rtol=1e-11, atol=1e-12)
    assert np.allclose(out["S"][0, 0], den["S"], rtol=1e-11, atol=1e-12)
    assert abs(var - den["P"][0, 0]) < 1e-12 * max(1.0, den["P"][0, 0])


# ---------------------------------------------------------------------------
# P-g: delta-rule special cases (KDN notes motivation §1, method §3)
# ---------------------------------------------------------------------------
def test_iso_memory_path_is_gated_delta_rule(ora):
    rng = np.random.default_rng(6)
    T, dk, dv = 50, 6, 4
    q, k, v, alpha, omega, r = _rand_inputs(rng, 1, T, 1, dk, dv, "iso")
    S0 = rng.standard_normal((1, 1, dk, dv))
    out = ora.iso_fwd(q, k, v, alpha, omega, r, S0=S0, return_gain=True)
    ref = ora.gated_delta_rule(k[0, :, 0], v[0, :, 0], q[0, :, 0], alpha[0, :, 0],
                               out["beta"][0, :, 0], S0[0, 0])
    assert np.allclose(out["o"][0, :, 0], ref["o"], rtol=1e-12, atol=1e-12)
    assert np.allclose(out["S"][0, 0], ref["S"], rtol=1e-12, atol=1e-12)


def test_diag_isotropic_surrogate_is_gated_deltanet(ora):
    # Scalar decay per token, uniform process noise, uniform prior and mu = 0:
    # the predicted covariance stays b^_t I, so kappa = b^/(r + b^|k|^2) k
    # (the isotropic surrogate, KDN notes method §3 Eq. (18)-(20)) and the
    # memory is Gated DeltaNet with that beta.
    rng = np.random.default_rng(7)
    T, dk, dv = 40, 5, 3
    q, k, v, _, _, r = _rand_inputs(rng, 1, T, 1, dk, dv)
    k = k * (0.5 + rng.random((1, T, 1, 1)))
    a = 0.6 + 0.4 * rng.random(T)
    w = 0.05 + rng.random(T)
    alpha = np.broadcast_to(a[None, :, None, None], (1, T, 1, dk)).copy()
    omega = np.broadcast_to(w[None, :, None, None], (1, T, 1, dk)).copy()
    out = ora.diag_fwd(q, k, v, alpha, omega, r, p0=np.full((1, 1, dk), 0.8), mu=0.0)
    bh = np.zeros(T)
    prev = 0.8
    for t in range(T):
        bh[t] = a[t] ** 2 * prev + w[t]
        prev = bh[t]
    nrm = np.sum(k[0, :, 0] ** 2, axis=1)
    beta = bh / (r[0, :, 0] + bh * nrm)
    ref = ora.gated_delta_rule(k[0, :, 0], v[0, :, 0], q[0, :, 0], alpha[0, :, 0], beta,
                               np.zeros((dk, dv)))
    assert np.allclose(out["o"][0, :, 0], ref["o"], rtol=1e-12, atol=1e-12)
    assert np.allclose(out["S"][0, 0], ref["S"], rtol=1e-12, atol=1e-12)


def test_iso_fixed_beta_deltanet(ora):
    # mu = 0, alpha = 1, omega = 0: b stays b0, beta = b0/(r + b0|k|^2) is
    # fixed and the layer is DeltaNet.
    rng = np.random.default_rng(8)
    T, dk, dv = 30, 4, 6
    q, k, v, _, _, _ = _rand_inputs(rng, 1, T, 1, dk, dv, "iso")
    r = np.full((1, T, 1), 0.3)
    out = ora.iso_fwd(q, k, v, np.ones((1, T, 1, dk)), np.zeros((1, T, 1)), r,
                      b0=np.full((1, 1), 2.0), mu=0.0)
    beta = np.full(T, 2.0 / (0.3 + 2.0))
    ref = ora.gated_delta_rule(k[0, :, 0], v[0, :, 0], q[0, :, 0], np.ones((T, dk)), beta,
                               np.zeros((dk, dv)))
    assert np.allclose(out["o"][0, :, 0], ref["o"], rtol=1e-12, atol=1e-12)
    assert abs(out["b"][0, 0] - 2.0) < 1e-15


# ---------------------------------------------------------------------------
# P-h: Moebius composition (KDN notes method §6)
# ---------------------------------------------------------------------------
def test_mobius_bracketings_match_sequential(ora):
    rng = np.random.default_rng(9)
    T, dk, dv = 200, 8, 2
    q, k, v, alpha, omega, r = _rand_inputs(rng, 1, T, 1, dk, dv)
    mu = float(dk)
    p0 = 0.1 + rng.random((1, 1, dk))
    out = ora.diag_fwd(q, k, v, alpha, omega, r, p0=p0, mu=mu, return_gain=True)
    u = (mu / r[0, :, 0, None]) * k[0, :, 0] ** 2
    for i in range(dk):
        Ms = ora.mobius_factors(alpha[0, :, 0, i], omega[0, :, 0, i], u[:, i])
        PL = ora.mobius_fold_left(Ms)
        PT = ora.mobius_fold_tree(Ms)
        for P in (PL, PT):
            pT = ora.mobius_apply(P, p0[0, 0, i])
            assert abs(pT - out["p"][0, 0, i]) <= 1e-13 * out["p"][0, 0, i]
        # every exclusive prefix gives the p_{t-1} that the gain uses
        for t in (1, 17, 100, T - 1):
            pprev = ora.mobius_apply(ora.mobius_fold_tree(Ms[:t]), p0[0, 0, i])
            phat = alpha[0, t, 0, i] ** 2 * pprev + omega[0, t, 0, i]
            assert abs(phat - out["phat"][0, t, 0, i]) <= 1e-13 * phat
    # order matters: reversing the tokens changes the result (not commutative)
    Ms = ora.mobius_factors(alpha[0, :, 0, 0], omega[0, :, 0, 0], u[:, 0])
    assert abs(ora.mobius_apply(ora.mobius_fold_left(Ms[::-1]), p0[0, 0, 0])
               - out["p"][0, 0, 0]) > 1e-9


# ---------------------------------------------------------------------------
# P-j: invariants (KDN notes method §2 beta_eff, §4, §5)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_invariants_random(ora, variant):
    rng = np.random.default_rng(10)
    B, T, H, dk, dv = 2, 64, 2, 16, 8
    q, k, v, alpha, omega, r = _rand_inputs(rng, B, T, H, dk, dv, variant)
    mu = float(dk)
    S = np.zeros((B, H, dk, dv))
    var = np.full((B, H, dk) if variant == "diag" else (B, H), 1.0)
    bound = np.maximum(1.0, np.max(omega) / (1 - np.max(alpha) ** 2))
    for t in range(T):
        st = ora.step(variant, q[:, t], k[:, t], v[:, t], alpha[:, t], omega[:, t], r[:, t],
                      S, var, mu=mu)
        a2 = alpha[:, t] ** 2
        if variant == "diag":
            phat = a2 * var + omega[:, t]
            kk = k[:, t] ** 2
            z = np.sum(phat * kk, axis=-1)
            kappa = phat * k[:, t] / (r[:, t] + z)[..., None]
            newv = st["var"]
            assert np.all(newv > 0) and np.all(newv <= phat)
            assert np.all(newv < r[:, t][..., None] / (mu * kk))
        else:
            phat = np.mean(a2, axis=-1) * var + omega[:, t]
            n = np.sum(k[:, t] ** 2, axis=-1)
            kappa = (phat / (r[:, t] + phat * n))[..., None] * k[:, t]
            newv = st["var"]
            assert np.all(newv > 0) and np.all(newv <= phat)
        assert np.all(newv <= bound)
        beta_eff = np.sum(k[:, t] * kappa, axis=-1)
        assert np.all(beta_eff >= 0) and np.all(beta_eff < 1)
        # the state after the write matches S^ + kappa delta^T with this kappa
        Sh = alpha[:, t][..., None] * S
        delta = v[:, t] - np.einsum("bhij,bhi->bhj", Sh, k[:, t])
        assert np.allclose(st["S"], Sh + kappa[..., None] * delta[..., None, :],
                           rtol=1e-12, atol=1e-12)
        # read after write
        assert np.allclose(st["o"], np.einsum("bhij,bhi->bhj", st["S"], q[:, t]),
                           rtol=1e-12, atol=1e-12)
        S, var = st["S"], newv


# ---------------------------------------------------------------------------
# P-k: mu leaves the current write unchanged (KDN notes method §5)
# ---------------------------------------------------------------------------
def test_mu_does_not_change_current_write(ora):
    rng = np.random.default_rng(11)
    T, dk, dv = 12, 8, 5
    q, k, v, alpha, omega, r = _rand_inputs(rng, 1, T, 1, dk, dv)
    first = [ora.diag_fwd(q[:, :1], k[:, :1], v[:, :1], alpha[:, :1], omega[:, :1],
                          r[:, :1], mu=mu, return_gain=True) for mu in (0.0, 1.0, float(dk))]
    for o in first[1:]:
        assert np.array_equal(o["kappa"], first[0]["kappa"])
        assert np.array_equal(o["S"], first[0]["S"])
        assert np.array_equal(o["o"], first[0]["o"])
    assert not np.allclose(first[1]["p"], first[2]["p"])
    # switch mu at token t: kappa_{<=t} unchanged, kappa_{t+1} changes
    t = 6
    full = ora.diag_fwd(q, k, v, alpha, omega, r, mu=1.0, return_gain=True)
    head = ora.diag_fwd(q[:, :t], k[:, :t], v[:, :t], alpha[:, :t], omega[:, :t],
                        r[:, :t], mu=1.0)
    tail = ora.diag_fwd(q[:, t:], k[:, t:], v[:, t:], alpha[:, t:], omega[:, t:], r[:, t:],
                        S0=head["S"], p0=head["p"], mu=float(dk), return_gain=True)
    assert np.allclose(tail["kappa"][:, 0], full["kappa"][:, t], rtol=1e-14, atol=1e-15)
    assert not np.allclose(tail["kappa"][:, 1], full["kappa"][:, t + 1], rtol=1e-6)


# ---------------------------------------------------------------------------
# P-l: resume and decode consistency (KDN notes method §8)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_resume_and_step_consistency(ora, variant):
    rng = np.random.default_rng(12)
    B, T, H, dk, dv = 2, 20, 3, 8, 6
    q, k, v, alpha, omega, r = _rand_inputs(rng, B, T, H, dk, dv, variant)
    fwd = ora.diag_fwd if variant == "diag" else ora.iso_fwd
    vkey = "p" if variant == "diag" else "b"
    full = fwd(q, k, v, alpha, omega, r)
    t1 = 7
    a = fwd(q[:, :t1], k[:, :t1], v[:, :t1], alpha[:, :t1], omega[:, :t1], r[:, :t1])
    kw = {"p0": a["p"]} if variant == "diag" else {"b0": a["b"]}
    b = fwd(q[:, t1:], k[:, t1:], v[:, t1:], alpha[:, t1:], omega[:, t1:], r[:, t1:],
            S0=a["S"], **kw)
    assert np.allclose(np.concatenate([a["o"], b["o"]], axis=1), full["o"], rtol=1e-13,
                       atol=1e-14)
    assert np.allclose(b["S"], full["S"], rtol=1e-13, atol=1e-14)
    assert np.allclose(b[vkey], full[vkey], rtol=1e-13)
    S = np.zeros((B, H, dk, dv))
    var = np.ones(full[vkey].shape)
    for t in range(T):
        st = ora.step(variant, q[:, t], k[:, t], v[:, t], alpha[:, t], omega[:, t], r[:, t],
                      S, var)
        assert np.allclose(st["o"], full["o"][:, t], rtol=1e-13, atol=1e-14)
        S, var = st["S"], st["var"]
    assert np.allclose(S, full["S"], rtol=1e-13, atol=1e-14)


def test_oracle_rejects_bad_sizes(ora):
    with pytest.raises(Exception):
        ora.diag_fwd(np.zeros((1, 2, 1, 3)), np.zeros((1, 2, 1, 4)), np.zeros((1, 2, 1, 2)),
                     np.zeros((1, 2, 1, 4)), np.zeros((1, 2, 1, 4)), np.zeros((1, 2, 1)))


def test_empty_sequence_returns_initial_state(ora):
    rng = np.random.default_rng(13)
    S0 = rng.standard_normal((1, 2, 4, 3))
    p0 = 0.5 + rng.random((1, 2, 4))
    z4 = np.zeros((1, 0, 2, 4))
    out = ora.diag_fwd(z4, z4, np.zeros((1, 0, 2, 3)), z4, z4, np.zeros((1, 0, 2)),
                       S0=S0, p0=p0)
    assert out["o"].shape == (1, 0, 2, 3)
    assert np.array_equal(out["S"], S0) and np.array_equal(out["p"], p0)


# ---------------------------------------------------------------------------
# P-m: per-head trained parameters (KDN notes method §8: a learned initial
# covariance c_{0,h} I and scale mu per head) and the effective write strength
# (method §2: beta_eff = k^T kappa = z / (r + z))
# ---------------------------------------------------------------------------
def _fwd(ora, variant, *args, **kw):
    if variant == "iso" and "p0" in kw:
        kw["b0"] = kw.pop("p0")
    return (ora.diag_fwd if variant == "diag" else ora.iso_fwd)(*args, **kw)


def test_beta_eff_equals_dense_kf_write_strength(ora):
    # axis-aligned keys keep the exact posterior diagonal (pinned above), so
    # beta_eff must be z / (r + z) with z = k^T P^ k of the dense filter
    rng = np.random.default_rng(21)
    T, dk, dv = 50, 4, 3
    q, _, v, alpha, omega, r = _rand_inputs(rng, 1, T, 1, dk, dv)
    k = np.zeros((1, T, 1, dk))
    idx = rng.integers(0, dk, T)
    k[0, np.arange(T), 0, idx] = 0.3 + 2 * rng.random(T)
    p0 = 0.2 + rng.random((1, 1, dk))
    out = ora.diag_fwd(q, k, v, alpha, omega, r, p0=p0, mu=1.0, return_beta_eff=True)
    D = np.stack([np.diag(a) for a in alpha[0, :, 0]])
    Om = np.stack([np.diag(w) for w in omega[0, :, 0]])
    den = ora.dense_kf(k[0, :, 0], v[0, :, 0], q[0, :, 0], D, Om, r[0, :, 0],
                       np.zeros((dk, dv)), np.diag(p0[0, 0]))
    ref = den["z"] / (r[0, :, 0] + den["z"])
    assert np.allclose(out["beta_eff"][0, :, 0], ref, rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_beta_eff_is_key_times_gain(ora, variant):
    rng = np.random.default_rng(22)
    B, T, H, dk, dv = 2, 40, 3, 6, 5
    q, k, v, alpha, omega, r = _rand_inputs(rng, B, T, H, dk, dv, variant)
    k = k * (0.2 + 3 * rng.random((B, T, H, 1)))
    out = _fwd(ora, variant, q, k, v, alpha, omega, r, return_gain=True,
               return_beta_eff=True)
    if variant == "diag":
        ref = (out["kappa"] * k).sum(-1)
    else:
        ref = out["beta"] * (k * k).sum(-1)
    assert np.allclose(out["beta_eff"], ref, rtol=1e-12, atol=1e-15)
    assert (out["beta_eff"] >= 0).all() and (out["beta_eff"] < 1).all()


@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_per_head_mu_is_each_head_with_its_own_mu(ora, variant):
    rng = np.random.default_rng(23)
    B, T, H, dk, dv = 2, 30, 3, 6, 5
    q, k, v, alpha, omega, r = _rand_inputs(rng, B, T, H, dk, dv, variant)
    mu_h = np.array([0.5, 6.0, 40.0])
    full = _fwd(ora, variant, q, k, v, alpha, omega, r, mu_h=mu_h, return_beta_eff=True)
    var = "p" if variant == "diag" else "b"
    for h in range(H):
        sl = lambda x: np.ascontiguousarray(x[:, :, h:h + 1])
        one = _fwd(ora, variant, sl(q), sl(k), sl(v), sl(alpha), sl(omega), sl(r),
                   mu=float(mu_h[h]), return_beta_eff=True)
        assert np.array_equal(full["o"][:, :, h], one["o"][:, :, 0])
        assert np.array_equal(full["S"][:, h], one["S"][:, 0])
        assert np.array_equal(full[var][:, h], one[var][:, 0])
        assert np.array_equal(full["beta_eff"][:, :, h], one["beta_eff"][:, :, 0])
    flat = _fwd(ora, variant, q, k, v, alpha, omega, r, mu=float(dk))
    assert not np.allclose(full[var], flat[var])


@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_c0_is_a_filled_initial_variance(ora, variant):
    rng = np.random.default_rng(24)
    B, T, H, dk, dv = 2, 25, 3, 6, 5
    q, k, v, alpha, omega, r = _rand_inputs(rng, B, T, H, dk, dv, variant)
    c0 = np.array([0.3, 1.7, 4.0])
    a = _fwd(ora, variant, q, k, v, alpha, omega, r, c0_h=c0)
    shape = (B, H, dk) if variant == "diag" else (B, H)
    filled = np.ascontiguousarray(np.broadcast_to(
        c0[None, :, None] if variant == "diag" else c0[None, :], shape))
    b = _fwd(ora, variant, q, k, v, alpha, omega, r, p0=filled)
    for key in a:
        assert np.array_equal(a[key], b[key])
    ones = _fwd(ora, variant, q, k, v, alpha, omega, r)
    assert not np.allclose(a["o"], ones["o"])
