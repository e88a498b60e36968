"""fp64 CPU oracle for the Kalman Delta Network (KDN) mixer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``kalman_delta_rule_amd``) and never imports it.

Contents
--------
* ``diag_fwd`` / ``iso_fwd`` / ``step`` -- the token-by-token recurrences of
  Diagonal and Isotropic KDN, in plain C (``kdn_oracle.c``), fp64, one
  independent problem per (batch, head).  See that file for the equations and
  their citations (KDN reading notes, method part, §2, §4, §5, §7).
* ``bwd`` -- the backward pass of both recurrences (reverse-mode derivative,
  derived in ``kdn_oracle.c`` since the notes print no gradient formulas;
  pinned in the tests against finite differences of the forward).
* ``gate_prologue`` -- the gates from their pre-activations (KDN reading
  notes, method part §8): alpha = sigmoid(a), omega = softplus(w),
  r = r_min + softplus(rho); numpy, fp64.
* ``bwd_preact`` -- the backward of the forward from pre-activations (the
  chain rule through the prologue; pinned to finite differences).
* ``dense_kf`` -- the exact dense-covariance Kalman memory (KDN reading notes,
  method part §2, Eq. (12)-(17)); numpy, fp64, for tiny d_k only.
* ``mobius_factors`` / ``mobius_fold_left`` / ``mobius_fold_tree`` /
  ``mobius_apply`` -- the 2x2 Moebius form of the per-channel variance
  recurrence (KDN reading notes, method part §6, Eq. (32)-(39)), with the
  ratio-preserving max-abs rescaling the notes describe for Appendix D.
* ``gated_delta_rule`` -- the textbook delta-rule family
  S_t = D_t S_{t-1} + beta_t k_t (v_t - (D_t S_{t-1})^T k_t)^T
  (KDN reading notes, motivation part §1, the unified form and its table).

Inputs may be any float dtype; they are upcast exactly to float64 (bf16 and
fp32 values are representable in fp64), so the oracle reads the same values
the GPU reads.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkdn_oracle.so")
_lib = None


def build_oracle(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
             "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"],
            check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_oracle(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        for name in ("kdn_oracle_diag_fwd", "kdn_oracle_iso_fwd"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = ([ctypes.c_int] * 5 + [dp] * 9 + [ctypes.c_double]
                           + [dp] * 7 + [ctypes.c_int])
        lib.kdn_oracle_bwd.restype = ctypes.c_int
        lib.kdn_oracle_bwd.argtypes = ([ctypes.c_int] * 6 + [dp] * 9 + [ctypes.c_double]
                                       + [dp] * 13 + [ctypes.c_int])
        lib.kdn_oracle_max_threads.restype = ctypes.c_int
        lib.kdn_oracle_max_threads.argtypes = []
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().kdn_oracle_max_threads())


def _f64(x) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor on the CPU
        x = x.detach().to("cpu")
        x = x.double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _head_vec(x, H):
    x = _f64(x)
    if x is not None:
        assert x.shape == (H,)
    return x


def diag_fwd(q, k, v, alpha, omega, r, S0=None, p0=None, mu=None,
             return_gain: bool = False, nthreads: int = 0,
             mu_h=None, c0_h=None, return_beta_eff: bool = False) -> dict:
    """Diagonal KDN forward (KDN reading notes, method part §4-§5).

    Shapes: q,k [B,T,H,dk]; v [B,T,H,dv]; alpha, omega [B,T,H,dk]; r [B,T,H];
    S0 [B,H,dk,dv] or None (zeros); p0 [B,H,dk] or None (c0_h[h] per head,
    or ones); mu defaults to dk, mu_h [H] overrides it per head (method part
    §8: learned per-head scale and initial covariance).  Returns a dict with
    o [B,T,H,dv], S [B,H,dk,dv], p [B,H,dk], with ``return_gain`` also kappa
    and phat [B,T,H,dk], with ``return_beta_eff`` beta_eff [B,T,H] (method
    part §2: k^T kappa = z / (r + z)).
    """
    q, k, v, alpha, omega, r = map(_f64, (q, k, v, alpha, omega, r))
    S0, p0 = _f64(S0), _f64(p0)
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    assert q.shape == k.shape == alpha.shape == omega.shape
    assert v.shape == (B, T, H, dv) and r.shape == (B, T, H)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    if p0 is not None:
        assert p0.shape == (B, H, dk)
    mu = float(dk if mu is None else mu)
    mu_h, c0_h = _head_vec(mu_h, H), _head_vec(c0_h, H)
    o = np.zeros((B, T, H, dv))
    S = np.zeros((B, H, dk, dv))
    p = np.zeros((B, H, dk))
    kap = np.zeros((B, T, H, dk)) if return_gain else None
    ph = np.zeros((B, T, H, dk)) if return_gain else None
    be = np.zeros((B, T, H)) if return_beta_eff else None
    rc = _load().kdn_oracle_diag_fwd(
        B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(omega),
        _ptr(r), _ptr(S0), _ptr(p0), _ptr(c0_h), mu, _ptr(mu_h), _ptr(o), _ptr(S), _ptr(p),
        _ptr(kap), _ptr(ph), _ptr(be), int(nthreads))
    if rc != 0:
        raise RuntimeError("kdn_oracle_diag_fwd failed (%d)" % rc)
    out = {"o": o, "S": S, "p": p}
    if return_gain:
        out["kappa"] = kap
        out["phat"] = ph
    if return_beta_eff:
        out["beta_eff"] = be
    return out


def iso_fwd(q, k, v, alpha, omega, r, S0=None, b0=None, mu=None,
            return_gain: bool = False, nthreads: int = 0,
            mu_h=None, c0_h=None, return_beta_eff: bool = False) -> dict:
    """Isotropic KDN forward (KDN reading notes, method part §7, Eq. (40)).

    omega is [B,T,H]; b0 is [B,H] or None (c0_h[h] per head, or ones);
    mu_h as in diag_fwd.  Returns o, S, b, with ``return_gain`` also beta and
    bhat [B,T,H], with ``return_beta_eff`` beta_eff [B,T,H].
    """
    q, k, v, alpha, omega, r = map(_f64, (q, k, v, alpha, omega, r))
    S0, b0 = _f64(S0), _f64(b0)
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    assert q.shape == k.shape == alpha.shape
    assert omega.shape == (B, T, H) and r.shape == (B, T, H)
    assert v.shape == (B, T, H, dv)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    if b0 is not None:
        assert b0.shape == (B, H)
    mu = float(dk if mu is None else mu)
    mu_h, c0_h = _head_vec(mu_h, H), _head_vec(c0_h, H)
    o = np.zeros((B, T, H, dv))
    S = np.zeros((B, H, dk, dv))
    b = np.zeros((B, H))
    beta = np.zeros((B, T, H)) if return_gain else None
    bh = np.zeros((B, T, H)) if return_gain else None
    be = np.zeros((B, T, H)) if return_beta_eff else None
    rc = _load().kdn_oracle_iso_fwd(
        B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(omega),
        _ptr(r), _ptr(S0), _ptr(b0), _ptr(c0_h), mu, _ptr(mu_h), _ptr(o), _ptr(S), _ptr(b),
        _ptr(beta), _ptr(bh), _ptr(be), int(nthreads))
    if rc != 0:
        raise RuntimeError("kdn_oracle_iso_fwd failed (%d)" % rc)
    out = {"o": o, "S": S, "b": b}
    if return_gain:
        out["beta"] = beta
        out["bhat"] = bh
    if return_beta_eff:
        out["beta_eff"] = be
    return out


def step(variant: str, q, k, v, alpha, omega, r, S, var, mu=None, mu_h=None) -> dict:
    """One decode step: the forward recurrence at T = 1 (KDN reading notes,
    method part §8: scanned training and token-by-token inference are the same
    recurrence).  q,k,v,alpha: [B,H,D]; omega [B,H,dk] (diag) or [B,H] (iso);
    r [B,H]; S [B,H,dk,dv]; var = p [B,H,dk] or b [B,H]; mu_h [H] or None.
    Returns o [B,H,dv], the new S and variance, and beta_eff [B,H]."""
    t1 = lambda x: None if x is None else _f64(x)[:, None]
    if variant == "diag":
        out = diag_fwd(t1(q), t1(k), t1(v), t1(alpha), t1(omega), t1(r),
                       S0=S, p0=var, mu=mu, mu_h=mu_h, return_beta_eff=True)
        return {"o": out["o"][:, 0], "S": out["S"], "var": out["p"],
                "beta_eff": out["beta_eff"][:, 0]}
    if variant == "iso":
        out = iso_fwd(t1(q), t1(k), t1(v), t1(alpha), t1(omega), t1(r),
                      S0=S, b0=var, mu=mu, mu_h=mu_h, return_beta_eff=True)
        return {"o": out["o"][:, 0], "S": out["S"], "var": out["b"],
                "beta_eff": out["beta_eff"][:, 0]}
    raise ValueError("variant must be 'diag' or 'iso'")


def bwd(variant: str, q, k, v, alpha, omega, r, do, S0=None, var0=None, mu=None,
        mu_h=None, c0_h=None, dS_T=None, dvar_T=None, nthreads: int = 0) -> dict:
    """Backward of ``diag_fwd`` / ``iso_fwd`` for the loss
    L = sum(do * o) + sum(dS_T * S_T) + sum(dvar_T * var_T).

    Forward arguments as in those calls (var0 = p0 or b0); do has o's shape,
    dS_T and dvar_T default to zero.  Returns dq, dk, dv, dalpha, domega, dr
    (the shapes of the inputs), dS0, dvar0 (shape of the initial variance, also
    when it came from c0_h or the default) and dmu [B,H], the derivative by the
    information scale that (b,h) used.
    """
    if variant not in ("diag", "iso"):
        raise ValueError("variant must be 'diag' or 'iso'")
    iso = variant == "iso"
    q, k, v, alpha, omega, r, do = map(_f64, (q, k, v, alpha, omega, r, do))
    S0, var0, dS_T, dvar_T = map(_f64, (S0, var0, dS_T, dvar_T))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    var_shape = (B, H) if iso else (B, H, dk)
    assert q.shape == k.shape == alpha.shape and v.shape == do.shape == (B, T, H, dv)
    assert omega.shape == ((B, T, H) if iso else (B, T, H, dk)) and r.shape == (B, T, H)
    for x, shp in ((S0, (B, H, dk, dv)), (dS_T, (B, H, dk, dv)), (var0, var_shape),
                   (dvar_T, var_shape)):
        assert x is None or x.shape == shp
    mu = float(dk if mu is None else mu)
    mu_h, c0_h = _head_vec(mu_h, H), _head_vec(c0_h, H)
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
           "dalpha": np.zeros_like(alpha), "domega": np.zeros_like(omega),
           "dr": np.zeros_like(r), "dS0": np.zeros((B, H, dk, dv)),
           "dvar0": np.zeros(var_shape), "dmu": np.zeros((B, H))}
    rc = _load().kdn_oracle_bwd(
        int(iso), B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(omega), _ptr(r),
        _ptr(S0), _ptr(var0), _ptr(c0_h), mu, _ptr(mu_h), _ptr(do), _ptr(dS_T), _ptr(dvar_T),
        *[_ptr(out[n]) for n in ("dq", "dk", "dv", "dalpha", "domega", "dr", "dS0", "dvar0",
                                 "dmu")],
        int(nthreads))
    if rc != 0:
        raise RuntimeError("kdn_oracle_bwd failed (%d)" % rc)
    return out


def gate_prologue(a_pre, w_pre, r_pre, r_min: float = 0.01) -> dict:
    """The gates of the end-to-end network from their pre-activations (KDN
    reading notes, method part §8, where r_min = 0.01): alpha = sigmoid(a),
    omega = softplus(w) (one per channel for Diagonal, per token for
    Isotropic), r = r_min + softplus(rho), in fp64.  softplus(x) =
    log(1 + e^x) is evaluated as max(x, 0) + log1p(e^-|x|), the same value
    without overflow."""
    a, w, rho = map(_f64, (a_pre, w_pre, r_pre))
    softplus = lambda x: np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))
    return {"alpha": 1.0 / (1.0 + np.exp(-a)), "omega": softplus(w),
            "r": float(r_min) + softplus(rho)}


def bwd_preact(variant: str, q, k, v, a_pre, w_pre, r_pre, do, r_min: float = 0.01,
               **kw) -> dict:
    """Backward of the forward from gate pre-activations (``gate_prologue``
    followed by ``diag_fwd`` / ``iso_fwd``): ``bwd`` on the gates, then the
    chain rule through the activations, d sigmoid(a)/da = alpha (1 - alpha)
    and d softplus(x)/dx = sigmoid(x).  Returns bwd's dict with da_pre, dw_pre
    and dr_pre in place of dalpha, domega and dr.  Other keyword arguments go
    to ``bwd``."""
    g = gate_prologue(a_pre, w_pre, r_pre, r_min)
    out = bwd(variant, q, k, v, g["alpha"], g["omega"], g["r"], do, **kw)
    sig = lambda x: 1.0 / (1.0 + np.exp(-_f64(x)))
    out["da_pre"] = out.pop("dalpha") * g["alpha"] * (1.0 - g["alpha"])
    out["dw_pre"] = out.pop("domega") * sig(w_pre)
    out["dr_pre"] = out.pop("dr") * sig(r_pre)
    return out


# --------------------------------------------------------------------------
# Exact dense Kalman memory (test-only reference for tiny d_k)
# --------------------------------------------------------------------------
def dense_kf(k, v, q, D, Omega, r, S0, P0):
    """Exact dense Kalman associative memory, one head, token by token.

    KDN reading notes, method part §2, Eq. (12)-(17):
      S^ = D S,  P^ = D P D^T + Omega,  delta = v - S^^T k,
      kappa = P^ k / (r + k^T P^ k),  S = S^ + kappa delta^T,
      P = (I - kappa k^T) P^,  o = S^T q.
    k, q: [T,dk]; v: [T,dv]; D, Omega: [T,dk,dk] (full matrices); r: [T];
    S0 [dk,dv]; P0 [dk,dk].  Returns o [T,dv], S, P, kappa [T,dk],
    z [T] (= k^T P^ k) and Phat [T,dk,dk].
    """
    k, v, q = _f64(k), _f64(v), _f64(q)
    D, Omega, r = _f64(D), _f64(Omega), _f64(r)
    S = _f64(S0).copy()
    P = _f64(P0).copy()
    T, dk = k.shape
    dv = v.shape[1]
    o = np.zeros((T, dv))
    kap = np.zeros((T, dk))
    zs = np.zeros(T)
    Phats = np.zeros((T, dk, dk))
    eye = np.eye(dk)
    for t in range(T):
        Sh = D[t] @ S
        Ph = D[t] @ P @ D[t].T + Omega[t]
        delta = v[t] - Sh.T @ k[t]
        z = float(k[t] @ Ph @ k[t])
        kappa = Ph @ k[t] / (r[t] + z)
        S = Sh + np.outer(kappa, delta)
        P = (eye - np.outer(kappa, k[t])) @ Ph
        o[t] = S.T @ q[t]
        kap[t] = kappa
        zs[t] = z
        Phats[t] = Ph
    return {"o": o, "S": S, "P": P, "kappa": kap, "z": zs, "Phat": Phats}


# --------------------------------------------------------------------------
# 2x2 Moebius form of the per-channel variance recurrence
# --------------------------------------------------------------------------
def mobius_factors(alpha, omega, u):
    """M_t = [[alpha^2, omega], [u alpha^2, 1 + u omega]] for each t
    (KDN reading notes, method part §6, Eq. (32)-(39)).  Returns [T,2,2]."""
    a2 = _f64(alpha) ** 2
    w = _f64(omega)
    u = _f64(u)
    M = np.empty(a2.shape + (2, 2))
    M[..., 0, 0] = a2
    M[..., 0, 1] = w
    M[..., 1, 0] = u * a2
    M[..., 1, 1] = 1.0 + u * w
    return M


def _rescale(M):
    # homogeneous coordinates: dividing by a positive number keeps n/d
    return M / np.max(np.abs(M))


def mobius_fold_left(Ms):
    """Compose M_T ... M_1 by left-multiplication in token order, rescaling
    after every product.  Ms: [T,2,2] with Ms[0] the first token."""
    P = np.eye(2)
    for M in Ms:
        P = _rescale(M @ P)
    return P


def mobius_fold_tree(Ms):
    """Same product as ``mobius_fold_left`` but with a balanced bracketing:
    the left half's product is applied first, i.e. prod = R @ L."""
    n = len(Ms)
    if n == 0:
        return np.eye(2)
    if n == 1:
        return _rescale(np.array(Ms[0], dtype=np.float64))
    mid = n // 2
    L = mobius_fold_tree(Ms[:mid])
    R = mobius_fold_tree(Ms[mid:])
    return _rescale(R @ L)


def mobius_apply(P, x0):
    """p = n / d for [n; d] = P [x0; 1]."""
    n = P[0, 0] * x0 + P[0, 1]
    d = P[1, 0] * x0 + P[1, 1]
    return n / d


# --------------------------------------------------------------------------
# Textbook delta-rule family
# --------------------------------------------------------------------------
def gated_delta_rule(k, v, q, decay, beta, S0):
    """S_t = D_t S_{t-1} + beta_t k_t (v_t - (D_t S_{t-1})^T k_t)^T,
    o_t = S_t^T q_t, with D_t = diag(decay_t) (decay [T,dk]; a scalar per
    token gives Gated DeltaNet, all ones gives DeltaNet).
    KDN reading notes, motivation part §1 (unified form and model table)."""
    k, v, q = _f64(k), _f64(v), _f64(q)
    decay, beta = _f64(decay), _f64(beta)
    S = _f64(S0).copy()
    T = k.shape[0]
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        DS = decay[t][:, None] * S
        S = DS + beta[t] * np.outer(k[t], v[t] - DS.T @ k[t])
        o[t] = S.T @ q[t]
    return {"o": o, "S": S}
