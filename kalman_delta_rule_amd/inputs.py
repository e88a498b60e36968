"""Seeded synthetic inputs for the KDN mixer.

This module holds none of the method's arithmetic: it only draws random
tensors with the shapes and distributions of the mixer workloads, so that the
HIP path and the fp64 oracle consume identical values.  It imports nothing
from the rest of the package.

Recipe (per (b,t,h), numpy PCG64, draws and transforms in fp32):
  q, k ~ N(0, I) then L2-normalised over d_k; v ~ N(0, I);
  alpha = sigmoid(N(2, 0.5)) per key channel (the per-channel decay);
  omega = softplus(N(0, 1)) per key channel (Diagonal) or per head (Isotropic);
  r = softplus(N(0, 1)) per head;  S0 = 0, p0 = b0 = 1.
bf16 workloads round q, k, v to bf16 (round to nearest even) here, so the
values both sides read are bit-identical; alpha, omega, r stay fp32.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED_BASE = 20260


@dataclass(frozen=True)
class Workload:
    name: str
    variant: str          # "diag" | "iso"
    io: str               # "f32" | "bf16"   (dtype of q, k, v and o)
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int = 64
    structure: str = "random"   # "random" | "retrieval" | "decode"
    steps: int = 0              # decode workloads: tokens per sequence
    seed: int = SEED_BASE

    @property
    def tokens(self) -> int:
        return self.B * self.T


# The five mixer workloads.  Shapes: 16 heads of width 128 at hidden size
# 2048 and a 4K context are the shapes of the KDN pre-training runs; the
# throughput figure on the pages uses d_model 2048 and batch 4.
WORKLOADS = {
    0: Workload("diag-f32-B1H2T256-d64", "diag", "f32", 1, 2, 256, 64, 64, 64,
                seed=SEED_BASE + 0),
    1: Workload("iso-bf16-B4H16T2048-d128", "iso", "bf16", 4, 16, 2048, 128, 128,
                seed=SEED_BASE + 1),
    2: Workload("diag-bf16-B8H16T4096-d128", "diag", "bf16", 8, 16, 4096, 128, 128,
                seed=SEED_BASE + 2),
    3: Workload("diag-bf16-B1H16T65536-d128-retrieval", "diag", "bf16", 1, 16, 65536,
                128, 128, structure="retrieval", seed=SEED_BASE + 3),
    4: Workload("decode-bf16-B256H16-d128-1024steps", "both", "bf16", 256, 16, 1, 128,
                128, structure="decode", steps=1024, seed=SEED_BASE + 4),
}


def workload(i: int, **overrides) -> Workload:
    w = WORKLOADS[i]
    return replace(w, **overrides) if overrides else w


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32.
    uint32 arithmetic cannot wrap for finite inputs (only NaN bit patterns
    reach the top of the range)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    out = (bits + (lsb + np.uint32(0x7FFF))) & np.uint32(0xFFFF0000)
    return out.view(np.float32)


def _sigmoid(x):
    x = np.asarray(x, dtype=np.float32)
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-x))).astype(np.float32)


def _softplus(x):
    x = np.asarray(x, dtype=np.float32)
    return (np.maximum(x, np.float32(0.0)) + np.log1p(np.exp(-np.abs(x)))).astype(np.float32)


def _unit(x, axis=-1):
    n = np.sqrt(np.sum(np.square(x, dtype=np.float32), axis=axis, keepdims=True))
    return (x / np.maximum(n, np.float32(1e-30))).astype(np.float32)


def _draw_tokens(rng, variant, B, T, H, dk, dv, io, preact=False):
    """q, k, v and the gates; with ``preact`` the gates' pre-activations
    (alpha's, omega's, r's) in place of the gates, from the same draws."""
    f32 = np.float32
    q = _unit(rng.standard_normal((B, T, H, dk), dtype=f32))
    k = _unit(rng.standard_normal((B, T, H, dk), dtype=f32))
    v = rng.standard_normal((B, T, H, dv), dtype=f32)
    a_pre = f32(2.0) + f32(0.5) * rng.standard_normal((B, T, H, dk), dtype=f32)
    wshape = (B, T, H, dk) if variant == "diag" else (B, T, H)
    w_pre = rng.standard_normal(wshape, dtype=f32)
    r_pre = rng.standard_normal((B, T, H), dtype=f32)
    if preact:
        return q, k, v, a_pre, w_pre, r_pre
    return q, k, v, _sigmoid(a_pre), _softplus(w_pre), _softplus(r_pre)


TOKEN_BLOCK = 1024   # tokens per independently seeded generation block


def make_preact_inputs(w: Workload, variant: Optional[str] = None, threads: int = 0) -> dict:
    """Inputs of the forward from gate pre-activations: q, k, v as in
    make_fwd_inputs and, instead of the gates, a_pre [B,T,H,dk], w_pre
    ([B,T,H,dk] Diagonal, [B,T,H] Isotropic) and r_pre [B,T,H], drawn from the
    same streams (so sigmoid(a_pre) etc. are the gates make_fwd_inputs draws)
    and rounded to bf16 when ``w.io == 'bf16'``."""
    return make_fwd_inputs(w, variant, threads, preact=True)


def make_fwd_inputs(w: Workload, variant: Optional[str] = None, threads: int = 0,
                    preact: bool = False) -> dict:
    """Forward inputs for workload ``w`` as fp32 numpy arrays (q, k, v already
    rounded to bf16 when ``w.io == 'bf16'``) plus S0 / p0 (or b0).

    Each (batch row, block of TOKEN_BLOCK tokens) draws from its own PCG64
    stream seeded by (seed, variant, b, block), so the result does not depend
    on how many threads generate it."""
    variant = variant or w.variant
    assert variant in ("diag", "iso")
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    f32 = np.float32
    q = np.empty((B, T, H, dk), f32)
    k = np.empty((B, T, H, dk), f32)
    v = np.empty((B, T, H, dv), f32)
    alpha = np.empty((B, T, H, dk), f32)
    omega = np.empty((B, T, H, dk) if variant == "diag" else (B, T, H), f32)
    r = np.empty((B, T, H), f32)
    vcode = 0 if variant == "diag" else 1
    blocks = [(b, t0) for b in range(B) for t0 in range(0, T, TOKEN_BLOCK)]

    def fill(job):
        b, t0 = job
        t1 = min(T, t0 + TOKEN_BLOCK)
        rng = np.random.Generator(np.random.PCG64([w.seed, vcode, b, t0 // TOKEN_BLOCK]))
        parts = _draw_tokens(rng, variant, 1, t1 - t0, H, dk, dv, w.io, preact)
        for dst, src in zip((q, k, v, alpha, omega, r), parts):
            dst[b:b + 1, t0:t1] = src

    if threads <= 0:
        threads = min(16, os.cpu_count() or 1)
    if threads > 1 and len(blocks) > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, blocks))
    else:
        for job in blocks:
            fill(job)
    if w.structure == "retrieval":
        rng = np.random.Generator(np.random.PCG64([w.seed, vcode, 1 << 20]))
        _insert_retrieval(rng, q, k, v, n_pairs=min(512, T // 2))
    if w.io == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    if preact:
        if w.io == "bf16":
            alpha, omega, r = round_bf16(alpha), round_bf16(omega), round_bf16(r)
        return {"q": q, "k": k, "v": v, "a_pre": alpha, "w_pre": omega, "r_pre": r}
    out = {"q": q, "k": k, "v": v, "alpha": alpha, "omega": omega, "r": r,
           "S0": np.zeros((B, H, dk, dv), np.float32)}
    if variant == "diag":
        out["p0"] = np.ones((B, H, dk), np.float32)
    else:
        out["b0"] = np.ones((B, H), np.float32)
    return out


def _insert_retrieval(rng, q, k, v, n_pairs):
    """Key-value retrieval structure: per (b,h), ``n_pairs`` unit keys with
    N(0,1) values are written at distinct positions drawn uniformly from
    [0, T - n_pairs); the last ``n_pairs`` tokens query those keys in a random
    order.  Everything else keeps the filler distribution."""
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    for b in range(B):
        for h in range(H):
            keys = _unit(rng.standard_normal((n_pairs, dk), dtype=np.float32))
            vals = rng.standard_normal((n_pairs, dv), dtype=np.float32)
            pos = rng.choice(T - n_pairs, size=n_pairs, replace=False)
            k[b, pos, h] = keys
            v[b, pos, h] = vals
            perm = rng.permutation(n_pairs)
            q[b, T - n_pairs:, h] = keys[perm]


def make_decode_state(w: Workload, variant: str) -> dict:
    """Seeded random decode state: S0 ~ N(0,1) iid, p0 (or b0) ~ U[0.1, 1]."""
    rng = np.random.Generator(np.random.PCG64([w.seed, 0 if variant == "diag" else 1]))
    S0 = rng.standard_normal((w.B, w.H, w.dk, w.dv), dtype=np.float32)
    if variant == "diag":
        var0 = rng.uniform(0.1, 1.0, (w.B, w.H, w.dk)).astype(np.float32)
    else:
        var0 = rng.uniform(0.1, 1.0, (w.B, w.H)).astype(np.float32)
    return {"S0": S0, "var0": var0}


def make_decode_step(w: Workload, variant: str, step: int) -> dict:
    """Inputs of one decode step (one token per sequence), [B,H,D], drawn
    from a per-step seed so any step can be regenerated on its own."""
    rng = np.random.Generator(np.random.PCG64([w.seed, 2 if variant == "diag" else 3, step]))
    q, k, v, alpha, omega, r = _draw_tokens(rng, variant, w.B, 1, w.H, w.dk, w.dv, w.io)
    sq = lambda x: np.ascontiguousarray(x[:, 0])
    q, k, v, alpha, omega, r = map(sq, (q, k, v, alpha, omega, r))
    if w.io == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return {"q": q, "k": k, "v": v, "alpha": alpha, "omega": omega, "r": r}
