"""Helpers shared by the GPU tests: uploading seeded inputs, running the
oracle on sampled (batch, head) problems and the relative-L2 metric.

Tolerances (relative L2 over each compared tensor, fp64): 1e-4 when q, k, v
are fp32 and 2e-2 when they are bf16; both sides read bit-identical inputs.
"""
import numpy as np
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    if den == 0.0:
        return float(num)
    return float(num / den)


def to_dev(inp: dict, io: str, device="cuda") -> dict:
    """numpy fp32 arrays -> device tensors (q, k, v in the io dtype)."""
    out = {}
    for name, arr in inp.items():
        t = torch.from_numpy(np.ascontiguousarray(arr))
        if name in ("q", "k", "v") and io == "bf16":
            t = t.to(torch.bfloat16)  # exact: the values are already bf16-rounded
        out[name] = t.to(device)
    return out


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_heads(ora, variant: str, inp: dict, heads, mu=None, S0=None, var0=None):
    """Run the oracle on the (b, h) problems listed in ``heads`` (each one is
    independent; they are stacked as a batch so the oracle's threads share
    them).  Returns {(b, h): dict(o [T,dv], S [dk,dv], var)}."""
    stack = lambda x: np.ascontiguousarray(np.stack([x[b, :, h] for (b, h) in heads])[:, :, None])
    s0 = None if S0 is None else np.stack([S0[b, h] for (b, h) in heads])[:, None]
    v0 = None if var0 is None else np.stack([var0[b, h] for (b, h) in heads])[:, None]
    args = [stack(inp[n]) for n in ("q", "k", "v", "alpha", "omega", "r")]
    if variant == "diag":
        out = ora.diag_fwd(*args, S0=s0, p0=v0, mu=mu)
        var = out["p"][:, 0]
    else:
        out = ora.iso_fwd(*args, S0=s0, b0=v0, mu=mu)
        var = out["b"][:, 0]
    return {x: {"o": out["o"][i, :, 0], "S": out["S"][i, 0], "var": var[i]}
            for i, x in enumerate(heads)}


def compare_heads(res, o, S, var, heads):
    """Relative L2 over the sampled heads for o, S and the variances."""
    o_g = np.concatenate([o[b, :, h].ravel() for (b, h) in heads])
    o_r = np.concatenate([res[(b, h)]["o"].ravel() for (b, h) in heads])
    S_g = np.concatenate([S[b, h].ravel() for (b, h) in heads])
    S_r = np.concatenate([res[(b, h)]["S"].ravel() for (b, h) in heads])
    v_g = np.concatenate([np.ravel(var[b, h]) for (b, h) in heads])
    v_r = np.concatenate([np.ravel(res[(b, h)]["var"]) for (b, h) in heads])
    return {"o": rel_l2(o_g, o_r), "S": rel_l2(S_g, S_r), "var": rel_l2(v_g, v_r)}


def sample_heads(B, H, n, seed):
    rng = np.random.default_rng(seed)
    pairs = [(b, h) for b in range(B) for h in range(H)]
    idx = rng.choice(len(pairs), size=min(n, len(pairs)), replace=False)
    # always include the first and last problem (edges of the grid mapping)
    chosen = {pairs[0], pairs[-1]} | {pairs[i] for i in idx}
    return sorted(chosen)


def per_head_rel(x, ref, head_axes):
    """Relative L2 of every (b, h) problem: x and ref share a layout whose
    batch axis is 0 and whose head axis is ``head_axes[1]``; the other axes
    are summed over.  Returns a [B, H] array."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bax, hax = head_axes
    red = tuple(a for a in range(ref.ndim) if a not in (bax, hax))
    num = np.sqrt(np.sum(np.square(x - ref), axis=red)) if red else np.abs(x - ref)
    den = np.sqrt(np.sum(np.square(ref), axis=red)) if red else np.abs(ref)
    out = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    if hax < bax:
        out = out.T
    return out


def compare_whole(ref, o, S, var, o_head_axes=(0, 2)):
    """Relative L2 over the whole tensors o, S_T and the final variances (the
    metric of the parity bar), plus the worst single (b, h) problem of each
    as a diagnostic.  ``ref`` holds the oracle's o, S and var (or p / b)."""
    vref = ref["var"] if "var" in ref else ref.get("p", ref.get("b"))
    err = {"o": rel_l2(o, ref["o"]), "S": rel_l2(S, ref["S"]), "var": rel_l2(var, vref)}
    worst = {
        "o": float(per_head_rel(o, ref["o"], o_head_axes).max()),
        "S": float(per_head_rel(S, ref["S"], (0, 1)).max()),
        "var": float(per_head_rel(var, vref, (0, 1)).max()),
    }
    return err, worst
