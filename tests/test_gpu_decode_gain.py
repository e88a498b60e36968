"""GPU parity of the decode step (kdn_step) and of the standalone gain scan
(kdn_gain_scan) against the fp64 oracle."""
import numpy as np
import pytest
import torch

from kalman_delta_rule_amd import api, inputs
from kdn_testutil import TOL, host, per_head_rel, rel_l2, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a HIP GPU")
    torch.cuda.init()


def _decode_run(ora, w, variant, steps, heads):
    """Run `steps` decode steps on the GPU from the seeded state; run the
    oracle on the sampled heads over the same tokens.  Returns errors."""
    st = inputs.make_decode_state(w, variant)
    S = torch.from_numpy(st["S0"]).cuda()
    var = torch.from_numpy(st["var0"]).cuda()
    hb = torch.tensor([b for b, _ in heads], device="cuda")
    hh = torch.tensor([h for _, h in heads], device="cuda")
    o_hist = []
    seq = {n: [] for n in ("q", "k", "v", "alpha", "omega", "r")}
    for s in range(steps):
        x = inputs.make_decode_step(w, variant, s)
        for n in seq:
            seq[n].append(np.stack([x[n][b, h] for b, h in heads]))
        d = to_dev(x, w.io)
        o = api.kdn_step(variant, d["q"], d["k"], d["v"], d["alpha"], d["omega"], d["r"], S, var)
        o_hist.append(o[hb, hh])
    torch.cuda.synchronize()
    o_gpu = host(torch.stack(o_hist, dim=1))            # [n, steps, dv]
    # oracle: the sampled heads as a batch of independent sequences
    tok = {n: np.stack(seq[n], axis=1)[:, :, None] for n in seq}   # [n, steps, 1, ...]
    S0 = np.stack([st["S0"][b, h] for b, h in heads])[:, None]
    v0 = np.stack([st["var0"][b, h] for b, h in heads])[:, None]
    if variant == "diag":
        ref = ora.diag_fwd(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["omega"], tok["r"],
                           S0=S0, p0=v0)
        vref = ref["p"][:, 0]
    else:
        ref = ora.iso_fwd(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["omega"], tok["r"],
                          S0=S0, b0=v0)
        vref = ref["b"][:, 0]
    Sg, vg = host(S), host(var)
    return {
        "o": rel_l2(o_gpu, ref["o"][:, :, 0]),
        "S": rel_l2(np.stack([Sg[b, h] for b, h in heads]), ref["S"][:, 0]),
        "var": rel_l2(np.stack([vg[b, h] for b, h in heads]), vref),
    }


@pytest.mark.parametrize("variant", ["diag", "iso"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (128, 64), (64, 128)],
                         ids=lambda d: "dk%ddv%d" % d)
def test_decode_small(ora, variant, io, dims):
    dk, dv = dims
    w = inputs.Workload("t", variant, io, 3, 2, 1, dk, dv, structure="decode", steps=40,
                        seed=500 + dk + dv)
    heads = [(b, h) for b in range(3) for h in range(2)]
    err = _decode_run(ora, w, variant, 40, heads)
    print(variant, io, dims, err, flush=True)
    assert max(err.values()) <= TOL[io], err


def _decode_whole(ora, w, variant, group=16):
    """All ``w.steps`` decode steps on every (sequence, head) of the workload,
    in the launch configuration the benchmark times; then the oracle on the
    same tokens, ``group`` sequences at a time (each sequence is independent),
    with the relative-L2 sums of o (every step), S and the variances
    accumulated over the whole tensors.  Returns (errors, worst (b, h))."""
    B, H, dv, steps = w.B, w.H, w.dv, w.steps
    st = inputs.make_decode_state(w, variant)
    S = torch.from_numpy(st["S0"]).cuda()
    var = torch.from_numpy(st["var0"]).cuda()
    o_all = torch.empty((steps, B, H, dv), dtype=torch.bfloat16 if w.io == "bf16"
                        else torch.float32, device="cuda")
    xs = []
    for s in range(steps):
        x = inputs.make_decode_step(w, variant, s)
        xs.append(x)
        d = to_dev(x, w.io)
        api.kdn_step(variant, d["q"], d["k"], d["v"], d["alpha"], d["omega"], d["r"], S, var,
                     o=o_all[s])
    torch.cuda.synchronize()
    Sg, vg = host(S), host(var)
    acc = {n: [0.0, 0.0] for n in ("o", "S", "var")}
    worst = {n: 0.0 for n in acc}
    names = ("q", "k", "v", "alpha", "omega", "r")
    for b0 in range(0, B, group):
        b1 = min(B, b0 + group)
        tok = {n: np.stack([x[n][b0:b1] for x in xs], axis=1) for n in names}  # [g, steps, H, ...]
        if variant == "diag":
            ref = ora.diag_fwd(*(tok[n] for n in names), S0=st["S0"][b0:b1], p0=st["var0"][b0:b1])
            vref = ref["p"]
        else:
            ref = ora.iso_fwd(*(tok[n] for n in names), S0=st["S0"][b0:b1], b0=st["var0"][b0:b1])
            vref = ref["b"]
        og = host(o_all[:, b0:b1]).transpose(1, 0, 2, 3)                      # [g, steps, H, dv]
        for n, x, r, axes in (("o", og, ref["o"], (0, 2)), ("S", Sg[b0:b1], ref["S"], (0, 1)),
                              ("var", vg[b0:b1], vref, (0, 1))):
            acc[n][0] += float(np.sum(np.square(x - r)))
            acc[n][1] += float(np.sum(np.square(r)))
            worst[n] = max(worst[n], float(per_head_rel(x, r, axes).max()))
    err = {n: float(np.sqrt(a[0] / a[1])) for n, a in acc.items()}
    return err, worst


@pytest.mark.timeout(600)
@pytest.mark.parametrize("variant", ["diag", "iso"])
def test_config4_decode_full(ora, variant):
    w = inputs.workload(4)
    err, worst = _decode_whole(ora, w, variant)
    print("%s %s whole-tensor rel-L2 %s; worst (b,h) %s" % (w.name, variant, err, worst),
          flush=True)
    assert max(err.values()) <= TOL[w.io], err
    assert max(worst.values()) <= TOL[w.io], worst


def _gain_compare(ora, variant, w, heads=None):
    inp = inputs.make_fwd_inputs(w, variant)
    d = to_dev(inp, w.io)
    kappa, var_T = api.kdn_gain_scan(variant, d["k"], d["alpha"], d["omega"], d["r"])
    torch.cuda.synchronize()
    B, T, H, dk = inp["k"].shape
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    stack = lambda x: np.ascontiguousarray(np.stack([x[b, :, h] for (b, h) in heads])[:, :, None])
    args = [stack(inp[n]) for n in ("q", "k", "v", "alpha", "omega", "r")]
    kg = host(kappa)
    kg = np.stack([kg[b, :, h] for (b, h) in heads])
    vg = host(var_T)
    vg = np.stack([vg[b, h] for (b, h) in heads])
    if variant == "diag":
        ref = ora.diag_fwd(*args, return_gain=True)
        kref, vref = ref["kappa"][:, :, 0], ref["p"][:, 0]
    else:
        ref = ora.iso_fwd(*args, return_gain=True)
        kref = ref["beta"][:, :, 0, None] * args[1][:, :, 0]
        vref = ref["b"][:, 0]
    return {"kappa": rel_l2(kg, kref), "var": rel_l2(vg, vref)}


@pytest.mark.parametrize("variant", ["diag", "iso"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 256, 2, 64), (2, 333, 3, 128), (1, 4100, 1, 128)],
                         ids=lambda s: "B%dT%dH%ddk%d" % s)
def test_gain_scan(ora, variant, io, shape):
    B, T, H, dk = shape
    w = inputs.Workload("t", variant, io, B, H, T, dk, dk, seed=900 + T)
    err = _gain_compare(ora, variant, w)
    print(variant, io, shape, err, flush=True)
    # the gain path is fp32 arithmetic on both io dtypes
    assert err["kappa"] <= 1e-4 and err["var"] <= 1e-4, err


@pytest.mark.timeout(400)
def test_gain_scan_config2_shape(ora):
    w = inputs.workload(2)
    err = _gain_compare(ora, "diag", w)
    print(w.name, err, flush=True)
    assert err["kappa"] <= 1e-4 and err["var"] <= 1e-4, err
