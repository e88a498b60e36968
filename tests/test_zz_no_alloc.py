"""The allocation-free gain scan (kdn_gain_scan_static) against the gain scan
with a caller workspace (kdn_gain_scan), both called through the C ABI: same
kernels, so the outputs must agree bit for bit; two calls in a row on one
GPU (the second on a smaller input, which reuses the first call's scratch),
both variants, bf16 and fp32 keys.  Also: a shape beyond the static scratch
is rejected before any launch, and the calls leave the device's free memory
unchanged (no allocation behind the caller's back)."""
import ctypes

import numpy as np
import pytest
import torch

from kalman_delta_rule_amd import _lib, inputs
from kdn_testutil import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a HIP GPU")
    torch.cuda.init()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _call(static: bool, variant: str, d, var0=None, want_kappa=True):
    L = _lib.lib()
    var = 0 if variant == "diag" else 1
    B, T, H, dk = d["k"].shape
    io = 1 if d["k"].dtype == torch.bfloat16 else 0
    vshape = (B, H, dk) if variant == "diag" else (B, H)
    kappa = torch.full((B, T, H, dk), float("nan"), device="cuda") if want_kappa else None
    var_T = torch.full(vshape, float("nan"), device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    args = [var, B, T, H, dk, io, float(dk), _ptr(d["k"]), _ptr(d["alpha"]), _ptr(d["omega"]),
            _ptr(d["r"]), _ptr(var0), _ptr(kappa), _ptr(var_T)]
    if static:
        st = L.kdn_gain_scan_static(*args, stream)
    else:
        need = L.kdn_gain_workspace_size(var, B, T, H, dk)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        st = L.kdn_gain_scan(*args, _ptr(ws), ws.numel(), stream)
    assert st == 0, L.kdn_last_error_message().decode()
    torch.cuda.synchronize()
    return kappa, var_T


def _inputs(variant, io, B, T, H, dk, seed):
    w = inputs.Workload("t", variant, io, B, H, T, dk, dk, seed=seed)
    return to_dev(inputs.make_fwd_inputs(w, variant), io)


@pytest.mark.parametrize("variant", ["diag", "iso"])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_static_matches_workspace_twice(variant, io):
    big = _inputs(variant, io, 2, 1000, 8, 128, seed=31)   # 16 chunks of 64
    small = _inputs(variant, io, 1, 70, 3, 128, seed=32)   # 2 chunks, ragged
    rng = np.random.default_rng(33)
    v0 = torch.from_numpy(rng.uniform(0.2, 2.0, (1, 3, 128) if variant == "diag"
                                      else (1, 3)).astype(np.float32)).cuda()
    for d, var0 in ((big, None), (small, v0)):
        k_ref, p_ref = _call(False, variant, d, var0)
        k_st, p_st = _call(True, variant, d, var0)
        assert torch.equal(k_ref, k_st) and torch.equal(p_ref, p_st)
        assert torch.isfinite(k_st).all() and torch.isfinite(p_st).all()


def test_static_without_kappa_and_empty_sequence():
    d = _inputs("diag", "bf16", 1, 300, 4, 64, seed=41)
    _, p_ref = _call(False, "diag", d, want_kappa=False)
    _, p_st = _call(True, "diag", d, want_kappa=False)
    assert torch.equal(p_ref, p_st)
    e = _inputs("diag", "bf16", 1, 0, 2, 64, seed=42)
    _, p0 = _call(True, "diag", e, want_kappa=False)
    assert torch.equal(p0, torch.ones_like(p0))


def test_static_rejects_a_shape_beyond_its_scratch():
    L = _lib.lib()
    cap = L.kdn_gain_scan_static_max_bytes()
    assert cap == 32 << 20
    # B1 H16 T65536 dk128: 16 * 1024 chunks * 128 * 5 floats = 42 MB > 32 MiB
    assert L.kdn_gain_workspace_size(0, 1, 65536, 16, 128) > cap
    big = _inputs("diag", "bf16", 1, 65536, 16, 128, seed=43)
    var_T = torch.zeros((1, 16, 128), device="cuda")
    st = L.kdn_gain_scan_static(0, 1, 65536, 16, 128, 1, 128.0, _ptr(big["k"]),
                                _ptr(big["alpha"]), _ptr(big["omega"]), _ptr(big["r"]), None,
                                None, _ptr(var_T), torch.cuda.current_stream().cuda_stream)
    assert st == -3
    assert "static scratch" in L.kdn_last_error_message().decode()
    torch.cuda.synchronize()
    assert torch.equal(var_T, torch.zeros_like(var_T))  # nothing ran


def test_static_calls_allocate_nothing():
    d = _inputs("diag", "bf16", 2, 1000, 8, 128, seed=51)
    kappa = torch.empty((2, 1000, 8, 128), device="cuda")
    var_T = torch.empty((2, 8, 128), device="cuda")
    L = _lib.lib()
    stream = torch.cuda.current_stream().cuda_stream
    args = [0, 2, 1000, 8, 128, 1, 128.0, _ptr(d["k"]), _ptr(d["alpha"]), _ptr(d["omega"]),
            _ptr(d["r"]), None, _ptr(kappa), _ptr(var_T), stream]
    assert L.kdn_gain_scan_static(*args) == 0   # first call on the device: address lookup
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(5):
        assert L.kdn_gain_scan_static(*args) == 0
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0
