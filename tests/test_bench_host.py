"""Host-side logic of bench.py (no GPU): the one-GPU contract, the
algorithmic byte counts the roofline is priced with, and the rule that
counter-measured traffic is reported only for the sources it was taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and "--gpus 2" in res.stderr
    assert res.stdout.strip() == ""


@pytest.mark.parametrize("variant,per_ht", [("diag", 2052), ("iso", 1544)])
def test_bytes_per_head_token(variant, per_ht):
    # per head-token at d = 128, bf16 io: q, k, v read and o written (2 B
    # each), fp32 gates (alpha, and omega per channel for Diagonal or per
    # token for Isotropic) and r
    B, T, H, d = 1, 1000, 1, 128
    state = (d * d * 4 + d * 4) if variant == "diag" else (d * d * 4 + 4)
    assert bench.alg_bytes_fwd(variant, B, T, H, d, d, 2) == T * per_ht + state


def test_bytes_config2_forward():
    # B = 8, H = 16, T = 4096, d = 128: 524,288 head-tokens at 2052 B plus the
    # final state and variances of 128 heads
    assert bench.alg_bytes_fwd("diag", 8, 4096, 16, 128, 128, 2) == 1_084_293_120


def test_bytes_decode_step():
    # per head: state read and written (2 d^2 4 B), q, k, v, o, alpha, omega,
    # r and the variances read and written
    d = 128
    per_head = 2 * d * d * 4 + 3 * d * 2 + d * 2 + 2 * d * 4 + 4 + 2 * d * 4
    assert bench.alg_bytes_step("diag", 256, 16, d, d, 2) == 256 * 16 * per_head


def test_forward_kernel_by_io_dtype():
    assert bench.fwd_kernel_name("bf16") == "kdn_walk_fwd_kernel"
    assert bench.fwd_kernel_name("f32") == "kdn_chunk_fwd_kernel"


def test_traffic_only_for_the_profiled_sources(tmp_path, monkeypatch):
    kern = "kdn_walk_fwd_kernel"
    key = bench.traffic_key(kern, "w", "diag")
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    f.write_text(json.dumps({key: {"source_hash": bench.kernel_source_hash(kern),
                                   "bytes_per_launch": 123.0}}))
    assert bench.traffic_for(kern, key) == 123.0
    f.write_text(json.dumps({key: {"source_hash": "0" * 16, "bytes_per_launch": 123.0}}))
    assert bench.traffic_for(kern, key) is None
    assert bench.traffic_for(kern, bench.traffic_key(kern, "other", "diag")) is None
    f.write_text("not json")
    assert bench.traffic_for(kern, key) is None


def test_bytes_backward_per_head_token():
    # Diagonal, d = 128, bf16: q, k, v, do read and dq, dk, dv written (2 B
    # each), alpha, omega read and their gradients written (fp32), r and dr;
    # per head dS0 (d^2 fp32), dp0 (d fp32) and dmu
    d = 128
    per_ht = 7 * d * 2 + 4 * d * 4 + 8
    assert per_ht == 3848
    assert bench.alg_bytes_bwd("diag", 1, 10, 1, d, d, 2) == 10 * per_ht + d * d * 4 + d * 4 + 4
    # Isotropic: omega and domega are one fp32 per token
    per_ht_iso = 7 * d * 2 + 2 * (d + 1) * 4 + 8
    assert bench.alg_bytes_bwd("iso", 1, 10, 1, d, d, 2) == 10 * per_ht_iso + d * d * 4 + 4 + 4


def test_bytes_preact_per_head_token():
    # Diagonal, d = 128, bf16: q, k, v, o and the three pre-activations
    # (a and w per channel, rho per token) at 2 B -- the ~1540 B/head-token
    # the fused prologue is priced at
    d = 128
    assert bench.alg_bytes_preact("diag", 1, 10, 1, d, d, 2) == 10 * 1538 + d * d * 4 + d * 4
    # Isotropic: q, k, v, o, a per channel, w and rho per token: (5 d + 2) x 2 B
    assert bench.alg_bytes_preact("iso", 1, 10, 1, d, d, 2) == 10 * 1284 + d * d * 4 + 4


def test_mfma_flops_per_head_token():
    # d = 128, 16-token chunks: 6 d^2 for the three state contractions and
    # 4 C (dk + dv) for L', Aqk, T (V - Kb S) and Aqk D'; the split-product
    # path does each three times
    assert bench.mfma_flops_fwd(1, 1, 1, 128, 128, False) == 6 * 128 * 128 + 4 * 16 * 256
    assert bench.mfma_flops_fwd(8, 4096, 16, 128, 128, True) == 3 * 524288 * 114688


def test_input_sets_rotate_cache_sized_workloads():
    # the Isotropic B4 H16 T2048 forward (207 MB) fits the 256 MB cache: four
    # sets; the B8 H16 T4096 Diagonal one (1.08 GB) does not: one
    assert bench.input_sets(bench.alg_bytes_fwd("iso", 4, 2048, 16, 128, 128, 2)) == 4
    assert bench.input_sets(bench.alg_bytes_fwd("diag", 8, 4096, 16, 128, 128, 2)) == 1


def test_traffic_key_names_the_contraction_mode():
    assert bench.traffic_key("k", "w", "diag", "split") == "k:w:diag:split"
    assert bench.traffic_key("k", "w", "diag") == "k:w:diag"
