"""Benchmark of the KDN mixer forward on one MI355X.

Default workload: Diagonal KDN forward, bf16 q/k/v with fp32 gates and state,
B=8, H=16, T=4096, d_k=d_v=128 (the mixer of a hidden-2048 / 16-head layer
at a 4K context), synthetic seeded inputs resident in HBM before timing.
One step = one forward call over the whole batch (gain scan, chunked memory
update, readout, final state).  Prints ONE JSON line.  The Diagonal forward
runs its chunk contractions as split-bf16 products (three bf16 products of
hi / lo operand halves, fp32 accumulation), the higher-precision Diagonal the
KDN reading notes' throughput figure used; --math bf16 times the
single-product contractions instead.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--math split|bf16]

Other modes (same JSON form, not the default): --workload 1 / 3 / 4 (the
Isotropic, long-sequence and decode workloads), --preact (the forward from
bf16 gate pre-activations, kdn_fwd_preact), --bwd (the backward pass,
kdn_bwd, priced against its own algorithmic bytes) and --gain (the gain scan
alone, kdn_gain_scan with kappa).

Roofline: achieved = algorithmic bytes per launch / mean launch time (HIP
events on the launch stream, one pair per launch: the median launch is
reported beside the mean).  Algorithmic bytes read every input once and
write every output once (per head-token: 3 d s_io + 2 d * 4 + 4 + d s_io for
Diagonal; plus the final state and variances per head).  `traffic` (HBM bytes
per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a plain-copy
calibration) is read from profiles/ and reported only while the kernel
sources still hash to what was profiled.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_FLOPS = 2.5e15  # MI355X dense bf16 matrix peak, published
LLC_BYTES = 256 * 2**20         # MI355X last-level (Infinity) cache
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
# sources each measured kernel is built from (traffic figures go stale when they change)
KERNEL_SOURCES = {
    "kdn_walk_fwd_kernel": ["kdn_walk.hip", "kdn_common.h", "kdn_internal.h"],
    "kdn_chunk_fwd_kernel": ["kdn_chunk.hip", "kdn_common.h", "kdn_internal.h"],
    "kdn_step_kernel": ["kdn_step.hip", "kdn_common.h", "kdn_internal.h"],
    "kdn_gain_scan": ["kdn_gain.hip", "kdn_common.h", "kdn_ops.h"],
}


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for s in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "kalman_delta_rule_amd", "csrc", s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def alg_bytes_fwd(variant: str, B, T, H, dk, dv, s_io: int) -> int:
    n_ht = B * T * H
    if variant == "diag":
        per_ht = 2 * dk * s_io + dv * s_io + 2 * dk * 4 + 4 + dv * s_io
        state = B * H * (dk * dv * 4 + dk * 4)
    else:
        per_ht = 2 * dk * s_io + dv * s_io + dk * 4 + 4 + 4 + dv * s_io
        state = B * H * (dk * dv * 4 + 4)
    return n_ht * per_ht + state


def alg_bytes_preact(variant: str, B, T, H, dk, dv, s_io: int) -> int:
    """The forward's algorithmic bytes with the fp32 gates replaced by their
    pre-activations in the io dtype: q, k, v read, o written, a_pre and
    w_pre (per channel for Diagonal, per token for Isotropic) and r_pre read,
    plus the final state and variances."""
    n_ht = B * T * H
    w = dk if variant == "diag" else 1
    per_ht = (2 * dk + dv) * s_io + dv * s_io + (dk + w + 1) * s_io
    state = B * H * (dk * dv * 4 + w * 4)
    return n_ht * per_ht + state


def alg_bytes_step(variant: str, B, H, dk, dv, s_io: int) -> int:
    per_head = 2 * dk * s_io + dv * s_io + dk * 4 + 4 + dv * s_io + 2 * dk * dv * 4
    per_head += (2 * dk * 4 + dk * 4) if variant == "diag" else (4 + 2 * 4)
    return B * H * per_head


def alg_bytes_bwd(variant: str, B, T, H, dk, dv, s_io: int) -> int:
    """Algorithmic HBM bytes of one backward call: q, k, v and do read and dq,
    dk, dv written in the io dtype; alpha, omega, r read and their gradients
    written in fp32 (omega per channel for Diagonal, per token for Isotropic);
    per head the initial-state, initial-variance and information-scale
    gradients written.  The forward's recomputation and the workspace are the
    implementation's, not the algorithm's."""
    w = dk if variant == "diag" else 1
    per_ht = (4 * dk + 3 * dv) * s_io + 2 * (dk + w) * 4 + 2 * 4
    per_head = dk * dv * 4 + w * 4 + 4
    return B * T * H * per_ht + B * H * per_head


def fwd_kernel_name(io: str) -> str:
    """The kernel one forward call launches: bf16 io runs the walk kernel,
    fp32 io the fp32 chunk kernel."""
    return "kdn_walk_fwd_kernel" if io == "bf16" else "kdn_chunk_fwd_kernel"


def traffic_key(kernel: str, workload: str, variant: str, mode: str = "") -> str:
    return "%s:%s:%s" % (kernel, workload, variant) + (":" + mode if mode else "")


def traffic_for(kernel: str, key: str):
    """HBM bytes per launch measured by counters, if still valid."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(key)
    if not ent or ent.get("source_hash") != kernel_source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


def copy_calibration(dev):
    """Three plain 1 GiB device-to-device copies: a kernel of known traffic
    (1 GiB read, 1 GiB written) that scales the HBM traffic counters."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("[bench] copy calibration: 3 x 1 GiB device copies done", file=sys.stderr, flush=True)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, variant):
    """The fp64 oracle, untuned, on the same seeded inputs the GPU consumed,
    timed on the host: all cores (OpenMP over the independent (batch, head)
    problems) on the whole workload when it finishes in about half a minute
    of CPU time, else on the leading batch rows that fit, and one thread on
    one batch row.  Reported in the GPU's unit (tokens/s)."""
    import numpy as np
    import oracle

    nproc = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = max(1, min(oracle.max_threads(), w.B * w.H))
    fn = oracle.diag_fwd if variant == "diag" else oracle.iso_fwd
    names = ("q", "k", "v", "alpha", "omega", "r")
    # probe one row to size the sample
    rows, done_rows, dt_total = 1, 0, 0.0
    while done_rows < w.B:
        n = min(rows, w.B - done_rows)
        sl = {k: np.ascontiguousarray(inp[k][done_rows:done_rows + n]) for k in names}
        t0 = time.perf_counter()
        fn(*(sl[k] for k in names), nthreads=threads)
        dt = time.perf_counter() - t0
        done_rows += n
        dt_total += dt
        if dt_total * threads > 20.0:
            break
        rows = max(1, int(n * 2))
    tokens = done_rows * w.T
    # one thread on one batch row (H heads x T tokens)
    sl = {k: np.ascontiguousarray(inp[k][:1]) for k in names}
    t0 = time.perf_counter()
    fn(*(sl[k] for k in names), nthreads=1)
    dt1 = time.perf_counter() - t0
    return {"value": tokens / dt_total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d batch rows of the workload (%d heads x %d tokens each), fp64 C "
                      "token recurrence with OpenMP over heads, %.2f s wall"
                      % (done_rows, w.B, w.H, w.T, dt_total),
            "nproc": nproc, "cpu_model": _cpu_model(),
            "single_thread": {"value": w.T / dt1, "unit": "tokens/s",
                              "sample": "1 batch row (%d heads x %d tokens), 1 thread, %.2f s wall"
                                        % (w.H, w.T, dt1)}}


def time_launches(launch, stream, steps, warmup):
    """W untimed launches, then exactly K timed ones with an event pair
    around each (recorded on the launch stream) and around all of them;
    synchronised on both sides.  Returns (total ms, per-launch ms, wall s)."""
    import torch
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(steps):
        launch()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[-1]), per, wall


def input_sets(alg_bytes: int) -> int:
    """Input sets a forward is timed over: one when its bytes exceed the
    last-level cache, else enough (at most 4) that the sets together span
    three times the cache."""
    if alg_bytes >= LLC_BYTES:
        return 1
    return int(min(4, -(-3 * LLC_BYTES // alg_bytes)))


def mfma_flops_fwd(B, T, H, dk, dv, split: bool) -> int:
    """bf16 matrix-core flops of one forward as the walk kernel contracts it
    (16-token chunks): per head-token 2 dk dv for each of Kb S, Qb S and the
    state update, 2 C dk for L' and Aqk, 2 C dv for T (V - Kb S) and Aqk D';
    the split-product path does each three times."""
    C = 16
    per_ht = 6 * dk * dv + 4 * C * (dk + dv)
    return B * T * H * per_ht * (3 if split else 1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the defaults run long enough (about 0.1 s of launches) for the GPU clocks
    # to settle before the timed region
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--variant", default=None, help="override: diag | iso")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--preact", action="store_true",
                    help="time the forward from gate pre-activations (kdn_fwd_preact) instead")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward pass (kdn_bwd) on the workload instead")
    ap.add_argument("--bwd-serial", action="store_true",
                    help="with --bwd: a workspace one byte short of kdn_bwd_workspace_size, so "
                         "that shapes the backward splits over the sequence run without the split")
    ap.add_argument("--gain", action="store_true",
                    help="time the gain scan alone (kdn_gain_scan, with kappa) on the workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--math", choices=("split", "bf16"), default="split",
                    help="Diagonal bf16 contractions: split-bf16 products (default) or single "
                         "bf16 products")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the KDN mixer runs on a single MI355X "
              "(heads and batch rows would shard across GPUs with no communication); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from kalman_delta_rule_amd import api, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a HIP GPU", file=sys.stderr)
        sys.exit(1)
    from kalman_delta_rule_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()

    dev = torch.device("cuda:0")
    w = inputs.workload(args.workload)
    if w.structure == "decode":
        return bench_decode(args, w)
    variant = args.variant or w.variant
    if args.preact:
        return bench_preact(args, w, variant)
    io_dt = torch.bfloat16 if w.io == "bf16" else torch.float32
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    s_io = 2 if w.io == "bf16" else 4
    alg = alg_bytes_fwd(variant, B, T, H, dk, dv, s_io)
    # a workload whose inputs would stay in the 256 MB last-level cache is timed
    # over several input sets in turn (each its own seed), so every launch
    # reads its inputs from HBM
    nsets = 1 if (args.bwd or args.gain) else input_sets(alg)

    def upload(inp):
        d = {}
        for n in ("q", "k", "v", "alpha", "omega", "r"):
            t = torch.from_numpy(inp[n])
            d[n] = (t.to(io_dt) if n in ("q", "k", "v") else t).to(dev)
        return d

    print("[bench] generating %s (%s), %d input set(s)" % (w.name, variant, nsets),
          file=sys.stderr, flush=True)
    inp = inputs.make_fwd_inputs(w, variant)
    sets = [upload(inp)]
    for i in range(1, nsets):
        sets.append(upload(inputs.make_fwd_inputs(inputs.workload(args.workload,
                                                                  seed=w.seed + 1000 * i),
                                                  variant)))
    if args.bwd:
        return bench_bwd(args, w, variant, sets[0], io_dt)
    if args.gain:
        return bench_gain(args, w, variant, sets[0])
    split = variant == "diag" and w.io == "bf16" and args.math == "split"
    math = None if (split or w.io != "bf16") else "bf16"
    # arguments checked and marshalled once; each step is one library call
    launchers = [api.fwd_launcher(variant, d["q"], d["k"], d["v"], d["alpha"], d["omega"],
                                  d["r"], math=math)[1] for d in sets]
    turn = [0]

    def step():
        launchers[turn[0] % nsets]()
        turn[0] += 1

    stream = torch.cuda.current_stream(dev)
    print("[bench] warmup %d, %d timed steps" % (args.warmup, args.steps), file=sys.stderr,
          flush=True)
    ms_total, per, wall = time_launches(step, stream, args.steps, args.warmup)
    ms_step = ms_total / args.steps
    ms_med = sorted(per)[len(per) // 2]
    tokens = B * T
    value = tokens * args.steps / (ms_total / 1e3)
    achieved = alg / (ms_step / 1e3) / 1e9
    kname = fwd_kernel_name(w.io)
    mode = "split" if split else ("bf16" if w.io == "bf16" else "f32")
    traffic = traffic_for(kname, traffic_key(kname, w.name, variant, mode))
    print("[bench] %d steps: %.4f ms/step mean, %.4f median (events), wall %.3f s"
          % (args.steps, ms_step, ms_med, wall), file=sys.stderr, flush=True)

    if args.copy_calibration:
        copy_calibration(dev)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, inp, variant)

    flops = mfma_flops_fwd(B, T, H, dk, dv, split) if w.io == "bf16" else None
    line = {
        "metric": "KDN mixer fwd tokens/sec at T=%d (1 GPU); %% of MFMA/HBM roofline" % T,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_median": ms_med,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"split": "bf16x3", "bf16": "bf16", "f32": "f32"}[mode],
        "data": "synthetic",
        "config": {"workload": w.name, "variant": variant, "B": B, "T": T, "H": H, "dk": dk,
                   "dv": dv, "chunk": 16, "io": w.io, "gates": "f32", "state": "f32",
                   "contractions": {"split": "split-bf16: hi.hi + lo.hi + hi.lo, fp32 accumulate",
                                    "bf16": "bf16 products, fp32 accumulate",
                                    "f32": "fp32 products"}[mode],
                   "global_batch": B, "seq_len": T, "parallelism": "single-gpu",
                   "input_sets": nsets},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "alg_bytes_per_launch": alg, "kernel": kname,
                     "mfma_bf16_flops_per_launch": flops,
                     "mfma_bf16_frac": (flops / (ms_step / 1e3) / MFMA_BF16_PEAK_FLOPS
                                        if flops else None)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_preact(args, w, variant):
    """Forward from bf16 (or fp32) gate pre-activations: kdn_fwd_preact, its
    gate workspace allocated once outside the timed region."""
    import torch
    from kalman_delta_rule_amd import _lib, api, inputs

    dev = torch.device("cuda:0")
    print("[bench] generating %s pre-activations (%s)" % (w.name, variant), file=sys.stderr,
          flush=True)
    inp = inputs.make_preact_inputs(w, variant)
    io_dt = torch.bfloat16 if w.io == "bf16" else torch.float32
    d = {n: torch.from_numpy(inp[n]).to(io_dt).to(dev) for n in inp}
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    var = {"diag": 0, "iso": 1}[variant]
    ws = torch.empty(max(int(_lib.lib().kdn_fwd_preact_workspace_size(var, B, T, H, dk)), 1),
                     dtype=torch.uint8, device=dev)
    o = torch.empty((B, T, H, dv), dtype=io_dt, device=dev)
    S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    var_T = torch.empty((B, H, dk) if variant == "diag" else (B, H), dtype=torch.float32,
                        device=dev)

    mth = "bf16" if (args.math == "bf16" and variant == "diag" and w.io == "bf16") else None

    def step():
        api.kdn_fwd_preact(variant, d["q"], d["k"], d["v"], d["a_pre"], d["w_pre"], d["r_pre"],
                           r_min=0.01, o=o, S_T=S_T, var_T=var_T, workspace=ws, math=mth)

    # for comparison, the same result in two calls: the gates into HBM
    # (kdn_gates_from_preact), then the forward reading them (kdn_fwd_ex)
    L = _lib.lib()
    f32 = torch.float32
    g_al = torch.empty((B, T, H, dk), dtype=f32, device=dev)
    g_om = torch.empty(tuple(d["w_pre"].shape), dtype=f32, device=dev)
    g_r = torch.empty((B, T, H), dtype=f32, device=dev)
    io_code = 1 if w.io == "bf16" else 0

    def step_two_calls():
        st = L.kdn_gates_from_preact(var, B, T, H, dk, io_code, d["a_pre"].data_ptr(),
                                     d["w_pre"].data_ptr(), d["r_pre"].data_ptr(), 0.01,
                                     g_al.data_ptr(), g_om.data_ptr(), g_r.data_ptr(),
                                     torch.cuda.current_stream(dev).cuda_stream)
        _lib.check(st)
        api.kdn_fwd_ex(variant, d["q"], d["k"], d["v"], g_al, g_om, g_r, o=o, S_T=S_T,
                       var_T=var_T, math=mth)

    stream = torch.cuda.current_stream(dev)

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(steps):
            fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps

    ms_two = timed(step_two_calls, max(args.steps // 2, 1), max(args.warmup // 2, 1))
    ms_step = timed(step, args.steps, args.warmup)
    s_io = 2 if w.io == "bf16" else 4
    alg = alg_bytes_preact(variant, B, T, H, dk, dv, s_io)
    achieved = alg / (ms_step / 1e3) / 1e9
    line = {
        "metric": "KDN mixer fwd from gate pre-activations, tokens/sec at T=%d (1 GPU)" % T,
        "value": B * T / (ms_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.io == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "variant": variant, "B": B, "T": T, "H": H, "dk": dk,
                   "dv": dv, "io": w.io, "gates": "pre-activations", "r_min": 0.01,
                   "contractions": ("bf16 products, fp32 accumulate" if mth == "bf16" or
                                    variant == "iso" else "split-bf16 products, fp32 accumulate")
                   if w.io == "bf16" else "fp32"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "alg_bytes_per_launch": alg,
                     "kernel": ("kdn_gate_prologue (r%s) + %s reading a_pre%s" % (
                         ", omega" if variant == "iso" else "", fwd_kernel_name(w.io),
                         "" if variant == "iso" else " and w_pre") if w.io == "bf16" else
                         "kdn_gate_prologue (x3) + %s" % fwd_kernel_name(w.io))},
        "cpu_baseline": None,
        # the same result from kdn_gates_from_preact + kdn_fwd_ex (gates
        # through HBM), timed in the same run
        "two_calls_ms_per_step": ms_two,
    }
    print(json.dumps(line), flush=True)


def alg_bytes_gain(variant: str, B, T, H, dk, s_io: int) -> int:
    """Gain scan with kappa: k, alpha, omega (per channel for Diagonal, per
    head for Isotropic) and r read once, kappa (fp32) written once, plus the
    final variances."""
    om = dk * 4 if variant == "diag" else 4
    per_ht = dk * s_io + dk * 4 + om + 4 + dk * 4
    return B * T * H * per_ht + B * H * (dk if variant == "diag" else 1) * 4


def bench_gain(args, w, variant, d):
    """The gain scan on its own (kdn_gain_scan with kappa), outputs and
    workspace allocated once outside the timed region."""
    import torch
    from kalman_delta_rule_amd import _lib

    L = _lib.lib()
    dev = d["k"].device
    B, T, H, dk = w.B, w.T, w.H, w.dk
    var = {"diag": 0, "iso": 1}[variant]
    io = 1 if w.io == "bf16" else 0
    kappa = torch.empty((B, T, H, dk), dtype=torch.float32, device=dev)
    var_T = torch.empty((B, H, dk) if variant == "diag" else (B, H), dtype=torch.float32,
                        device=dev)
    ws_bytes = int(L.kdn_gain_workspace_size(var, B, T, H, dk))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    h = stream.cuda_stream
    ptrs = [d[n].data_ptr() for n in ("k", "alpha", "omega", "r")]

    def step():
        _lib.check(L.kdn_gain_scan(var, B, T, H, dk, io, float(dk), *ptrs, None,
                                   kappa.data_ptr(), var_T.data_ptr(), ws.data_ptr(), ws.numel(),
                                   h))

    print("[bench] gain scan warmup %d, %d timed steps" % (args.warmup, args.steps),
          file=sys.stderr, flush=True)
    ms_total, per, wall = time_launches(step, stream, args.steps, args.warmup)
    ms_step = ms_total / args.steps
    ms_med = sorted(per)[len(per) // 2]
    if args.copy_calibration:
        copy_calibration(dev)
    s_io = 2 if w.io == "bf16" else 4
    alg = alg_bytes_gain(variant, B, T, H, dk, s_io)
    achieved = alg / (ms_step / 1e3) / 1e9
    line = {
        "metric": "KDN gain scan tokens/sec at T=%d (1 GPU)" % T,
        "value": B * T / (ms_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_median": ms_med,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "variant": variant, "B": B, "T": T, "H": H, "dk": dk,
                   "io": w.io, "pass": "gain scan with kappa"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic_for("kdn_gain_scan",
                                            traffic_key("kdn_gain_scan", w.name, variant)),
                     "alg_bytes_per_launch": alg,
                     "kernel": "gain_summary + gain_carry + gain_replay"},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bench_bwd(args, w, variant, d, io_dt):
    """Backward pass of the forward workload: kdn_bwd with a seeded dL/do and
    no final-state gradient, its workspace allocated once outside the timed
    region."""
    import torch
    from kalman_delta_rule_amd import _lib, api

    dev = d["q"].device
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    gen = torch.Generator(device="cpu").manual_seed(w.seed + 77)
    d_o = torch.randn((B, T, H, dv), generator=gen).to(io_dt).to(dev)
    var = {"diag": 0, "iso": 1}[variant]
    need = int(_lib.lib().kdn_bwd_workspace_size(var, B, T, H, dk, dv))
    ws = torch.empty(max(need - (1 if args.bwd_serial else 0), 1), dtype=torch.uint8, device=dev)

    def step():
        api.kdn_bwd(variant, d["q"], d["k"], d["v"], d["alpha"], d["omega"], d["r"], d_o,
                    workspace=ws)

    print("[bench] backward warmup %d (workspace %.2f GB)" % (args.warmup, ws.numel() / 1e9),
          file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    if args.copy_calibration:
        copy_calibration(dev)
    s_io = 2 if w.io == "bf16" else 4
    alg = alg_bytes_bwd(variant, B, T, H, dk, dv, s_io)
    achieved = alg / (ms_step / 1e3) / 1e9
    line = {
        "metric": "KDN mixer bwd tokens/sec at T=%d (1 GPU)" % T,
        "value": B * T * args.steps / (ms_step * args.steps / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "variant": variant, "B": B, "T": T, "H": H, "dk": dk,
                   "dv": dv, "io": w.io, "pass": "backward",
                   "workspace": "short by one byte" if args.bwd_serial else "full"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "alg_bytes_per_launch": alg,
                     "kernel": "kdn_bwd_gain_fwd + kdn_bwd_mem + kdn_bwd_gain_rev"},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bench_decode(args, w):
    """Decode workload: `w.steps` consecutive kdn_step calls (one token per
    sequence each) from a seeded random state, inputs pre-staged."""
    import torch
    from kalman_delta_rule_amd import api, inputs

    dev = torch.device("cuda:0")
    variant = args.variant or "diag"
    io_dt = torch.bfloat16
    nsteps = w.steps
    print("[bench] staging %d decode steps (%s)" % (nsteps, variant), file=sys.stderr, flush=True)
    st = inputs.make_decode_state(w, variant)
    S = torch.from_numpy(st["S0"]).to(dev)
    var = torch.from_numpy(st["var0"]).to(dev)
    seq = []
    for s in range(nsteps):
        x = inputs.make_decode_step(w, variant, s)
        seq.append({n: (torch.from_numpy(x[n]).to(io_dt) if n in ("q", "k", "v")
                        else torch.from_numpy(x[n])).to(dev) for n in x})
    o = torch.empty((w.B, w.H, w.dv), dtype=io_dt, device=dev)
    for s in range(min(args.warmup, nsteps)):
        x = seq[s]
        api.kdn_step(variant, x["q"], x["k"], x["v"], x["alpha"], x["omega"], x["r"], S, var, o=o)
    torch.cuda.synchronize()
    S.copy_(torch.from_numpy(st["S0"]).to(dev))
    var.copy_(torch.from_numpy(st["var0"]).to(dev))
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for x in seq:
        api.kdn_step(variant, x["q"], x["k"], x["v"], x["alpha"], x["omega"], x["r"], S, var, o=o)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_launch = ms_total / nsteps
    if args.copy_calibration:
        copy_calibration(dev)
    alg = alg_bytes_step(variant, w.B, w.H, w.dk, w.dv, 2)
    achieved = alg / (ms_launch / 1e3) / 1e9
    line = {
        "metric": "KDN decode tokens/sec (1 GPU)",
        "value": w.B * nsteps / (ms_total / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": nsteps,
        "warmup": args.warmup,
        "ms_per_step": ms_launch,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "variant": variant, "B": w.B, "H": w.H, "dk": w.dk,
                   "dv": w.dv, "io": "bf16", "state": "f32"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic_for("kdn_step_kernel",
                                            traffic_key("kdn_step_kernel", w.name, variant)),
                     "alg_bytes_per_launch": alg, "kernel": "kdn_step_kernel"},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
