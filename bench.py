"""Benchmark of the chunkwise gated delta rule forward on one MI355X.

One step = one full forward (every kernel of the path) over one batch of the
workload, inputs already resident in HBM.  Prints ONE JSON line on stdout;
diagnostics go to stderr.  The timed region holds only the steps; per-kernel
durations (for the roofline) come from the library's HIP events in a second
run of the same number of steps.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload main-bf16]

Default workload: main-bf16 (B=2, H=16, T=8192, dk=dv=128, chunk 64, scalar
gate, start state N(0, 0.02^2)).  The long workload runs the sequence-parallel
entry point (8 segments) and also reports the single-stream time beside it.
--workload decode-bf16 times gdn_decode_step instead: one token for each of
256 x 16 persistent states, updated in place.  --backward times gdn_backward
(gradients through the recurrence) on the workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/sec + % MFMA/HBM roofline, gated-delta chunk fwd H=16 d=128 T=8K"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w) -> float:
    """HBM bytes the method must move: read q, k, v (input dtype), alpha,
    beta (fp32; alpha is dk wide for the channel gate), write O (fp32);
    per head read the start state (if any) and write the final state."""
    s_in = 2 if w.dtype == "bf16" else 4
    per_ht = (2 * w.dk + w.dv) * s_in + 4 + (4 * w.dk if w.gate == "channel" else 4) + 4 * w.dv
    per_head = 4 * w.dv * w.dk * (2 if w.state0_std > 0 else 1)
    return float(per_ht * w.head_tokens + per_head * w.B * w.H)


def algorithmic_flops(w) -> float:
    """5 C^2 d + 6 C d^2 + C^3 / 3 per chunk-head (d = dk = dv)."""
    C, d = w.chunk, w.dk
    nch = w.B * w.H * ((w.T + C - 1) // C)
    return float(nch * (5 * C * C * d + 6 * C * d * d + C ** 3 / 3))


def kernel_source_hash() -> str:
    """sha256 of the HIP sources: a stored counter measurement is used only
    while the kernels it was taken on are unchanged."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_12_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload_name, kernel):
    """HBM bytes (read + write) of one launch of `kernel` from
    profiles/traffic_<workload>.json (FETCH_SIZE and WRITE_SIZE per dispatch,
    scaled by the plain-copy calibration), or None when absent, taken on
    other kernel sources, or not recorded for that kernel."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    k = rec.get("per_kernel", {}).get(kernel)
    return None if k is None else round(k["read_bytes"] + k["write_bytes"])


def copy_calibration(mbytes: int, reps: int = 5):
    """A plain device copy of known size, for scaling the FETCH_SIZE and
    WRITE_SIZE counters: each rep reads and writes mbytes MiB."""
    import torch
    n = mbytes * (1 << 20) // 4
    src = torch.rand(n, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "reps": reps}), flush=True)


def cpu_baseline(w, inp, max_threads=16, target_s=10.0):
    """Time the oracle on a bounded sample of (batch, head) slices."""
    import numpy as np

    import oracle
    cores = max(1, min(max_threads, len(os.sched_getaffinity(0))))
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    g = oracle.GATE_SCALAR if w.gate == "scalar" else oracle.GATE_CHANNEL

    def run(n_pairs, n_tok):
        sel = pairs[:n_pairs]
        q = np.stack([inp["q"][b, :n_tok, h] for b, h in sel])[:, :, None]
        k = np.stack([inp["k"][b, :n_tok, h] for b, h in sel])[:, :, None]
        v = np.stack([inp["v"][b, :n_tok, h] for b, h in sel])[:, :, None]
        a = np.stack([inp["alpha"][b, :n_tok, h] for b, h in sel])[:, :, None]
        be = np.stack([inp["beta"][b, :n_tok, h] for b, h in sel])[:, :, None]
        s0 = None
        if inp["state0"] is not None:
            s0 = np.stack([inp["state0"][b, h] for b, h in sel])[:, None]
        t = time.perf_counter()
        oracle.forward(q, k, v, a, be, s0, gate=g, threads=min(cores, n_pairs))
        return time.perf_counter() - t

    # probe with one slice of up to 1024 tokens, then size the sample: every
    # (batch, head) slice in full if that fits the time target, else a prefix
    n_tok = min(w.T, 1024)
    t1 = run(1, n_tok)
    n_pairs = len(pairs)
    waves = -(-n_pairs // cores)
    est = t1 * (w.T / n_tok) * waves
    n_tok = w.T if est <= target_s else max(256, int(w.T * target_s / est))
    # a workload the cores finish well inside the target is repeated, so that
    # the timing spans about target_s
    reps = 1 if est >= target_s / 2 else max(1, min(100, int(target_s / max(est, 1e-3))))
    dt = sum(run(n_pairs, n_tok) for _ in range(reps))
    head_tokens = reps * n_pairs * n_tok
    tok_per_s = head_tokens / dt / w.H   # tokens of the workload (all H heads) per second
    return {"value": tok_per_s, "unit": "tokens/sec", "cores": min(cores, n_pairs),
            "kind": "oracle",
            "sample": f"{reps} x {n_pairs} (batch,head) slices x {n_tok} tokens of {w.name}, "
                      f"fp64 token loop, {dt:.2f} s; tokens/s = head-tokens/s / H"}


def decode_bytes(w) -> float:
    """HBM bytes one decode step must move per batch: read and write every
    state (fp32), read the token's q, k, v, alpha, beta, write o."""
    s_in = 2 if w.dtype == "bf16" else 4
    per_head = (8 * w.dk * w.dv + (2 * w.dk + w.dv) * s_in + 4
                + (4 * w.dk if w.gate == "channel" else 4) + 4 * w.dv)
    return float(per_head * w.B * w.H)


def cpu_baseline_decode(w, inp, max_threads=16, target_s=10.0, n_pairs=1024):
    """Time the oracle's token loop (T = 1) on a sample of (batch, head)
    states of the decode batch."""
    import numpy as np

    import oracle
    cores = max(1, min(max_threads, len(os.sched_getaffinity(0))))
    g = oracle.GATE_SCALAR if w.gate == "scalar" else oracle.GATE_CHANNEL
    sel = [(b, h) for b in range(w.B) for h in range(w.H)][:n_pairs]
    pick = lambda name: np.stack([inp[name][b, :, h] for b, h in sel])[:, :, None]
    q, k, v, a, be = (pick(n) for n in ("q", "k", "v", "alpha", "beta"))
    s0 = np.stack([inp["state0"][b, h] for b, h in sel])[:, None]
    reps, dt = 0, 0.0
    while dt < target_s and reps < 10000:
        t = time.perf_counter()
        oracle.forward(q, k, v, a, be, s0, gate=g, threads=cores)
        dt += time.perf_counter() - t
        reps += 1
    return {"value": reps * len(sel) / w.H / dt, "unit": "tokens/sec", "cores": cores,
            "kind": "oracle",
            "sample": f"{reps} x {len(sel)} (batch,head) states of {w.name}, one token each, "
                      f"fp64 token loop, {dt:.2f} s; tokens/s = head-steps/s / H"}


def bench_decode(args, w):
    """One step = gdn_decode_step over the whole batch, in place."""
    import torch

    from gated_delta_rule_12_amd import gdn
    from gated_delta_rule_12_amd.workloads import make_inputs, to_device
    inp = make_inputs(w)
    d = to_device(inp, w, "cuda")
    tok = {n: d[n][:, 0].contiguous() for n in ("q", "k", "v", "alpha", "beta")}
    st = d["state0"].clone()
    out = torch.empty((w.B, w.H, w.dv), dtype=torch.float32, device="cuda")

    def step():
        gdn.decode_step(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], st,
                        out=out, inplace=True)

    for _ in range(args.warmup):
        step()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gdn.gdn_profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kern = gdn.gdn_profile_read()
    gdn.gdn_profile_enable(False)
    k_us = 1e3 * kern["k_decode"][0] / kern["k_decode"][1]
    # the fused-prologue entry point on the same tensors (read as raw
    # projections and logits): same traffic, a few more operations per head
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        gdn.decode_step(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], st,
                        out=out, inplace=True, raw=True)
    e1.record(stream)
    torch.cuda.synchronize()
    raw_ms = e0.elapsed_time(e1) / args.steps
    abytes = decode_bytes(w)
    achieved = abytes / (k_us * 1e-6) / 1e9
    log(f"step {ms * 1e3:.1f} us, k_decode {k_us:.1f} us per launch")
    cpu = None if args.no_cpu_baseline else cpu_baseline_decode(w, inp)
    res = {"metric": "decode tokens/sec (one gated-delta token per sequence, H=16 d=128)",
           "value": round(w.B / (ms * 1e-3), 1), "unit": "tokens/sec", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic",
           "config": {"workload": w.name, "B": w.B, "H": w.H, "dk": w.dk, "dv": w.dv,
                      "gate": w.gate, "input_dtype": w.dtype, "entry": "gdn_decode_step",
                      "state": "in place", "global_batch": w.B, "parallelism": "single-gpu"},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": stored_traffic(w.name, "k_decode"), "kernel": "k_decode",
                        "kernel_timing": "HIP events around each launch, in a second run of the same steps after the timed region",
                        "kernel_avg_launch_us": round(k_us, 2), "algorithmic_bytes": abytes,
                        "step_achieved": round(abytes / (ms * 1e-3) / 1e9, 1)},
           "cpu_baseline": cpu, "raw_prologue_ms_per_step": round(raw_ms, 5)}
    print(json.dumps(res), flush=True)


def backward_bytes(w) -> float:
    """HBM bytes gdn_backward must move: read q, k, v, the gates, beta and
    dL/dout, write dq, dk, dv, dalpha, dbeta (per head-token); read the start
    state and dL/dS_T and write dL/dS_0 (per head)."""
    s_in = 2 if w.dtype == "bf16" else 4
    gate = 4 * w.dk if w.gate == "channel" else 4
    per_tok = ((2 * w.dk + w.dv) * s_in + gate + 4 + 4 * w.dv
               + 8 * w.dk + 4 * w.dv + gate + 4)
    return float(per_tok * w.B * w.T * w.H + 12 * w.dk * w.dv * w.B * w.H)


def cpu_baseline_backward(w, inp, gr, max_threads=16, target_s=10.0):
    """Time the oracle's backward on (batch, head) slices of the workload,
    the first n_tok tokens of each."""
    import numpy as np

    import oracle
    cores = max(1, min(max_threads, len(os.sched_getaffinity(0))))
    g = oracle.GATE_SCALAR if w.gate == "scalar" else oracle.GATE_CHANNEL
    sel = [(b, h) for b in range(w.B) for h in range(w.H)][:cores]
    n_tok = min(w.T, 1024)
    pick = lambda x: np.stack([x[b, :n_tok, h] for b, h in sel])[:, :, None]
    args = [pick(inp[n]) for n in ("q", "k", "v", "alpha", "beta")]
    s0 = np.stack([inp["state0"][b, h] for b, h in sel])[:, None]
    ds = np.stack([gr["dstate"][b, h] for b, h in sel])[:, None]
    dout = pick(gr["dout"])
    reps, dt = 0, 0.0
    while dt < target_s and reps < 1000:
        t = time.perf_counter()
        oracle.backward(*args, s0, dout, ds, gate=g, threads=cores)
        dt += time.perf_counter() - t
        reps += 1
    return {"value": reps * len(sel) * n_tok / w.H / dt, "unit": "tokens/sec", "cores": cores,
            "kind": "oracle",
            "sample": f"{reps} x {len(sel)} (batch,head) slices x {n_tok} tokens of {w.name}, "
                      f"fp64 backward over stored states, {dt:.2f} s; tokens/s = head-tokens/s / H"}


def bench_backward(args, w):
    """One step = gdn_backward over the whole batch (dL/dout and dL/dS_T
    given, dL/dS_0 wanted)."""
    import torch

    from gated_delta_rule_12_amd import gdn
    from gated_delta_rule_12_amd.workloads import make_grads, make_inputs, to_device
    inp = make_inputs(w)
    gr = make_grads(w)
    d = to_device(inp, w, "cuda")
    g_out = torch.from_numpy(gr["dout"]).cuda()
    g_st = torch.from_numpy(gr["dstate"]).cuda()
    gate = gdn.GDN_GATE_SCALAR if w.gate == "scalar" else gdn.GDN_GATE_CHANNEL
    ws = torch.empty(max(1, gdn.gdn_backward_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, gate)),
                     dtype=torch.uint8, device="cuda")

    def step():
        gdn.backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], g_out, g_st,
                     workspace=ws)

    for _ in range(args.warmup):
        step()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gdn.gdn_profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kern = gdn.gdn_profile_read()
    gdn.gdn_profile_enable(False)
    k_us = 1e3 * kern["k_backward"][0] / kern["k_backward"][1]
    abytes = backward_bytes(w)
    achieved = abytes / (k_us * 1e-6) / 1e9
    log(f"step {ms * 1e3:.1f} us, k_backward {k_us:.1f} us per launch")
    cpu = None if args.no_cpu_baseline else cpu_baseline_backward(w, inp, gr)
    res = {"metric": "backward tokens/sec (gradients through the gated-delta recurrence, H=16 d=128 T=8K)",
           "value": round(w.tokens / (ms * 1e-3), 1), "unit": "tokens/sec", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic",
           "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
                      "gate": w.gate, "input_dtype": w.dtype, "entry": "gdn_backward",
                      "global_batch": w.B, "seq_len": w.T, "parallelism": "single-gpu"},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": stored_traffic(w.name + "-backward", "k_backward"),
                        "kernel": "k_backward",
                        "kernel_timing": "HIP events around each launch, in a second run of the same steps after the timed region",
                        "kernel_avg_launch_us": round(k_us, 2), "algorithmic_bytes": abytes,
                        "kernel_us_per_step": {n: round(1e3 * v[0] / args.steps, 2)
                                               for n, v in kern.items()},
                        "step_achieved": round(abytes / (ms * 1e-3) / 1e9, 1)},
           "cpu_baseline": cpu}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the GPU clock takes tens of milliseconds of load to settle: 200 untimed
    # steps (about 0.1 s on the main workload) before the timed region
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="main-bf16")
    ap.add_argument("--segments", type=int, default=None,
                    help="sequence-parallel segments (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time gdn_backward on the workload instead of the forward")
    ap.add_argument("--no-single-stream", action="store_true",
                    help="sequence parallel: skip the single-stream comparison (for kernel traces)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path is single-GPU: no sharding or collectives are built)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from gated_delta_rule_12_amd import gdn
    from gated_delta_rule_12_amd.workloads import make_inputs, to_device, workload

    w = workload(int(args.workload) if args.workload.isdigit() else args.workload)
    if w.name == "decode-bf16":
        bench_decode(args, w)
        return
    if args.backward:
        bench_backward(args, w)
        return
    # None: gdn_chunk_fwd with the library's schedule; a count: gdn_seqpar_fwd
    G = args.segments if args.segments is not None else (w.n_segments if w.n_segments > 1 else None)
    log(f"workload {w}, segments {G if G is not None else 'library schedule'}")
    t = time.time()
    inp = make_inputs(w)
    d = to_device(inp, w, "cuda")
    log(f"inputs ready in {time.time() - t:.1f} s")
    dt_code = gdn.GDN_BF16 if w.dtype == "bf16" else gdn.GDN_F32
    gate_code = gdn.GDN_GATE_SCALAR if w.gate == "scalar" else gdn.GDN_GATE_CHANNEL
    path = gdn.gdn_chunk_path(w.dk, w.dv, w.chunk, dt_code, gate_code)
    out = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.float32, device="cuda")
    st = torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")
    ws = gdn.workspace_for(d["q"], d["v"], d["alpha"], w.chunk, G)

    def step(nseg=G):
        gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"],
                      chunk=w.chunk, n_segments=nseg, out=out, state_out=st,
                      workspace=ws if nseg == G else None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")

    # timed region: events on the stream the kernels are launched on, and no
    # per-kernel events inside it (each costs a few microseconds of GPU time
    # between kernels: ~28 us per step on the main workload)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # per-kernel durations: the same number of steps again, each kernel
    # bracketed by the library's HIP events on the launch stream
    gdn.gdn_profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kern = gdn.gdn_profile_read()
    gdn.gdn_profile_enable(False)
    # per step: total time of each kernel (several launches per step when the
    # path is pipelined over chunk slabs) and its launches
    per_kernel_us = {k: 1e3 * v[0] / args.steps for k, v in kern.items()}
    launches = {k: v[1] / args.steps for k, v in kern.items()}
    dominant = max(per_kernel_us, key=per_kernel_us.get) if per_kernel_us else None
    log(f"step {ms * 1e3:.1f} us; kernel time per step (us): "
        + ", ".join(f"{k} {v:.1f} ({launches[k]:g} launches)" for k, v in per_kernel_us.items()))

    tokens = w.B * w.T
    value = tokens / (ms * 1e-3)
    abytes = algorithmic_bytes(w)
    aflops = algorithmic_flops(w)
    # dominant kernel: each launch covers an equal share of the head-tokens and
    # their algorithmic bytes, so bytes per launch / average launch time equals
    # bytes per step / that kernel's time per step
    dom_us = per_kernel_us[dominant]
    achieved = abytes / (dom_us * 1e-6) / 1e9
    step_achieved = abytes / (ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": stored_traffic(w.name, dominant) if args.segments is None else None,
            "kernel": dominant,
            "kernel_timing": "HIP events around each launch, in a second run of the same steps after the timed region",
            "kernel_launches_per_step": launches[dominant],
            "kernel_avg_launch_us": round(dom_us / launches[dominant], 2),
            "kernel_us_per_step": {k: round(v, 2) for k, v in per_kernel_us.items()},
            "algorithmic_bytes": abytes,
            "step_achieved": round(step_achieved, 1),
            "step_frac": round(step_achieved / HBM_PEAK_GBS, 4),
            "mfma_frac": round(aflops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}

    extra = {}
    if G is not None and G > 1 and not args.no_single_stream:
        for _ in range(2):
            step(1)
        torch.cuda.synchronize()
        e0.record(stream)
        n1 = max(1, args.steps // 5)
        for _ in range(n1):
            step(1)
        e1.record(stream)
        torch.cuda.synchronize()
        extra["single_stream_ms"] = round(e0.elapsed_time(e1) / n1, 4)
        extra["seqpar_ms"] = round(ms, 4)
        log(f"single-stream {extra['single_stream_ms']} ms vs seq-par {ms:.4f} ms")

    cpu = None
    if not args.no_cpu_baseline and int(os.environ.get("RANK", "0")) == 0:
        cpu = cpu_baseline(w, inp)
        log(f"cpu baseline: {cpu}")

    res = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/sec", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if path == gdn.GDN_PATH_MFMA else "f32",
           "data": "synthetic",
           "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
                      "chunk": w.chunk, "gate": w.gate, "input_dtype": w.dtype,
                      "entry": "gdn_seqpar_fwd" if G is not None else "gdn_chunk_fwd",
                      "segments": G if G is not None else gdn.gdn_chunk_segments(
                          w.B, w.T, w.H, w.dk, w.dv, w.chunk, dt_code, gate_code),
                      "global_batch": w.B, "seq_len": w.T,
                      "parallelism": "single-gpu",
                      "kernel_path": "mfma" if path == gdn.GDN_PATH_MFMA else "valu"},
           "roofline": roof, "cpu_baseline": cpu}
    res.update(extra)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
