"""Benchmark of the chunkwise gated delta rule forward on one MI355X.

One step = one full forward (every kernel of the path) over one batch of the
workload, inputs already resident in HBM.  Prints ONE JSON line on stdout;
diagnostics go to stderr.  After the W warmup steps, untimed steps run for a
settle period (--settle-ms, default 500 ms: the GPU clock takes tens to
hundreds of milliseconds of load to reach its working frequency), reported
as settle_ms / settle_steps.  The timed region holds only the K steps.
roofline.achieved / frac are the whole step's algorithmic bytes over the
step's time; per-kernel durations (the dominant kernel's figures) come from
HIP events the library records on the launch stream into a caller-owned
timer, in a second run of the same number of steps.  Achievable peaks (a
device copy and an MFMA loop) are measured in the same run.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload main-bf16]

Default workload: main-bf16 (B=2, H=16, T=8192, dk=dv=128, chunk 64, scalar
gate, start state N(0, 0.02^2)).  The long workload runs the sequence-parallel
entry point (8 segments, which the library cuts finer to fill the device:
see gdn_seqpar_segments) and also reports the single-stream time beside it.
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
MFMA_F32_PEAK_TFLOPS = 157.3    # MI355X dense fp32 MFMA, vendor figure


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


def settle(step, settle_ms: float):
    """Untimed steps until settle_ms of wall time have passed (at least one
    step); returns (milliseconds, steps)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while True:
        step()
        n += 1
        if n % 8 == 0 or settle_ms <= 0:
            torch.cuda.synchronize()
            el = (time.perf_counter() - t0) * 1e3
            if el >= settle_ms:
                return round(el, 1), n


def measure_peaks():
    """Achievable peaks on this device, for fractions beside the vendor ones:
    a plain 1 GiB device copy (bytes read + written per second) and eight
    independent chains of 16x16x32 bf16 MFMAs on two waves per SIMD."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "gated_delta_rule_12_amd", "libgdn_peaks.so")
    L = ctypes.CDLL(path)
    L.gdn_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.gdn_peak_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    cp = lambda: L.gdn_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                 nbytes, sp)
    for _ in range(3):
        assert cp() == 0
    reps = 10
    e0.record(stream)
    for _ in range(reps):
        cp()
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    blocks, iters = 2 * 256, 2000
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2 * 4 * blocks, dtype=torch.int64, device="cuda")
    mf = {}
    for shape, name, flop in ((0, "16x16x32", 16384), (1, "32x32x16", 32768)):
        run = lambda: L.gdn_peak_mfma(ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(clk.data_ptr()),
                                      shape, blocks, iters, sp)
        assert run() == 0
        e0.record(stream)
        for _ in range(3):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        tfs = 3 * blocks * 4 * 8 * iters * flop / (e0.elapsed_time(e1) * 1e-3) / 1e12
        c = clk.view(-1, 2).double().mean(0)
        mf[name] = {"TFs": round(tfs, 1),
                    # two waves share a SIMD: its cycles per MFMA
                    "cycles_per_mfma_per_simd": round(float(c[0]) / (8 * iters * 2), 2),
                    "shader_clock_GHz": round(float(c[0]) / (float(c[1]) / 1e8) / 1e9, 3)}
    best = max(v["TFs"] for v in mf.values())
    torch.cuda.empty_cache()
    return {"hbm_copy_GBs": round(copy_gbs, 1), "mfma_bf16_TFs": best, "mfma_bf16_shapes": mf,
            "how": "1 GiB device copy (16-byte non-temporal loads and stores), read + write bytes; "
                   "8 independent bf16 MFMA chains per wave, 2 waves per SIMD, best shape"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores() -> int:
    """Cores this process may use: its CPU affinity, capped by
    OMP_NUM_THREADS when the environment sets it (the share of the host a
    one-GPU job is given)."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return n


def host_info() -> dict:
    return {"nproc": len(os.sched_getaffinity(0)), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "cpu_model": cpu_model()}


def stored_step_traffic(tag, kernels=None):
    """HBM bytes per step of the listed kernels (None: every kernel the
    record holds) from profiles/traffic_<tag>.json, or None when absent,
    taken on other kernel sources, or missing one of them."""
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    per = rec.get("per_kernel", {})
    names = list(per) if kernels is None else list(kernels)
    if not names or any(k not in per for k in names):
        return None
    return round(sum(per[k]["read_bytes"] + per[k]["write_bytes"] for k in names))


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


def cpu_baseline(w, inp, target_s=10.0):
    """Time the oracle on a bounded sample of (batch, head) slices, with
    min(host cores, B * H) threads (OpenMP over the slices)."""
    import numpy as np

    import oracle
    cores = max(1, host_cores())
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
            "kind": "oracle", **host_info(),
            "sample": f"{reps} x {n_pairs} (batch,head) slices x {n_tok} tokens of {w.name}, "
                      f"fp64 token loop, {dt:.2f} s; tokens/s = head-tokens/s / H"}


def decode_bytes(w) -> float:
    """HBM bytes one decode step must move per batch: read and write every
    state (fp32), read the token's q, k, v, alpha, beta, write o."""
    s_in = 2 if w.dtype == "bf16" else 4
    per_head = (8 * w.dk * w.dv + (2 * w.dk + w.dv) * s_in + 4
                + (4 * w.dk if w.gate == "channel" else 4) + 4 * w.dv)
    return float(per_head * w.B * w.H)


def cpu_baseline_decode(w, inp, target_s=10.0, n_pairs=1024):
    """Time the oracle's token loop (T = 1) on a sample of (batch, head)
    states of the decode batch, one thread per host core."""
    import numpy as np

    import oracle
    cores = max(1, host_cores())
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
            "kind": "oracle", **host_info(),
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
    settle_ms, settle_steps = settle(step, args.settle_ms)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    timer = gdn.Timer()
    for _ in range(args.steps):
        gdn.decode_step(tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], st,
                        out=out, inplace=True, timer=timer)
    torch.cuda.synchronize()
    kern = timer.read()
    timer.close()
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
    peaks = None if args.no_peaks else measure_peaks()
    cpu = None if args.no_cpu_baseline else cpu_baseline_decode(w, inp)
    res = {"metric": "decode tokens/sec (one gated-delta token per sequence, H=16 d=128)",
           "value": round(w.B / (ms * 1e-3), 1), "unit": "tokens/sec", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "settle_ms": settle_ms,
           "settle_steps": settle_steps, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic",
           "config": {"workload": w.name, "B": w.B, "H": w.H, "dk": w.dk, "dv": w.dv,
                      "gate": w.gate, "input_dtype": w.dtype, "entry": "gdn_decode_step",
                      "state": "in place", "global_batch": w.B, "parallelism": "single-gpu"},
           "roofline": {"bound": "hbm", "achieved": round(abytes / (ms * 1e-3) / 1e9, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(abytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "traffic": stored_step_traffic(w.name, ["k_decode"]),
                        "kernel": "whole step: k_decode", "algorithmic_bytes": abytes,
                        "kernel_timing": "HIP events around each launch (caller-owned timer), in a second run of the same steps after the timed region",
                        "dominant_kernel": {"kernel": "k_decode", "launches_per_step": 1,
                                            "avg_launch_us": round(k_us, 2), "achieved": round(achieved, 1),
                                            "frac": round(achieved / HBM_PEAK_GBS, 4),
                                            "traffic": stored_step_traffic(w.name, ["k_decode"])},
                        "frac_of_achievable_copy": round(abytes / (ms * 1e-3) / 1e9 / peaks["hbm_copy_GBs"], 4)
                        if peaks else None,
                        "achievable_peaks": peaks},
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


def backward_chunk_flops(w) -> dict:
    """Algorithmic flops of the chunked backward per step, by kernel: per
    (batch, head) and chunk of C = 64 tokens at d = dk = dv, the products of
    the chunk-form chain rule with their triangular structure (a lower-
    triangular C x C operand counts half):
      k_bprep   K K^T, Q K^T (C^2 d / 2 each), the UT inverse (C^3 / 6)
      k_bchain  forward: K S^T, S update (C d^2 each), T U' (C^2 d / 2);
                reverse: K dS^T, Q^T dO, K^T dU' (C d^2 each), P^T dO,
                T^T dDelta (C^2 d / 2 each)
      k_bgrad   dO S, dU' S, Delta dS (C d^2 each); dO Delta^T, dDelta U^T,
                (dP o M) K, (dP o M)^T Q (C^2 d / 2 each), (W + W^T) K (C^2 d),
                T^T dT T^T (C^3 / 3)
    as multiply-adds, two flops each."""
    C, d = 64, w.dk
    n = w.B * w.H * ((w.T + C - 1) // C)
    mac = {"k_bprep": C * C * d + C ** 3 / 6,
           "k_bchain": 5 * C * d * d + 1.5 * C * C * d,
           "k_bgrad": 3 * C * d * d + 3 * C * C * d + C ** 3 / 3}
    return {k: 2.0 * v * n for k, v in mac.items()}


def cpu_baseline_backward(w, inp, gr, target_s=10.0):
    """Time the oracle's backward on (batch, head) slices of the workload,
    the first n_tok tokens of each, one slice per host core."""
    import numpy as np

    import oracle
    cores = max(1, host_cores())
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
    return {"value": reps * len(sel) * n_tok / w.H / dt, "unit": "tokens/sec",
            "cores": min(cores, len(sel)), "kind": "oracle", **host_info(),
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
    settle_ms, settle_steps = settle(step, args.settle_ms)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    timer = gdn.Timer()
    for _ in range(args.steps):
        gdn.backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], g_out, g_st,
                     workspace=ws, timer=timer)
    torch.cuda.synchronize()
    kern = timer.read()
    timer.close()
    chunked = gdn.gdn_backward_path(w.dk, w.dv, gate) == gdn.GDN_BWD_CHUNKED
    dom = max(kern, key=lambda n: kern[n][0])
    k_us = 1e3 * kern[dom][0] / kern[dom][1]
    log(f"step {ms * 1e3:.1f} us, " + ", ".join(f"{n} {1e3 * v[0] / args.steps:.1f} us" for n, v in kern.items())
        + " per step")
    peaks = None if args.no_peaks else measure_peaks()
    cpu = None if args.no_cpu_baseline else cpu_baseline_backward(w, inp, gr)
    abytes = backward_bytes(w)
    kernel_us = {n: round(1e3 * v[0] / args.steps, 2) for n, v in kern.items()}
    timing = "HIP events around each launch (caller-owned timer), in a second run of the same steps after the timed region"
    if chunked:
        fl = backward_chunk_flops(w)
        step_tf = sum(fl.values()) / (ms * 1e-3) / 1e12
        dom_tf = fl[dom] / kern[dom][1] * args.steps / (k_us * 1e-6) / 1e12 if dom in fl else None
        roof = {"bound": "mfma", "achieved": round(step_tf, 2), "peak": MFMA_F32_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(step_tf / MFMA_F32_PEAK_TFLOPS, 4),
                "traffic": stored_step_traffic(w.name + "-backward", list(kern)),
                "kernel": "whole step: " + " + ".join(kern), "algorithmic_flops": sum(fl.values()),
                "algorithmic_flops_by_kernel": fl, "mfma_dtype": "fp32 (16x16x4)",
                "hbm_bytes_moved_min": abytes,
                "kernel_timing": timing, "kernel_us_per_step": kernel_us,
                "dominant_kernel": {"kernel": dom, "launches_per_step": kern[dom][1] / args.steps,
                                    "avg_launch_us": round(k_us, 2),
                                    "achieved": round(dom_tf, 2) if dom_tf else None,
                                    "frac": round(dom_tf / MFMA_F32_PEAK_TFLOPS, 4) if dom_tf else None,
                                    "traffic": stored_step_traffic(w.name + "-backward", [dom])},
                "achievable_peaks": peaks}
    else:
        achieved = abytes / (k_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(abytes / (ms * 1e-3) / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(abytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "traffic": stored_step_traffic(w.name + "-backward", list(kern)),
                "kernel": "whole step: " + " + ".join(kern), "algorithmic_bytes": abytes,
                "kernel_timing": timing, "kernel_us_per_step": kernel_us,
                "dominant_kernel": {"kernel": dom, "launches_per_step": kern[dom][1] / args.steps,
                                    "avg_launch_us": round(k_us, 2), "achieved": round(achieved, 1),
                                    "frac": round(achieved / HBM_PEAK_GBS, 4),
                                    "traffic": stored_step_traffic(w.name + "-backward", [dom])},
                "frac_of_achievable_copy": round(abytes / (ms * 1e-3) / 1e9 / peaks["hbm_copy_GBs"], 4)
                if peaks else None,
                "achievable_peaks": peaks}
    res = {"metric": "backward tokens/sec (gradients through the gated-delta recurrence, H=16 d=128 T=8K)",
           "value": round(w.tokens / (ms * 1e-3), 1), "unit": "tokens/sec", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "settle_ms": settle_ms,
           "settle_steps": settle_steps, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic",
           "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
                      "gate": w.gate, "input_dtype": w.dtype, "entry": "gdn_backward",
                      "algorithm": "chunked" if chunked else "token",
                      "global_batch": w.B, "seq_len": w.T, "parallelism": "single-gpu"},
           "roofline": roof,
           "cpu_baseline": cpu}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    # the GPU clock takes tens to hundreds of milliseconds of load to reach
    # its working frequency: untimed steps for this long after the warmup
    ap.add_argument("--settle-ms", type=float, default=500.0)
    ap.add_argument("--workload", default="main-bf16")
    ap.add_argument("--segments", type=int, default=None,
                    help="sequence-parallel segments (default: the workload's)")
    ap.add_argument("--library-schedule", action="store_true",
                    help="gdn_chunk_fwd with the library's own schedule even where the workload "
                         "names a segment count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the achievable-peak probes (profiler runs)")
    ap.add_argument("--raw", action="store_true",
                    help="time gdn_chunk_fwd_raw (raw q, k and gate / beta logits, the block's "
                         "prologue fused in) on the workload's shapes")
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
    if args.library_schedule:
        G = None
    log(f"workload {w}, segments {G if G is not None else 'library schedule'}"
        + (f" (run as {gdn.gdn_seqpar_segments(w.B, w.T, w.H, w.dk, w.dv, w.chunk, 1 if w.dtype == 'bf16' else 0, 0 if w.gate == 'scalar' else 1, G)})"
           if G is not None else ""))
    t = time.time()
    if args.raw:
        from gated_delta_rule_12_amd.workloads import make_raw_inputs
        inp = make_raw_inputs(w)
    else:
        inp = make_inputs(w)
    d = to_device(inp, w, "cuda")
    log(f"inputs ready in {time.time() - t:.1f} s")
    dt_code = gdn.GDN_BF16 if w.dtype == "bf16" else gdn.GDN_F32
    gate_code = gdn.GDN_GATE_SCALAR if w.gate == "scalar" else gdn.GDN_GATE_CHANNEL
    path = gdn.gdn_chunk_path(w.dk, w.dv, w.chunk, dt_code, gate_code)
    out = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.float32, device="cuda")
    st = torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")
    ws = gdn.workspace_for(d["q"], d["v"], d["alpha"], w.chunk, G)
    ws_raw = None
    if args.raw:
        if G is not None:
            raise SystemExit("--raw runs the library's schedule (gdn_chunk_fwd_raw); no --segments")
        ws_raw = torch.empty(max(1, gdn.lib().gdn_raw_workspace_bytes(
            w.B, w.T, w.H, w.dk, w.dv, w.chunk, dt_code, gate_code)), dtype=torch.uint8, device="cuda")

    def step(nseg=G, timer=None):
        if args.raw:
            gdn.chunk_fwd_raw(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"],
                              chunk=w.chunk, out=out, state_out=st, workspace=ws_raw, timer=timer)
            return
        gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"],
                      chunk=w.chunk, n_segments=nseg, out=out, state_out=st,
                      workspace=ws if nseg == G else None, timer=timer)

    for _ in range(args.warmup):
        step()
    settle_ms, settle_steps = settle(step, args.settle_ms)
    log(f"warmup done ({args.warmup} steps, then {settle_steps} steps in {settle_ms} ms to settle)")

    # timed region: events on the stream the kernels are launched on, and no
    # per-kernel events inside it (each costs a few microseconds of GPU time
    # between kernels)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # per-kernel durations: the same number of steps again through the timed
    # entry point, each kernel bracketed by HIP events on the launch stream
    timer = gdn.Timer()
    for _ in range(args.steps):
        step(timer=timer)
    torch.cuda.synchronize()
    kern = timer.read()
    timer.close()
    # per step: total time of each kernel and its launches
    per_kernel_us = {k: 1e3 * v[0] / args.steps for k, v in kern.items()}
    launches = {k: v[1] / args.steps for k, v in kern.items()}
    dominant = max(per_kernel_us, key=per_kernel_us.get) if per_kernel_us else None
    log(f"step {ms * 1e3:.1f} us; kernel time per step (us): "
        + ", ".join(f"{k} {v:.1f} ({launches[k]:g} launches)" for k, v in per_kernel_us.items()))

    tokens = w.B * w.T
    value = tokens / (ms * 1e-3)
    abytes = algorithmic_bytes(w)
    aflops = algorithmic_flops(w)
    peaks = None if args.no_peaks else measure_peaks()
    if peaks:
        log(f"achievable peaks: {peaks}")
    # the roofline is the whole step's: its algorithmic bytes over its time
    step_achieved = abytes / (ms * 1e-3) / 1e9
    # counted HBM traffic of the step: every kernel's stored counters (only
    # while they were taken on the current kernel sources)
    # (the counters were taken on the default command of each record: the
    # workload's own segments, the library schedule, or the raw entry point)
    rec_tag = w.name + ("-raw" if args.raw else "-library" if args.library_schedule else "")
    traffic = None
    if args.segments is None:
        traffic = stored_step_traffic(rec_tag, list(per_kernel_us) or None)
    # the dominant kernel (longest per step): each launch covers every
    # head-token, so the step's algorithmic bytes over its average launch
    dom = None
    if dominant is not None:
        dom_us = per_kernel_us[dominant]
        dom_achieved = abytes / (dom_us * 1e-6) / 1e9
        dom = {"kernel": dominant, "launches_per_step": launches[dominant],
               "avg_launch_us": round(dom_us / launches[dominant], 2),
               "achieved": round(dom_achieved, 1), "frac": round(dom_achieved / HBM_PEAK_GBS, 4),
               "traffic": stored_step_traffic(rec_tag, [dominant]) if args.segments is None else None}
    roof = {"bound": "hbm", "achieved": round(step_achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(step_achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "whole step: " + (" + ".join(per_kernel_us) if per_kernel_us else "gdn_chunk_fwd_raw"),
            "algorithmic_bytes": abytes,
            "frac_of_achievable_copy": round(step_achieved / peaks["hbm_copy_GBs"], 4) if peaks else None,
            "mfma_frac": round(aflops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "mfma_frac_of_achievable": round(aflops / (ms * 1e-3) / 1e12 / peaks["mfma_bf16_TFs"], 4) if peaks else None,
            "kernel_us_per_step": {k: round(v, 2) for k, v in per_kernel_us.items()},
            "kernel_timing": "HIP events around each launch (caller-owned timer), in a second run of the same steps after the timed region",
            "dominant_kernel": dom,
            "achievable_peaks": peaks}

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
           "steps": args.steps, "warmup": args.warmup, "settle_ms": settle_ms,
           "settle_steps": settle_steps, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if path == gdn.GDN_PATH_MFMA else "f32",
           "data": "synthetic",
           "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
                      "chunk": w.chunk, "gate": w.gate, "input_dtype": w.dtype,
                      "entry": "gdn_chunk_fwd_raw" if args.raw else (
                          "gdn_seqpar_fwd" if G is not None else "gdn_chunk_fwd"),
                      "segments": G if G is not None else gdn.gdn_chunk_segments(
                          w.B, w.T, w.H, w.dk, w.dv, w.chunk, dt_code, gate_code),
                      "segments_run": gdn.gdn_seqpar_segments(
                          w.B, w.T, w.H, w.dk, w.dv, w.chunk, dt_code, gate_code, G)
                      if G is not None else gdn.gdn_chunk_segments(
                          w.B, w.T, w.H, w.dk, w.dv, w.chunk, dt_code, gate_code),
                      "global_batch": w.B, "seq_len": w.T,
                      "parallelism": "single-gpu",
                      "kernel_path": "mfma" if path == gdn.GDN_PATH_MFMA else "valu"},
           "roofline": roof, "cpu_baseline": cpu}
    res.update(extra)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
