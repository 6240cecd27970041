"""Seeded synthetic workloads for the gated delta rule forward pass.

This module draws inputs only; it holds none of the method's arithmetic, and
both the HIP path's tests/bench and the oracle-based checks take their inputs
from it.  The recipe (one numpy PCG64 stream per workload, fixed draw order):

  1. q ~ N(0,1), then L2-normalised per (batch, token, head) along features
     in fp64 (the per-head L2 norm of q and k in the DeltaNet block);
  2. k ~ N(0,1), normalised the same way;
  3. v ~ N(0,1);
  4. alpha = sigmoid(N(mu_a, 0.5)) — one value per token-head (scalar gate)
     or one per key channel (channel gate); mu_a = 2 for every listed workload;
  5. beta = sigmoid(N(0,1)) per token-head;
  6. state0 ~ N(0, std^2) per head when std > 0, else no start state.

Values are drawn in fp64, rounded to fp32, and q/k/v are then rounded to
bf16 (round-to-nearest-even) for bf16 workloads.  The arrays returned hold
exactly the values that are uploaded, so any checker reads the same numbers.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int
    dtype: str = "bf16"          # dtype of q, k, v: "bf16" or "f32"
    gate: str = "scalar"         # "scalar" or "channel"
    state0_std: float = 0.0      # 0 -> zero start state
    n_segments: int = 1          # >1: sequence-parallel split
    alpha_mean: float = 2.0      # mean of the gate logits
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.B * self.T

    @property
    def head_tokens(self) -> int:
        return self.B * self.T * self.H

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of this path, index 0..4.
WORKLOADS = [
    Workload("tiny-f32", B=1, H=1, T=256, dk=16, dv=16, chunk=16, dtype="f32",
             seed=1234),
    Workload("small-bf16", B=4, H=8, T=2048, dk=64, dv=64, chunk=64, seed=1235),
    Workload("main-bf16", B=2, H=16, T=8192, dk=128, dv=128, chunk=64,
             state0_std=0.02, seed=1236),
    Workload("long-seqpar-bf16", B=1, H=4, T=65536, dk=128, dv=128, chunk=64,
             n_segments=8, seed=1237),
    Workload("channel-gate-bf16", B=8, H=16, T=4096, dk=128, dv=128, chunk=64,
             gate="channel", seed=1238),
]

# One decode step (T = 1) of a serving batch: 256 sequences x 16 heads at
# d = 128, each with a persistent fp32 state.  The pages give no decode size;
# this batch makes the step stream 512 MiB of state (read and write), well
# past launch latency, with the main workload's head shape and distributions.
DECODE_WORKLOAD = Workload("decode-bf16", B=256, H=16, T=1, dk=128, dv=128, chunk=64,
                           state0_std=0.02, seed=1239)


def workload(key) -> Workload:
    if isinstance(key, Workload):
        return key
    if isinstance(key, int):
        return WORKLOADS[key]
    for w in WORKLOADS + [DECODE_WORKLOAD]:
        if w.name == key:
            return w
    raise KeyError(key)


def _l2_normalise(x):
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    n[n == 0.0] = 1.0
    return x / n


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _round_bf16(x32):
    """fp32 numpy -> bf16 values (RNE), returned as fp32 numpy."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16)
    return t.to(torch.float32).numpy()


def make_inputs(w: Workload, seed: int | None = None) -> dict:
    """Draw one workload.  Returns fp32 numpy arrays: q, k [B,T,H,dk],
    v [B,T,H,dv], alpha [B,T,H] or [B,T,H,dk], beta [B,T,H], and state0
    [B,H,dv,dk] or None."""
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    out = {}
    for name, d in (("q", dk), ("k", dk)):
        x = _l2_normalise(rng.standard_normal((B, T, H, d)))
        out[name] = x.astype(np.float32)
        del x
    out["v"] = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    ashape = (B, T, H) if w.gate == "scalar" else (B, T, H, dk)
    out["alpha"] = _sigmoid(rng.normal(w.alpha_mean, 0.5, ashape)).astype(np.float32)
    out["beta"] = _sigmoid(rng.standard_normal((B, T, H))).astype(np.float32)
    if w.state0_std > 0:
        out["state0"] = (w.state0_std * rng.standard_normal((B, H, dv, dk))).astype(np.float32)
    else:
        out["state0"] = None
    if w.dtype == "bf16":
        for name in ("q", "k", "v"):
            out[name] = _round_bf16(out[name])
    elif w.dtype != "f32":
        raise ValueError(w.dtype)
    return out


def make_raw_inputs(w: Workload, seed: int | None = None) -> dict:
    """Raw projections for the fused-prologue entry point: q, k ~ N(0,1)
    times a per-(batch, token, head) length drawn from U(0.2, 5), not
    normalised, with the key of token 0 of head 0 set to zero; v ~ N(0,1);
    alpha as logits N(mu_a, 0.5) (per token-head or per key channel); beta as
    logits N(0,1); state0 as in make_inputs.  Same fp32 / bf16 rounding and
    return layout as make_inputs, with alpha and beta holding logits."""
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    out = {}
    for name in ("q", "k"):
        x = rng.standard_normal((B, T, H, dk)) * rng.uniform(0.2, 5.0, (B, T, H, 1))
        out[name] = x.astype(np.float32)
    if T > 0:
        out["k"][0, 0, 0, :] = 0.0
    out["v"] = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    ashape = (B, T, H) if w.gate == "scalar" else (B, T, H, dk)
    out["alpha"] = rng.normal(w.alpha_mean, 0.5, ashape).astype(np.float32)
    out["beta"] = rng.standard_normal((B, T, H)).astype(np.float32)
    if w.state0_std > 0:
        out["state0"] = (w.state0_std * rng.standard_normal((B, H, dv, dk))).astype(np.float32)
    else:
        out["state0"] = None
    if w.dtype == "bf16":
        for name in ("q", "k", "v"):
            out[name] = _round_bf16(out[name])
    return out


def make_grads(w: Workload, seed: int | None = None, with_state: bool = True) -> dict:
    """Upstream gradients for a backward pass over workload w: dout
    ~ N(0, 1) [B,T,H,dv] and, with_state, dstate ~ N(0, 1) [B,H,dv,dk]
    (else None); fp32, from their own PCG64 stream (seed + 1 by default)."""
    rng = np.random.Generator(np.random.PCG64((w.seed + 1) if seed is None else seed))
    dout = rng.standard_normal((w.B, w.T, w.H, w.dv)).astype(np.float32)
    ds = rng.standard_normal((w.B, w.H, w.dv, w.dk)).astype(np.float32) if with_state else None
    return {"dout": dout, "dstate": ds}


def make_inputs_device(w: Workload, device="cuda") -> dict:
    """Workloads too large to draw on the host: the same recipe as
    make_inputs, drawn on the device by torch's seeded Philox generator (so
    the values differ from make_inputs' for the same seed), q and k
    L2-normalised in fp32 before the cast to the workload dtype.  Returns
    device tensors laid out as to_device's; checkers read the uploaded values
    of the slices they need with slice_inputs."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    res = {}
    for name, d in (("q", dk), ("k", dk)):
        x = torch.randn((B, T, H, d), generator=g, device=device)
        x /= torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)
        res[name] = x.to(dt)
        del x
    res["v"] = torch.randn((B, T, H, dv), generator=g, device=device).to(dt)
    ashape = (B, T, H) if w.gate == "scalar" else (B, T, H, dk)
    a = torch.randn(ashape, generator=g, device=device)
    res["alpha"] = torch.sigmoid(a * 0.5 + w.alpha_mean)
    del a
    res["beta"] = torch.sigmoid(torch.randn((B, T, H), generator=g, device=device))
    res["state0"] = (w.state0_std * torch.randn((B, H, dv, dk), generator=g, device=device)
                     if w.state0_std > 0 else None)
    return res


def make_grads_device(w: Workload, device="cuda", with_state: bool = True) -> dict:
    """make_grads' recipe drawn on the device (torch's seeded Philox
    generator, seed + 1), for workloads too large to draw on the host."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(w.seed + 1)
    dout = torch.randn((w.B, w.T, w.H, w.dv), generator=g, device=device)
    ds = torch.randn((w.B, w.H, w.dv, w.dk), generator=g, device=device) if with_state else None
    return {"dout": dout, "dstate": ds}


def slice_inputs(d: dict, pairs) -> dict:
    """The uploaded values of the listed (batch, head) slices of device
    inputs, as fp32 numpy arrays shaped like make_inputs' with B = len(pairs)
    and H = 1."""
    out = {}
    for name in ("q", "k", "v", "alpha", "beta"):
        out[name] = np.stack([d[name][b, :, h].float().cpu().numpy() for b, h in pairs])[:, :, None]
    s0 = d.get("state0")
    out["state0"] = None if s0 is None else np.stack([s0[b, h].cpu().numpy() for b, h in pairs])[:, None]
    return out


def to_device(inputs: dict, w: Workload, device="cuda"):
    """Upload to torch tensors: q/k/v in the workload dtype, the rest fp32."""
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    res = {}
    for name, arr in inputs.items():
        if arr is None:
            res[name] = None
            continue
        t = torch.from_numpy(np.ascontiguousarray(arr))
        if name in ("q", "k", "v"):
            t = t.to(dt)
        res[name] = t.to(device)
    return res
