"""GPU parity of gdn_chunk_fwd_raw (the block's prologue fused into the
chunked forward: per-head L2 norm of q and k, sigmoid of the gate and beta
logits) against the oracle's prologue followed by its token loop, every
(batch, head) slice, on every kernel family and path: the whole-head MFMA
loop (with segments), the sliced MFMA loop for both gate kinds, and the
vector-ALU family (fp32 and other shapes); the main and channel-gate
workloads at full size."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_12_amd import gdn
from gated_delta_rule_12_amd.workloads import WORKLOADS, Workload, make_raw_inputs, to_device
from parity import TOL, out_err, state_err

pytestmark = pytest.mark.gpu

PTD, DTP = gdn.GDN_PREDICT_THEN_DECAY, gdn.GDN_DECAY_THEN_PREDICT


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()


def run_and_check(w, order=PTD):
    import torch
    raw = make_raw_inputs(w)
    d = to_device(raw, w)
    o, s = gdn.chunk_fwd_raw(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"],
                             chunk=w.chunk, order=order)
    torch.cuda.synchronize()
    q, k, a, b = oracle.prologue(raw["q"], raw["k"], raw["alpha"], raw["beta"])
    g = oracle.GATE_SCALAR if w.gate == "scalar" else oracle.GATE_CHANNEL
    o_ref, s_ref = oracle.forward(q, k, raw["v"], a, b, raw["state0"], gate=g, order=order)
    o, s = o.cpu().numpy(), s.cpu().numpy()
    eo, es = out_err(o, o_ref), state_err(s, s_ref)
    to, ts = TOL[w.dtype]
    print(f"  {w.name}: out err {eo:.3e} (tol {to}), state err {es:.3e} (tol {ts})", flush=True)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert eo <= to and es <= ts, (eo, es)


CASES = [
    # B, H, T, dk, dv, chunk, dtype, gate, order, state0_std, alpha_mean
    (1, 32, 1000, 128, 128, 64, "bf16", "scalar", PTD, 0.5, 2.0),   # whole-head, 4 segments
    (1, 32, 700, 64, 64, 64, "bf16", "scalar", DTP, 0.3, 2.0),      # whole-head d = 64
    (1, 32, 512, 128, 128, 64, "bf16", "scalar", PTD, 0.0, 6.0),    # long memory
    (16, 16, 700, 128, 128, 64, "bf16", "scalar", DTP, 0.3, 2.0),   # whole-head, one pass
    (1, 3, 449, 128, 128, 64, "bf16", "scalar", PTD, 0.5, 2.0),     # sliced loop
    (1, 3, 449, 128, 128, 64, "bf16", "channel", PTD, 0.5, 2.0),    # sliced loop, channel gate
    (2, 2, 320, 64, 64, 64, "bf16", "channel", DTP, 0.5, 6.0),
    (1, 2, 512, 128, 128, 64, "bf16", "channel", PTD, 0.5, -6.0),   # direct diagonal blocks
    (1, 1, 256, 16, 16, 16, "f32", "scalar", PTD, 0.0, 2.0),        # vector-ALU family
    (2, 3, 100, 96, 112, 32, "bf16", "scalar", DTP, 0.5, 2.0),
    (1, 2, 133, 32, 48, 32, "f32", "channel", PTD, 0.5, 2.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_chunk_fwd_raw(case):
    B, H, T, dk, dv, C, dtype, gate, order, std, am = case
    w = Workload("raw", B=B, H=H, T=T, dk=dk, dv=dv, chunk=C, dtype=dtype, gate=gate,
                 state0_std=std, alpha_mean=am, seed=400 + T + dk)
    run_and_check(w, order)


@pytest.mark.parametrize("idx", [2, 4])
def test_chunk_fwd_raw_full_workload(idx):
    """The main (whole-head path, 8 segments) and channel-gate (sliced path)
    workloads at full size on raw projections and logits."""
    run_and_check(WORKLOADS[idx].with_(name=WORKLOADS[idx].name + "-raw"))


def test_raw_equals_normalised_inputs_for_unit_rows():
    """On inputs that are already unit rows and gates given as logits, the
    raw entry point and gdn_chunk_fwd on sigmoid(logits) agree to rounding."""
    import torch
    w = Workload("raw-unit", B=1, H=32, T=640, dk=128, dv=128, chunk=64, state0_std=0.3, seed=55)
    raw = make_raw_inputs(w)
    q, k, a, b = oracle.prologue(raw["q"], raw["k"], raw["alpha"], raw["beta"])
    unit = dict(raw, q=q.astype(np.float32), k=k.astype(np.float32), alpha=a.astype(np.float32),
                beta=b.astype(np.float32))
    w32 = w.with_(dtype="f32")
    d = to_device(unit, w32)
    dl = to_device(dict(raw, q=unit["q"], k=unit["k"]), w32)
    o1, s1 = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"])
    o2, s2 = gdn.chunk_fwd_raw(dl["q"], dl["k"], dl["v"], dl["alpha"], dl["beta"], dl["state0"])
    torch.cuda.synchronize()
    assert (o1 - o2).abs().max().item() <= 1e-5 * o1.abs().max().item()
    assert (s1 - s2).abs().max().item() <= 1e-5 * s1.abs().max().item()
