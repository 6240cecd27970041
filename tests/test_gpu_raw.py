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


def run_and_check(w, order=PTD, edit=None, in_place=False):
    """edit(raw) may change the drawn inputs in place before the call;
    in_place: state_out is the start state's buffer."""
    import torch
    raw = make_raw_inputs(w)
    if edit is not None:
        edit(raw)
    d = to_device(raw, w)
    s0 = d["state0"]
    so = None
    if in_place:
        s0 = s0.clone()
        so = s0
    o, s = gdn.chunk_fwd_raw(d["q"], d["k"], d["v"], d["alpha"], d["beta"], s0,
                             chunk=w.chunk, order=order, state_out=so)
    torch.cuda.synchronize()
    if T_empty(w):
        assert o.shape[1] == 0
        ref = raw["state0"] if raw["state0"] is not None else np.zeros((w.B, w.H, w.dv, w.dk), np.float32)
        assert np.array_equal(s.cpu().numpy(), ref)
        return
    q, k, a, b = oracle.prologue(raw["q"], raw["k"], raw["alpha"], raw["beta"])
    g = oracle.GATE_SCALAR if w.gate == "scalar" else oracle.GATE_CHANNEL
    o_ref, s_ref = oracle.forward(q, k, raw["v"], a, b, raw["state0"], gate=g, order=order)
    o, s = o.cpu().numpy(), s.cpu().numpy()
    eo, es = out_err(o, o_ref), state_err(s, s_ref)
    to, ts = TOL[w.dtype]
    print(f"  {w.name}: out err {eo:.3e} (tol {to}), state err {es:.3e} (tol {ts})", flush=True)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert eo <= to and es <= ts, (eo, es)


def T_empty(w):
    return w.T == 0


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
    (4, 16, 300, 128, 128, 64, "bf16", "channel", DTP, 0.5, 2.0),   # head-shared loop, channel gate
    (2, 32, 200, 128, 128, 64, "bf16", "channel", PTD, 0.3, -3.0),
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
    """The main (whole-head path, 8 segments) and channel-gate (head-shared
    path) workloads at full size on raw projections and logits."""
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


@pytest.mark.parametrize("T", [0, 1, 63, 65])
@pytest.mark.parametrize("H", [32, 2])
def test_raw_short_and_empty(T, H):
    """Empty and short sequences on the whole-head shape (32 heads) and the
    sliced one (2 heads)."""
    w = Workload("raw-short", B=1, H=H, T=T, dk=128, dv=128, chunk=64, state0_std=0.3,
                 seed=500 + T + H)
    run_and_check(w)


def test_raw_zero_rows_and_saturated_logits():
    """Zero q and k rows (a zero vector stays zero) and gate / beta logits
    far in both tails of the sigmoid."""
    w = Workload("raw-edges", B=1, H=32, T=700, dk=128, dv=128, chunk=64, state0_std=0.3, seed=61)

    def edit(raw):
        raw["q"][0, 5:70:7] = 0.0
        raw["k"][0, 3:300:11] = 0.0
        raw["alpha"][0, 100:160] = 30.0     # gate 1 (no decay) over a chunk
        raw["alpha"][0, 400:410] = -30.0    # gate e^-30: the state is forgotten
        raw["beta"][0, 200:230] = -30.0     # no write
        raw["beta"][0, 500:530] = 30.0      # full write
    run_and_check(w, edit=edit)


@pytest.mark.parametrize("H", [32, 2])
def test_raw_in_place_state(H):
    w = Workload("raw-inplace", B=1, H=H, T=900, dk=128, dv=128, chunk=64, state0_std=0.3,
                 seed=70 + H)
    run_and_check(w, in_place=True)


def test_raw_timed_equals_plain():
    """gdn_chunk_fwd_raw_timed gives bit for bit the plain call's results and
    names the kernels it ran."""
    import torch
    w = Workload("raw-timed", B=1, H=32, T=1000, dk=128, dv=128, chunk=64, state0_std=0.3, seed=81)
    d = to_device(make_raw_inputs(w), w)
    o1, s1 = gdn.chunk_fwd_raw(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"])
    timer = gdn.Timer()
    o2, s2 = gdn.chunk_fwd_raw(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], timer=timer)
    torch.cuda.synchronize()
    names = set(timer.read())
    timer.close()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert {"k_prep_mfma", "k_seg_out"} <= names, names
