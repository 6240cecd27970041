"""GPU parity: the HIP path (through the C ABI) against the oracle.

Every case is compared element by element over every (batch, head) slice:
small cases that span several chunks and a ragged tail, and the full-size
workloads in the launch configuration bench.py times (the oracle, OpenMP over
the slices, takes about a second on each).  Only the tensors past 2^31
elements, drawn on the device, are compared on sampled slices.
"""
import numpy as np
import pytest

from gated_delta_rule_12_amd import gdn
from gated_delta_rule_12_amd.workloads import WORKLOADS, Workload, make_inputs, to_device
from parity import TOL, oracle_on, out_err, state_err

pytestmark = pytest.mark.gpu

PTD, DTP = gdn.GDN_PREDICT_THEN_DECAY, gdn.GDN_DECAY_THEN_PREDICT


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()


def _np(t):
    return t.detach().float().cpu().numpy()


def run(w, inp, entry="chunk", order=PTD, n_segments=None):
    d = to_device(inp, w)
    if entry == "recurrent":
        o, s = gdn.recurrent_ref(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"],
                                 order=order)
    else:
        # None: gdn_chunk_fwd (the library's schedule)
        G = (w.n_segments if w.n_segments > 1 else None) if n_segments is None else n_segments
        o, s = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"],
                             chunk=w.chunk, order=order, n_segments=G)
    import torch
    torch.cuda.synchronize()
    return _np(o), _np(s)


def check(w, inp, o, s, order=PTD, bh=None, tol=None):
    o_ref, s_ref = oracle_on(inp, w.gate, order, bh)
    if bh is not None:
        o = np.stack([o[b, :, h:h + 1] for b, h in bh])
        s = np.stack([s[b, h] for b, h in bh])[:, None]
    to, ts = tol or TOL[w.dtype]
    eo, es = out_err(o, o_ref), state_err(s, s_ref)
    print(f"  {w.name}: out err {eo:.3e} (tol {to}), state err {es:.3e} (tol {ts})", flush=True)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert eo <= to, eo
    assert es <= ts, es
    return eo, es


# --------------------------------------------------------------------------
# the tiny fp32 workload, all entry points
# --------------------------------------------------------------------------

@pytest.mark.parametrize("entry", ["chunk", "recurrent", "seqpar"])
@pytest.mark.parametrize("order", [PTD, DTP])
def test_tiny_f32_workload(entry, order):
    w = WORKLOADS[0]
    inp = make_inputs(w)
    o, s = run(w, inp, entry if entry != "seqpar" else "chunk", order,
               n_segments=4 if entry == "seqpar" else None)
    check(w, inp, o, s, order)


# --------------------------------------------------------------------------
# random shapes: several chunks, ragged tail, nonzero start state
# --------------------------------------------------------------------------

CASES = [
    # dtype, dk, dv, chunk, T, gate, order
    ("f32", 16, 16, 16, 200, "scalar", PTD),
    ("f32", 32, 48, 32, 133, "channel", DTP),
    ("f32", 64, 64, 64, 300, "scalar", DTP),
    ("f32", 128, 128, 64, 190, "channel", PTD),
    ("bf16", 16, 32, 16, 77, "channel", PTD),
    ("bf16", 64, 64, 64, 257, "scalar", PTD),
    ("bf16", 64, 64, 64, 320, "channel", DTP),
    ("bf16", 128, 128, 64, 449, "scalar", DTP),
    ("bf16", 128, 128, 64, 384, "scalar", PTD),
    ("bf16", 128, 128, 64, 129, "channel", PTD),
    ("bf16", 96, 112, 32, 100, "scalar", PTD),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("entry", ["chunk", "recurrent"])
def test_random_shapes(case, entry):
    dtype, dk, dv, C, T, gate, order = case
    w = Workload("rand", B=2, H=3, T=T, dk=dk, dv=dv, chunk=C, dtype=dtype, gate=gate,
                 state0_std=0.5, seed=100 + dk + T)
    inp = make_inputs(w)
    o, s = run(w, inp, entry, order)
    check(w, inp, o, s, order)


@pytest.mark.parametrize("gate,alpha_mean", [
    ("scalar", 6.0), ("scalar", -1.0), ("scalar", -6.0),
    ("channel", 6.0), ("channel", -1.0), ("channel", -3.0), ("channel", -6.0)])
def test_gate_extremes(gate, alpha_mean):
    """Long memory (alpha ~ 0.998) to fast forgetting (alpha ~ 0.0025).  With
    per-channel gates at -3 a 16-token block decays by ~e^-48 per channel;
    at -6 by ~e^-96, past the range where the block is factored."""
    w = Workload("gates", B=1, H=2, T=512, dk=128, dv=128, chunk=64, state0_std=0.5,
                 gate=gate, alpha_mean=alpha_mean, seed=7)
    inp = make_inputs(w)
    o, s = run(w, inp)
    check(w, inp, o, s)
    o, s = run(w, inp, order=DTP)
    check(w, inp, o, s, DTP)


# --------------------------------------------------------------------------
# sequence parallel split
# --------------------------------------------------------------------------

@pytest.mark.parametrize("G", [1, 2, 3, 4, 8, 40])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_seqpar_segments(G, gate):
    w = Workload("seqpar", B=1, H=2, T=1000, dk=64, dv=64, chunk=64, gate=gate,
                 state0_std=0.5, seed=11 + G)
    inp = make_inputs(w)
    o, s = run(w, inp, n_segments=G)
    check(w, inp, o, s)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_seqpar_segments_span_several_correction_runs(gate):
    """Segments of 24 chunks (the correction takes runs of chunks of one
    segment) with a ragged last chunk."""
    w = Workload("seqpar-runs", B=1, H=2, T=4500, dk=64, dv=64, chunk=64, gate=gate,
                 state0_std=0.5, seed=77)
    inp = make_inputs(w)
    o, s = run(w, inp, n_segments=3)
    check(w, inp, o, s)


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T", [0, 1, 5, 63, 64, 65])
@pytest.mark.parametrize("entry", ["chunk", "recurrent", "seqpar"])
def test_short_sequences(T, entry):
    w = Workload("short", B=2, H=2, T=T, dk=128, dv=128, chunk=64, state0_std=0.5, seed=3)
    inp = make_inputs(w)
    o, s = run(w, inp, "recurrent" if entry == "recurrent" else "chunk",
               n_segments=3 if entry == "seqpar" else 1)
    if T == 0:
        np.testing.assert_array_equal(s, inp["state0"])
        assert o.shape == (2, 0, 2, 128)
    else:
        check(w, inp, o, s)


def test_empty_batch():
    import torch
    z = torch.zeros((0, 16, 2, 64), dtype=torch.bfloat16, device="cuda")
    a = torch.zeros((0, 16, 2), dtype=torch.float32, device="cuda")
    o, s = gdn.chunk_fwd(z, z, z, a, a)
    assert o.shape == (0, 16, 2, 64) and s.shape == (0, 2, 64, 64)


def test_zero_start_state_equals_null():
    import torch
    w = Workload("z", B=1, H=2, T=256, dk=128, dv=128, chunk=64, seed=5)
    d = to_device(make_inputs(w), w)
    o1, s1 = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], None)
    zero = torch.zeros((1, 2, 128, 128), dtype=torch.float32, device="cuda")
    o2, s2 = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], zero)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_streaming_equals_one_call():
    """Two calls with the state threaded through equal one call (resume)."""
    import torch
    w = Workload("stream", B=2, H=2, T=512, dk=128, dv=128, chunk=64, state0_std=0.3, seed=9)
    inp = make_inputs(w)
    d = to_device(inp, w)
    o, s = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"])
    cut = 192
    part = lambda x, a, b: x[:, a:b].contiguous()
    o1, s1 = gdn.chunk_fwd(*(part(d[n], 0, cut) for n in ("q", "k", "v", "alpha", "beta")),
                           d["state0"])
    o2, s2 = gdn.chunk_fwd(*(part(d[n], cut, 512) for n in ("q", "k", "v", "alpha", "beta")),
                           s1)
    torch.cuda.synchronize()
    oo = torch.cat([o1, o2], dim=1)
    assert (oo - o).abs().max().item() <= 1e-5 * o.abs().max().item()
    assert (s2 - s).abs().max().item() <= 1e-5 * s.abs().max().item()


@pytest.mark.parametrize("B,H,T,d,G,gate", [
    (1, 2, 300, 64, None, "scalar"),     # sliced path, one stream
    (1, 2, 1000, 64, 3, "scalar"),       # sliced path, increment-and-correct
    (1, 32, 1000, 128, None, "scalar"),  # whole-head path, library schedule (4 segments)
    (1, 32, 2000, 64, 8, "scalar"),      # whole-head path, 8 segments, d = 64
    (16, 16, 700, 128, None, "scalar"),  # whole-head path, one pass
    (4, 16, 700, 128, None, "channel"),  # channel gate, head-shared loop
])
def test_in_place_state(B, H, T, d, G, gate):
    """state_out == state0 (in-place streaming) on every path: the last
    segment's final state may not overwrite the start state before segment 0
    has read it."""
    import torch
    w = Workload("inplace", B=B, H=H, T=T, dk=d, dv=d, chunk=64, state0_std=0.3, gate=gate, seed=13 + T)
    inp = make_inputs(w)
    d_ = to_device(inp, w)
    st = d_["state0"].clone()
    o, s = gdn.chunk_fwd(d_["q"], d_["k"], d_["v"], d_["alpha"], d_["beta"], st, state_out=st,
                         n_segments=G)
    torch.cuda.synchronize()
    check(w, inp, _np(o), _np(st))


def test_two_streams_interleaved():
    """The library keeps no state between calls: calls enqueued on two
    streams at once (each with its own workspace) give bit for bit the
    results of the same calls made one after the other."""
    import torch
    wa = Workload("streams-a", B=2, H=16, T=1024, dk=128, dv=128, chunk=64, state0_std=0.3, seed=21)
    wb = Workload("streams-b", B=1, H=3, T=700, dk=64, dv=64, chunk=64, gate="channel",
                  state0_std=0.3, seed=22)
    da, db = to_device(make_inputs(wa), wa), to_device(make_inputs(wb), wb)
    args = lambda d: (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"])
    ref_a = gdn.chunk_fwd(*args(da))
    ref_b = gdn.seqpar_fwd(*args(db), n_segments=3)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    res = []
    for _ in range(3):
        oa = torch.empty_like(ref_a[0]); sa = torch.empty_like(ref_a[1])
        ob = torch.empty_like(ref_b[0]); sb = torch.empty_like(ref_b[1])
        wsa = gdn.workspace_for(da["q"], da["v"], da["alpha"])
        wsb = gdn.workspace_for(db["q"], db["v"], db["alpha"], n_segments=3)
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            gdn.chunk_fwd(*args(da), out=oa, state_out=sa, workspace=wsa)
        with torch.cuda.stream(s2):
            gdn.seqpar_fwd(*args(db), n_segments=3, out=ob, state_out=sb, workspace=wsb)
        torch.cuda.synchronize()
        res.append((oa, sa, ob, sb))
    for oa, sa, ob, sb in res:
        assert torch.equal(oa, ref_a[0]) and torch.equal(sa, ref_a[1])
        assert torch.equal(ob, ref_b[0]) and torch.equal(sb, ref_b[1])


def test_timed_calls_equal_plain_calls():
    """The *_timed entry points run the same kernels: identical results, and
    the timer names every kernel of the path with one launch per call."""
    import torch
    w = Workload("timed", B=2, H=16, T=1024, dk=128, dv=128, chunk=64, state0_std=0.3, seed=23)
    d = to_device(make_inputs(w), w)
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"])
    o1, s1 = gdn.chunk_fwd(*args)
    t = gdn.Timer()
    o2, s2 = gdn.chunk_fwd(*args, timer=t)
    o3, s3 = gdn.chunk_fwd(*args, timer=t)
    torch.cuda.synchronize()
    rec = t.read()
    t.close()
    assert torch.equal(o1, o2) and torch.equal(s1, s2) and torch.equal(o1, o3)
    assert set(rec) == {"k_prep_mfma", "k_seg_state", "k_chain", "k_seg_out"}, rec
    assert all(cnt == 2 and ms > 0 for ms, cnt in rec.values()), rec


def test_deterministic():
    import torch
    w = Workload("det", B=2, H=4, T=1024, dk=128, dv=128, chunk=64, state0_std=0.3, seed=17)
    d = to_device(make_inputs(w), w)
    r1 = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"])
    r2 = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"])
    r3 = gdn.seqpar_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], n_segments=4)
    r4 = gdn.seqpar_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], n_segments=4)
    torch.cuda.synchronize()
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])
    assert torch.equal(r3[0], r4[0]) and torch.equal(r3[1], r4[1])


def test_workspace_too_small_is_an_error():
    import torch
    w = Workload("ws", B=1, H=1, T=128, dk=64, dv=64, chunk=64, seed=1)
    d = to_device(make_inputs(w), w)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(gdn.GdnError) as ei:
        gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], workspace=ws)
    assert ei.value.status == gdn.GDN_E_WORKSPACE


# --------------------------------------------------------------------------
# full-size workloads (bench launch configuration), every slice
# --------------------------------------------------------------------------

# --------------------------------------------------------------------------
# whole-head chunk loop (scalar gate, at least 128 (head, segment) groups):
# two passes and the start-state chain, every head against the oracle
# --------------------------------------------------------------------------

WHOLE = [
    # B, H, T, d, G (None: gdn_chunk_fwd's schedule), order, state0_std, alpha_mean
    (1, 32, 1000, 128, 4, PTD, 0.5, 2.0),    # ragged tail, 4 chunks per segment
    (1, 32, 1050, 128, 5, DTP, 0.5, 2.0),    # last segment a single ragged chunk (its stage 1
                                             # in the state pass: one group of the pair idle)
    (1, 32, 700, 64, 4, DTP, 0.3, 2.0),
    (1, 64, 640, 128, 2, PTD, 0.5, 2.0),     # two segments: no chain step; the last
                                             # segment's five chunks end on an odd pair
    (2, 16, 2000, 128, None, PTD, 0.5, 2.0),  # library schedule (7 segments)
    (1, 32, 512, 128, 4, PTD, 0.0, 6.0),     # long memory, zero start state
    (1, 32, 512, 128, 4, DTP, 0.5, -6.0),    # fast forgetting
    (1, 20, 2048, 128, 8, PTD, 0.5, 2.0),    # head count not a multiple of 8
    # 16 maps and more: the start-state chain as a two-level scan over blocks
    (1, 16, 4608, 64, 18, PTD, 0.3, 6.0),    # 4 blocks of 4 maps, long memory
    (1, 8, 5120, 128, 20, PTD, 0.5, 6.0),    # blocks of 5, 5, 5, 3 maps
    (1, 4, 10240, 128, 40, DTP, 0.5, 6.0),   # blocks of 7 (x5) and 3, 4 heads
    # one chunk per segment: a scan over the per-chunk affine maps, ragged tail
    (1, 4, 4128, 128, 65, PTD, 0.5, 6.0),
]


@pytest.mark.parametrize("case", WHOLE, ids=lambda c: "-".join(map(str, c)))
def test_whole_head_path(case):
    B, H, T, d, G, order, std, am = case
    w = Workload("whole", B=B, H=H, T=T, dk=d, dv=d, chunk=64, state0_std=std,
                 alpha_mean=am, seed=T + H + d)
    if G is None:
        assert gdn.gdn_chunk_segments(B, T, H, d, d, 64, gdn.GDN_BF16, gdn.GDN_GATE_SCALAR) * B * H >= 128
    inp = make_inputs(w)
    o, s = run(w, inp, order=order, n_segments=G)
    check(w, inp, o, s, order)


@pytest.mark.parametrize("B,H,T,d,order", [
    (16, 16, 700, 128, PTD),   # 256 heads: one segment, ragged last chunk
    (8, 20, 256, 64, DTP),     # 160 heads, four chunks: too short to split
])
def test_whole_head_single_pass(B, H, T, d, order):
    """Enough heads to fill the device: gdn_chunk_fwd runs stage 1 and one
    pass of the whole-head chunk loop (no state pass, no chain)."""
    assert gdn.gdn_chunk_segments(B, T, H, d, d, 64, gdn.GDN_BF16, gdn.GDN_GATE_SCALAR) == 1
    assert gdn.gdn_chunk_path(d, d, 64, gdn.GDN_BF16, gdn.GDN_GATE_SCALAR) == gdn.GDN_PATH_MFMA
    w = Workload("single-pass", B=B, H=H, T=T, dk=d, dv=d, chunk=64, state0_std=0.3, seed=T + H + d)
    inp = make_inputs(w)
    o, s = run(w, inp, order=order)
    check(w, inp, o, s, order)


# --------------------------------------------------------------------------
# head-shared chunk loop (channel gate, dk = 128, at least 64 heads, one
# pass): two workgroups per head, each forming the gated rows once per chunk
# for its four waves of 16 value columns
# --------------------------------------------------------------------------

CHAN_HEAD = [
    # B, H, T, order, state0_std, alpha_mean
    (4, 16, 300, PTD, 0.5, 2.0),     # ragged tail; 64 heads, XCD placement
    (2, 32, 257, DTP, 0.5, 2.0),     # one token in the last chunk
    (5, 13, 130, PTD, 0.3, 2.0),     # 65 heads, not a multiple of 8
    (8, 8, 64, DTP, 0.0, 6.0),       # exactly one chunk, zero start state, long memory
    (1, 64, 1, PTD, 0.5, 2.0),       # one token
    (4, 16, 512, PTD, 0.5, -3.0),    # fast forgetting
    (4, 16, 512, DTP, 0.5, -6.0),    # stage 1 sums the diagonal blocks directly
]


@pytest.mark.parametrize("case", CHAN_HEAD, ids=lambda c: "-".join(map(str, c)))
def test_channel_head_shared(case):
    import torch
    B, H, T, order, std, am = case
    w = Workload("chan-head", B=B, H=H, T=T, dk=128, dv=128, chunk=64, gate="channel",
                 state0_std=std, alpha_mean=am, seed=31 + T + H)
    inp = make_inputs(w)
    d = to_device(inp, w)
    t = gdn.Timer()
    o, s = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], chunk=64,
                         order=order, timer=t)
    torch.cuda.synchronize()
    rec = t.read()
    t.close()
    assert set(rec) == {"k_prep_mfma", "k_chan_head"}, rec
    check(w, inp, _np(o), _np(s), order)


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_full_workload(idx):
    """The workloads at full size, every (batch, head) slice."""
    w = WORKLOADS[idx]
    inp = make_inputs(w)
    o, s = run(w, inp)
    check(w, inp, o, s)


def test_long_workload_library_schedule():
    """The long workload through gdn_chunk_fwd: the library cuts its four
    sequences into 64 segments (whole-head path, blocked start-state chain)."""
    import torch
    w = WORKLOADS[3]
    assert gdn.gdn_chunk_segments(w.B, w.T, w.H, w.dk, w.dv, w.chunk, gdn.GDN_BF16,
                                  gdn.GDN_GATE_SCALAR) == 64
    inp = make_inputs(w)
    d = to_device(inp, w)
    o, s = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], chunk=w.chunk)
    torch.cuda.synchronize()
    check(w, inp, _np(o), _np(s))


def test_long_workload_single_stream():
    """The long workload through the single-stream entry point as well."""
    w = WORKLOADS[3]
    inp = make_inputs(w)
    o, s = run(w, inp, n_segments=1)
    check(w, inp, o, s)


# --------------------------------------------------------------------------
# maximum sizes: more than 2^31 elements per tensor (64-bit offsets)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_tensors_past_2_31_elements(gate):
    """9 x 65536 x 32 x 128 = 2.4e9 elements in q, k, v and O (scalar gate:
    the whole-head path, 288 heads in one pass; channel gate: the
    head-shared path); heads whose data lie past element 2^31 checked
    against the oracle."""
    import torch
    from gated_delta_rule_12_amd.workloads import make_inputs_device, slice_inputs
    w = Workload("large", B=9, H=32, T=65536, dk=128, dv=128, chunk=64, gate=gate,
                 state0_std=0.02, seed=777)
    assert w.B * w.T * w.H * w.dk > 2 ** 31
    d = make_inputs_device(w)
    o, s = gdn.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], chunk=w.chunk)
    torch.cuda.synchronize()
    bh = [(8, 31), (8, 0), (4, 17)]   # (8, 31) holds the last elements of every tensor
    inp = slice_inputs(d, bh)
    ow = np.stack([o[b, :, h].cpu().numpy() for b, h in bh])[:, :, None]
    sw = np.stack([s[b, h].cpu().numpy() for b, h in bh])[:, None]
    del o, s, d
    torch.cuda.empty_cache()
    ws = w.with_(B=len(bh), H=1)
    check(ws, inp, ow, sw)
