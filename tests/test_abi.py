"""Host-side checks of the C ABI (no GPU needed, no compute calls).

The library loads without a GPU; validation, workspace sizing, path
selection and status strings are host-only, and argument errors return
before any HIP call is made.
"""
import os
import re
import subprocess

import pytest

from gated_delta_rule_12_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(gdn_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    declared = header_functions()
    assert len(declared) >= 10
    assert set(declared) == set(gdn.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (gdn_\w+)", out))
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    L = gdn.lib()
    for f in declared:
        assert hasattr(L, f)


def test_abi_version_and_status_strings():
    assert gdn.gdn_abi_version() == 2
    for s in (gdn.GDN_OK, gdn.GDN_E_ARG, gdn.GDN_E_SHAPE, gdn.GDN_E_UNSUPPORTED,
              gdn.GDN_E_WORKSPACE, gdn.GDN_E_HIP, gdn.GDN_E_SCRATCH):
        assert gdn.gdn_status_str(s).startswith("GDN_")
    assert "unknown" in gdn.gdn_status_str(42)


@pytest.mark.parametrize("args,want", [
    ((1, 256, 1, 16, 16, 16, 0, 0, 0, 1), gdn.GDN_OK),
    ((2, 8192, 16, 128, 128, 64, 1, 0, 0, 1), gdn.GDN_OK),
    ((1, 65536, 4, 128, 128, 64, 1, 0, 1, 8), gdn.GDN_OK),
    ((8, 4096, 16, 128, 128, 64, 1, 1, 0, 1), gdn.GDN_OK),
    ((1, 0, 1, 64, 64, 64, 1, 0, 0, 1), gdn.GDN_OK),          # empty sequence
    ((0, 100, 3, 64, 64, 64, 1, 0, 0, 1), gdn.GDN_OK),        # empty batch
    ((1, 100, 1, 64, 64, 64, 2, 0, 0, 1), gdn.GDN_E_ARG),     # dtype
    ((1, 100, 1, 64, 64, 64, 1, 2, 0, 1), gdn.GDN_E_ARG),     # gate
    ((1, 100, 1, 64, 64, 64, 1, 0, 5, 1), gdn.GDN_E_ARG),     # order
    ((-1, 100, 1, 64, 64, 64, 1, 0, 0, 1), gdn.GDN_E_SHAPE),
    ((1, -5, 1, 64, 64, 64, 1, 0, 0, 1), gdn.GDN_E_SHAPE),
    ((1, 100, 1, 64, 64, 64, 1, 0, 0, 0), gdn.GDN_E_SHAPE),   # n_segments
    ((1, 100, 1, 60, 64, 64, 1, 0, 0, 1), gdn.GDN_E_UNSUPPORTED),
    ((1, 100, 1, 64, 256, 64, 1, 0, 0, 1), gdn.GDN_E_UNSUPPORTED),
    ((1, 100, 1, 64, 64, 128, 1, 0, 0, 1), gdn.GDN_E_UNSUPPORTED),
])
def test_validate(args, want):
    assert gdn.gdn_validate(*args) == want


def test_workspace_sizes():
    # zero for empty work or bad arguments
    assert gdn.gdn_workspace_bytes(1, 0, 1, 64, 64, 64, 1, 0, 1) == 0
    assert gdn.gdn_workspace_bytes(1, 100, 1, 60, 64, 64, 1, 0, 1) == 0
    a = gdn.gdn_workspace_bytes(2, 8192, 16, 128, 128, 64, 1, 0, 1)
    b = gdn.gdn_workspace_bytes(2, 8192, 16, 128, 128, 64, 1, 0, 8)
    c = gdn.gdn_workspace_bytes(2, 8192, 16, 128, 128, 64, 1, 0, 16)
    assert a > 0 and b >= a and c > b and a % 256 == 0 and b % 256 == 0
    # n_segments = 1 also covers gdn_chunk_fwd's own schedule
    g = gdn.gdn_chunk_segments(2, 8192, 16, 128, 128, 64, 1, 0)
    assert a >= gdn.gdn_workspace_bytes(2, 8192, 16, 128, 128, 64, 1, 0, g)
    # grows with the number of chunks; a ragged tail rounds up to a chunk
    assert gdn.gdn_workspace_bytes(1, 129, 1, 64, 64, 64, 1, 0, 1) == \
        gdn.gdn_workspace_bytes(1, 192, 1, 64, 64, 64, 1, 0, 1)
    assert gdn.gdn_workspace_bytes(1, 1024, 1, 64, 64, 64, 1, 0, 1) > \
        gdn.gdn_workspace_bytes(1, 512, 1, 64, 64, 64, 1, 0, 1)


def test_chunk_path_selection():
    for d in (16, 32, 64, 128):
        assert gdn.gdn_chunk_path(d, d, 16, gdn.GDN_F32, 0) == gdn.GDN_PATH_VALU
    assert gdn.gdn_chunk_path(60, 64, 64, gdn.GDN_BF16, 0) == gdn.GDN_E_UNSUPPORTED
    # bf16, dk = dv in {64, 128}, chunk 64, either gate: the MFMA kernels
    for d in (64, 128):
        for gate in (0, 1):
            assert gdn.gdn_chunk_path(d, d, 64, gdn.GDN_BF16, gate) == gdn.GDN_PATH_MFMA
    assert gdn.gdn_chunk_path(128, 128, 64, gdn.GDN_F32, 0) == gdn.GDN_PATH_VALU
    assert gdn.gdn_chunk_path(128, 128, 32, gdn.GDN_BF16, 0) == gdn.GDN_PATH_VALU
    assert gdn.gdn_chunk_path(128, 64, 64, gdn.GDN_BF16, 0) == gdn.GDN_PATH_VALU


def test_entry_points_reject_bad_arguments_before_any_launch():
    """Argument checks return a status and touch no device; here they run on
    a host with no GPU."""
    import ctypes
    nul = ctypes.c_void_p(0)
    ten = [nul] * 8
    # bad dtype
    rc = gdn.gdn_chunk_fwd(1, 64, 1, 64, 64, 64, 7, 0, 0, 1.0, *ten, nul, 0, nul)
    assert rc == gdn.GDN_E_ARG
    # unsupported shape
    rc = gdn.gdn_seqpar_fwd(1, 64, 1, 60, 64, 64, 1, 0, 0, 1.0, 2, *ten, nul, 0, nul)
    assert rc == gdn.GDN_E_UNSUPPORTED
    # missing input pointers
    rc = gdn.gdn_chunk_fwd(1, 64, 1, 64, 64, 64, 1, 0, 0, 1.0, *ten, nul, 0, nul)
    assert rc == gdn.GDN_E_ARG
    rc = gdn.gdn_recurrent_ref(1, 64, 1, 64, 64, 1, 0, 0, 1.0, *ten, nul)
    assert rc == gdn.GDN_E_ARG
    # workspace too small (non-null fake pointers never dereferenced on this path)
    fake = ctypes.c_void_p(0x1000)
    rc = gdn.gdn_chunk_fwd(1, 64, 1, 64, 64, 64, 1, 0, 0, 1.0, *([fake] * 8), fake, 16, nul)
    assert rc == gdn.GDN_E_WORKSPACE
    # empty batch: nothing to do
    rc = gdn.gdn_chunk_fwd(0, 64, 1, 64, 64, 64, 1, 0, 0, 1.0, *ten, nul, 0, nul)
    assert rc == gdn.GDN_OK


def test_binding_has_no_fallback(tmp_path, monkeypatch):
    monkeypatch.setattr(gdn, "_lib", None)
    monkeypatch.setattr(gdn, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        gdn.lib()


def test_chunk_schedule():
    # gdn_chunk_fwd cuts sequences into segments only on the whole-head MFMA
    # path (bf16, scalar gate), when B * H heads leave the device idle and the
    # segments give at least 128 (head, segment) workgroups
    seg = gdn.gdn_chunk_segments
    assert seg(2, 8192, 16, 128, 128, 64, 1, 0) == 8       # 32 heads x 8 segments
    assert seg(1, 65536, 4, 128, 128, 64, 1, 0) == 64      # 4 heads, 1024 chunks
    assert seg(64, 8192, 16, 128, 128, 64, 1, 0) == 1      # heads fill the device
    assert seg(1, 256, 1, 64, 64, 64, 1, 0) == 1           # 4 chunks: one segment
    assert seg(4, 1024, 8, 64, 64, 64, 1, 0) == 4          # at least 4 chunks each
    assert seg(1, 1024, 1, 64, 64, 64, 1, 0) == 1          # too few groups: one stream
    assert seg(8, 4096, 16, 128, 128, 64, 1, 1) == 1       # channel gate
    assert seg(1, 256, 1, 16, 16, 16, 0, 0) == 1           # fp32 vector-ALU path
    assert seg(1, 100, 1, 60, 64, 64, 1, 0) < 0            # bad shape


def test_seqpar_schedule():
    # an explicit split runs as asked, or, when its (batch, head, segment)
    # groups are too few for the whole-head MFMA loop, each segment cut into
    # k equal runs (about 256 groups, at least 4 chunks a segment)
    seg = gdn.gdn_seqpar_segments
    assert seg(1, 65536, 4, 128, 128, 64, 1, 0, 8) == 64     # 32 groups -> 8 x 8 segments
    assert seg(1, 65536, 4, 128, 128, 64, 1, 0, 64) == 64    # already 256 groups
    assert seg(2, 8192, 16, 128, 128, 64, 1, 0, 8) == 8      # 256 groups
    assert seg(2, 8192, 16, 128, 128, 64, 1, 0, 2) == 8      # 64 groups -> 2 x 4
    assert seg(1, 65536, 4, 128, 128, 64, 1, 0, 1) == 1      # a single stream stays one
    assert seg(1, 1000, 2, 64, 64, 64, 1, 0, 3) == 3         # 16 chunks: no finer cut
    assert seg(8, 4096, 16, 128, 128, 64, 1, 1, 4) == 4      # channel gate: as asked
    assert seg(1, 256, 1, 16, 16, 16, 0, 0, 4) == 4          # fp32 vector-ALU path
    assert seg(1, 100, 1, 60, 64, 64, 1, 0, 2) < 0           # bad shape
    # the workspace follows the segments actually run
    assert gdn.gdn_workspace_bytes(1, 65536, 4, 128, 128, 64, 1, 0, 8) == \
        gdn.gdn_workspace_bytes(1, 65536, 4, 128, 128, 64, 1, 0, 64)


def test_decode_step_rejects_bad_arguments_before_any_launch():
    """gdn_decode_step's checks return before anything is enqueued (fake,
    never dereferenced pointers)."""
    import ctypes
    nul = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)
    shape = (2, 4, 128, 128)
    tail = (gdn.GDN_BF16, gdn.GDN_GATE_SCALAR, gdn.GDN_PREDICT_THEN_DECAY, 1.0)
    ok_ptrs = [fake] * 8
    # state_out is required (both decode entry points)
    rc = gdn.gdn_decode_step(*shape, *tail, *ok_ptrs[:7], nul, nul)
    assert rc == gdn.GDN_E_ARG
    rc = gdn.gdn_decode_step_raw(*shape, *tail, *ok_ptrs[:7], nul, nul)
    assert rc == gdn.GDN_E_ARG
    rc = gdn.gdn_decode_step_raw(*shape, *tail, ctypes.c_void_p(0x1004), *ok_ptrs[1:], nul)
    assert rc == gdn.GDN_E_ARG
    # the state moves in 16-byte pieces
    rc = gdn.gdn_decode_step(*shape, *tail, *ok_ptrs[:5], ctypes.c_void_p(0x1008), fake, fake, nul)
    assert rc == gdn.GDN_E_ARG
    # bf16 q, k in 8-byte pieces; fp32 in 16-byte pieces
    rc = gdn.gdn_decode_step(*shape, *tail, ctypes.c_void_p(0x1004), *ok_ptrs[1:], nul)
    assert rc == gdn.GDN_E_ARG
    rc = gdn.gdn_decode_step(*shape, gdn.GDN_F32, *tail[1:], fake, ctypes.c_void_p(0x1008),
                             *ok_ptrs[2:], nul)
    assert rc == gdn.GDN_E_ARG
    # a vector gate in 16-byte pieces
    rc = gdn.gdn_decode_step(*shape, gdn.GDN_BF16, gdn.GDN_GATE_CHANNEL, *tail[2:], fake, fake,
                             fake, ctypes.c_void_p(0x1004), *ok_ptrs[4:], nul)
    assert rc == gdn.GDN_E_ARG
    # enums and sizes as for the other entry points
    rc = gdn.gdn_decode_step(*shape, 9, *tail[1:], *ok_ptrs, nul)
    assert rc == gdn.GDN_E_ARG
    rc = gdn.gdn_decode_step(2, 4, 60, 128, *tail, *ok_ptrs, nul)
    assert rc == gdn.GDN_E_UNSUPPORTED
    rc = gdn.gdn_decode_step(-1, 4, 128, 128, *tail, *ok_ptrs, nul)
    assert rc == gdn.GDN_E_SHAPE
    # empty batch: nothing to do
    rc = gdn.gdn_decode_step(0, 4, 128, 128, *tail, *([nul] * 8), nul)
    assert rc == gdn.GDN_OK


def test_forward_entry_points_check_alignment_and_segment_count():
    """16-byte pieces: misaligned tensors are refused before any launch; a
    segment count below one is a shape error (fake, never dereferenced
    pointers)."""
    import ctypes
    nul = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)
    odd16 = ctypes.c_void_p(0x1008)   # 8-byte, not 16-byte aligned
    odd4 = ctypes.c_void_p(0x1002)    # not 4-byte aligned
    shape = (1, 64, 1, 64, 64, 64, gdn.GDN_BF16, gdn.GDN_GATE_SCALAR, gdn.GDN_PREDICT_THEN_DECAY, 1.0)
    ok = [fake] * 8
    # an aligned call gets as far as the workspace check
    assert gdn.gdn_chunk_fwd(*shape, *ok, fake, 16, nul) == gdn.GDN_E_WORKSPACE
    for idx in (0, 1, 2, 5, 6, 7):            # q, k, v, state0, out, state_out
        ptrs = list(ok)
        ptrs[idx] = odd16
        assert gdn.gdn_chunk_fwd(*shape, *ptrs, fake, 16, nul) == gdn.GDN_E_ARG, idx
        assert gdn.gdn_seqpar_fwd(*shape, 2, *ptrs, fake, 16, nul) == gdn.GDN_E_ARG, idx
        assert gdn.gdn_recurrent_ref(1, 64, 1, 64, 64, *shape[6:], *ptrs, nul) == gdn.GDN_E_ARG, idx
    # beta and a scalar gate per float; a channel gate in 16-byte pieces
    for idx in (3, 4):
        ptrs = list(ok)
        ptrs[idx] = odd4
        assert gdn.gdn_chunk_fwd(*shape, *ptrs, fake, 16, nul) == gdn.GDN_E_ARG, idx
    ptrs = list(ok)
    ptrs[3] = odd16
    assert gdn.gdn_chunk_fwd(*shape, *ptrs, fake, 16, nul) == gdn.GDN_E_WORKSPACE
    chan = shape[:7] + (gdn.GDN_GATE_CHANNEL,) + shape[8:]
    assert gdn.gdn_chunk_fwd(*chan, *ptrs, fake, 16, nul) == gdn.GDN_E_ARG
    # the workspace moves in 16-byte pieces too
    assert gdn.gdn_chunk_fwd(*shape, *ok, odd16, 1 << 30, nul) == gdn.GDN_E_ARG
    # segment counts below one
    for n in (0, -3):
        assert gdn.gdn_seqpar_fwd(*shape, n, *ok, fake, 1 << 30, nul) == gdn.GDN_E_SHAPE


def test_backward_rejects_bad_arguments_before_any_launch():
    """gdn_backward's checks return before anything is enqueued (fake, never
    dereferenced pointers): required tensors, alignment, workspace size,
    enums and shapes."""
    import ctypes
    nul = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)
    odd16 = ctypes.c_void_p(0x1008)
    odd4 = ctypes.c_void_p(0x1002)
    B, T, H, dk, dv = 1, 100, 2, 64, 64
    head = (B, T, H, dk, dv, gdn.GDN_BF16, gdn.GDN_GATE_SCALAR, gdn.GDN_PREDICT_THEN_DECAY, 1.0)
    S, CH = gdn.GDN_GATE_SCALAR, gdn.GDN_GATE_CHANNEL
    # which algorithm runs: chunked for a scalar gate at dk = dv in {64, 128}
    assert gdn.gdn_backward_path(64, 64, S) == gdn.GDN_BWD_CHUNKED
    assert gdn.gdn_backward_path(128, 128, S) == gdn.GDN_BWD_CHUNKED
    assert gdn.gdn_backward_path(64, 128, S) == gdn.GDN_BWD_TOKEN
    assert gdn.gdn_backward_path(32, 32, S) == gdn.GDN_BWD_TOKEN
    assert gdn.gdn_backward_path(64, 64, CH) == gdn.GDN_BWD_TOKEN
    assert gdn.gdn_backward_path(60, 64, S) < 0
    assert gdn.gdn_backward_path(64, 64, 5) < 0
    need = gdn.gdn_backward_workspace_bytes(B, T, H, dk, dv, S)
    # chunked: per (batch, head) and chunk of 64 tokens T, T^T, P^T, Atilde^T
    # (64 x 64), K^T and Q^T fragments (64 x dk each), the entry state, the
    # state gradient and scale Q^T diag(gamma) dO (dk x dv each), U, Delta,
    # dDelta, dU', scale P^T dO (64 x dv each) and eight gate rows of 64, fp32;
    # fifteen pieces
    nc = (T + 63) // 64
    assert need == 4 * B * H * nc * (4 * 64 * 64 + 2 * 64 * dk + 3 * dk * dv + 5 * 64 * dv + 8 * 64) + 15 * 256
    # token: a checkpoint at every 16-token run start per (batch, head), and
    # per block of 32 rows (16 lanes a row at dk = 64) a record of 2 dk + 4
    # floats per token
    align = lambda x: (x + 255) // 256 * 256
    dv2 = 128
    ckpt = 4 * dk * dv2 * 7 * B * H
    part = 4 * B * H * (dv2 // 32) * T * (2 * dk + 4)
    assert gdn.gdn_backward_workspace_bytes(B, T, H, dk, dv2, S) == align(ckpt) + align(part)
    chan = gdn.gdn_backward_workspace_bytes(B, T, H, dk, dv, CH)
    ckpt = 4 * dk * dv * 7 * B * H
    assert chan == align(ckpt) + align(4 * B * H * (dv // 32) * T * (3 * dk + 4))
    assert gdn.gdn_backward_workspace_bytes(B, T, H, 60, dv, 0) == 0
    assert gdn.gdn_backward_workspace_bytes(B, T, H, dk, dv, 5) == 0
    ok = [fake] * 14  # q k v alpha beta state0 dout dstate dq dk dv dalpha dbeta dstate0

    def call(ptrs, ws=fake, nbytes=need, head=head):
        return gdn.gdn_backward(*head, *ptrs, ws, nbytes, nul)

    # an aligned call gets past every check but the workspace size
    assert call(ok, nbytes=need - 1) == gdn.GDN_E_WORKSPACE
    assert call(ok, ws=nul) == gdn.GDN_E_WORKSPACE
    # required tensors (state0, dstate and dstate0 are optional)
    for idx in (0, 1, 2, 3, 4, 6, 8, 9, 10, 11, 12):
        ptrs = list(ok)
        ptrs[idx] = nul
        assert call(ptrs) == gdn.GDN_E_ARG, idx
    # 16-byte pieces: states, dq, dk and the workspace; 8-byte: bf16 q, k;
    # per element: the rest
    for idx in (5, 7, 8, 9, 13):
        ptrs = list(ok)
        ptrs[idx] = odd16
        assert call(ptrs) == gdn.GDN_E_ARG, idx
    assert call(ok, ws=odd16) == gdn.GDN_E_ARG
    for idx in (0, 1):
        ptrs = list(ok)
        ptrs[idx] = ctypes.c_void_p(0x1004)
        assert call(ptrs) == gdn.GDN_E_ARG, idx
    for idx in (3, 4, 6, 8, 9, 10, 11, 12):
        ptrs = list(ok)
        ptrs[idx] = odd4
        assert call(ptrs) == gdn.GDN_E_ARG, idx
    chan_head = head[:6] + (gdn.GDN_GATE_CHANNEL,) + head[7:]
    ptrs = list(ok)
    ptrs[3] = odd16
    assert call(ptrs, head=chan_head, nbytes=chan) == gdn.GDN_E_ARG
    ptrs = list(ok)
    ptrs[11] = odd16  # a channel gate's gradient goes out in 16-byte pieces too
    assert call(ptrs, head=chan_head, nbytes=chan) == gdn.GDN_E_ARG
    # a channel gate needs its own workspace
    assert call(ok, head=chan_head, nbytes=chan - 1) == gdn.GDN_E_WORKSPACE
    # the chunked path reads dL/d out in 16-byte pieces, the token path per float
    ptrs = list(ok)
    ptrs[6] = odd16
    assert call(ptrs) == gdn.GDN_E_ARG
    assert call(ptrs, head=chan_head, nbytes=chan - 1) == gdn.GDN_E_WORKSPACE
    # enums and sizes
    assert call(ok, head=head[:5] + (7,) + head[6:]) == gdn.GDN_E_ARG
    assert call(ok, head=head[:7] + (5,) + head[8:]) == gdn.GDN_E_ARG
    assert call(ok, head=(1, 100, 2, 72, 64) + head[5:]) == gdn.GDN_E_UNSUPPORTED
    assert call(ok, head=(1, -1, 2, 64, 64) + head[5:]) == gdn.GDN_E_SHAPE
    # empty batch: nothing to do
    assert gdn.gdn_backward(0, T, H, dk, dv, *head[5:], *([nul] * 14), nul, 0, nul) == gdn.GDN_OK


def test_timer_is_a_caller_owned_object():
    """Per-kernel timing lives in a timer the caller creates, passes to the
    *_timed entry points and destroys; an empty timer reads nothing, a
    timed call that fails its argument checks records nothing."""
    t = gdn.Timer()
    assert t.read() == {}
    L = gdn.lib()
    # bad dtype: rejected on the host before any launch or event
    rc = L.gdn_chunk_fwd_timed(1, 64, 1, 64, 64, 64, 7, 0, 0, 1.0, None, None, None, None, None,
                               None, None, None, None, 0, None, t.handle)
    assert rc == gdn.GDN_E_ARG
    assert t.read() == {}
    t2 = gdn.Timer()
    assert t2.handle.value != t.handle.value
    t.close()
    t2.close()
    assert L.gdn_timer_destroy(None) == gdn.GDN_OK
    assert L.gdn_timer_read(None, 0, None, 0, None, None) == gdn.GDN_E_ARG


def test_no_mutable_globals_in_the_library():
    """The library keeps no state between calls: its writable data sections
    hold only what the HIP runtime registers (code-object handles and the
    host stubs of the kernels) and, for gdn_chunk_fwd_noalloc, the host-side
    stand-in of its static device scratch and the per-device cache of that
    array's device address."""
    out = subprocess.run(["nm", "-C", "--defined-only", gdn.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    runtime = re.compile(r"^(__hip_|__do_init|__do_fini|__dso_handle|__init|__fini|_DYNAMIC|"
                         r"_GLOBAL_OFFSET_TABLE_|DW\.ref\.)")
    own = []
    for ln in out.splitlines():
        parts = ln.split(None, 2)
        if len(parts) < 3 or parts[1] not in "bBdD" or "(" in parts[2].replace("(anonymous namespace)", ""):
            continue
        if not runtime.match(parts[2]):
            own.append(parts[2])
    assert sorted(own) == ["(anonymous namespace)::g_scratch_addr", "(anonymous namespace)::scratch"], own


def test_noalloc_refuses_problems_past_the_scratch_on_the_host():
    """The size check runs on the host before any HIP call (no GPU needed)."""
    rc = gdn.lib().gdn_chunk_fwd_noalloc(8, 4096, 16, 128, 128, 64, gdn.GDN_BF16,
                                         gdn.GDN_GATE_CHANNEL, 0, 1.0, None, None, None, None,
                                         None, None, None, None, None)
    assert rc == gdn.GDN_E_SCRATCH
    assert gdn.gdn_workspace_bytes(2, 8192, 16, 128, 128, 64, gdn.GDN_BF16, 0, 1) <= gdn.GDN_NOALLOC_SCRATCH_BYTES
