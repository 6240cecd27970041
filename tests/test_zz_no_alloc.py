"""gdn_chunk_fwd_noalloc (workspace in the library's static device scratch)
against gdn_chunk_fwd with a caller workspace: identical results, on two
calls in a row, the second with a smaller input; a problem larger than the
scratch is refused before anything is enqueued."""
import pytest

from gated_delta_rule_12_amd import gdn
from gated_delta_rule_12_amd.workloads import WORKLOADS, Workload, make_inputs, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()


def _args(d):
    return d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"]


def test_noalloc_equals_chunk_fwd_on_two_calls():
    import torch
    big = WORKLOADS[2]   # main-bf16: 100.25 MiB of workspace, whole-head path, 8 segments
    small = Workload("noalloc-small", B=1, H=3, T=300, dk=64, dv=64, chunk=64, state0_std=0.3, seed=31)
    results = []
    for w in (big, small):
        d = to_device(make_inputs(w), w)
        ref = gdn.chunk_fwd(*_args(d), chunk=w.chunk)
        got = gdn.chunk_fwd_noalloc(*_args(d), chunk=w.chunk)
        torch.cuda.synchronize()
        results.append((w.name, ref, got))
    for name, (o_ref, s_ref), (o, s) in results:
        print(f"  {name}: max |out diff| {(o - o_ref).abs().max().item():.3e}", flush=True)
        assert torch.equal(o, o_ref), name
        assert torch.equal(s, s_ref), name


def test_noalloc_refuses_problems_past_the_scratch():
    import torch
    w = WORKLOADS[4]    # channel gate, 448 MiB of workspace
    dt, g = gdn.GDN_BF16, gdn.GDN_GATE_CHANNEL
    assert gdn.gdn_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, w.chunk, dt, g, 1) > gdn.GDN_NOALLOC_SCRATCH_BYTES
    L = gdn.lib()
    rc = L.gdn_chunk_fwd_noalloc(w.B, w.T, w.H, w.dk, w.dv, w.chunk, dt, g, 0, 1.0,
                                 None, None, None, None, None, None, None, None, None)
    assert rc == gdn.GDN_E_SCRATCH
    assert "static scratch" in gdn.gdn_status_str(rc)
