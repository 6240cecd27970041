"""The roofline accounting of bench.py against the per-unit figures it
states (host only, no GPU): algorithmic bytes per head-token and per head,
and the flop count per chunk-head, for the five workloads and the decode and
backward lines."""
import bench
from gated_delta_rule_12_amd.workloads import DECODE_WORKLOAD, workload


def test_forward_bytes_and_flops():
    w = workload("main-bf16")
    # bf16 q, k, v (3 x 128 x 2), alpha and beta (8), O in fp32 (512) per
    # head-token; start and final state (2 x 64 KiB) per head
    per_ht = 3 * 128 * 2 + 8 + 4 * 128
    assert bench.algorithmic_bytes(w) == per_ht * 2 * 8192 * 16 + 2 * 4 * 128 * 128 * 2 * 16
    assert round(bench.algorithmic_bytes(w) / 1e6, 1) == 341.8
    # 5 C^2 d + 6 C d^2 + C^3 / 3 per chunk-head, 4096 chunk-heads
    assert bench.algorithmic_flops(w) == 4096 * (5 * 64 * 64 * 128 + 6 * 64 * 128 * 128 + 64 ** 3 / 3)
    # a per-channel gate reads dk floats of alpha per head-token (in place of
    # the scalar one): q, k, v + beta + alpha + O
    c = workload("channel-gate-bf16")
    assert bench.algorithmic_bytes(c) == (3 * 128 * 2 + 4 + 4 * 128 + 4 * 128) * 8 * 4096 * 16 \
        + 4 * 128 * 128 * 8 * 16
    # fp32 inputs: 4 bytes per q, k, v element; no start state
    t = workload("tiny-f32")
    assert bench.algorithmic_bytes(t) == (3 * 16 * 4 + 8 + 4 * 16) * 256 + 4 * 16 * 16


def test_decode_and_backward_bytes():
    w = DECODE_WORKLOAD
    # state read and written (8 dk dv), the token's q, k, v, alpha, beta, o
    assert bench.decode_bytes(w) == (8 * 128 * 128 + 3 * 128 * 2 + 4 + 4 + 4 * 128) * 256 * 16
    m = workload("main-bf16")
    # read q, k, v, alpha, beta, dL/dout; write dq, dk, dv, dalpha, dbeta;
    # per head S_0 and dL/dS_T read, dL/dS_0 written
    per_ht = 3 * 128 * 2 + 4 + 4 + 4 * 128 + 8 * 128 + 4 * 128 + 4 + 4
    assert bench.backward_bytes(m) == per_ht * 2 * 8192 * 16 + 12 * 128 * 128 * 2 * 16
