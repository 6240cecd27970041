"""The chunk-level backward (``oracle.chunked``, the equations the chunked
backward kernels follow) against the token-level chain rule
(``oracle.backward``, pinned by finite differences of the forward oracle):
both gate orders, ragged and one-token sequences, small and long-memory
gates, with and without start state and final-state gradient."""
import numpy as np
import pytest

import oracle
from oracle.chunked import chunk_backward
from gated_delta_rule_12_amd.workloads import Workload, make_grads, make_inputs

PTD, DTP = 0, 1

CASES = [
    # T, dk, dv, order, state0_std, alpha_mean, with dL/dS_T, chunk
    (150, 32, 32, PTD, 0.3, 2.0, True, 64),    # two chunks and a ragged third
    (150, 32, 48, DTP, 0.3, 2.0, True, 64),    # dk != dv
    (200, 16, 16, PTD, 0.0, 6.0, True, 64),    # no start state, long memory
    (64, 16, 16, DTP, 0.5, 2.0, False, 64),    # exactly one chunk, no final gradient
    (5, 16, 16, PTD, 0.5, 2.0, True, 64),      # shorter than a chunk
    (1, 16, 16, DTP, 0.5, 2.0, True, 64),      # one token
    (129, 32, 32, DTP, 0.3, -3.0, True, 64),   # small gates
    (96, 16, 32, PTD, 0.3, -1.0, True, 16),    # another chunk length
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_chunk_backward_equals_token_backward(case):
    T, dk, dv, order, std, am, with_ds, C = case
    w = Workload("cb", B=1, H=2, T=T, dk=dk, dv=dv, chunk=C, dtype="bf16", state0_std=std,
                 alpha_mean=am, seed=900 + T + dk + dv)
    inp = make_inputs(w)
    gr = make_grads(w, with_state=with_ds)
    args = (inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["state0"], gr["dout"], gr["dstate"])
    ref = oracle.backward(*args, order=order, scale=0.8)
    got = chunk_backward(*args, order=order, scale=0.8, chunk=C)
    for name, x, r in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dstate0"), got, ref):
        err = np.abs(x - r).max() / max(np.abs(r).max(), 1e-300)
        assert err <= 1e-12, (name, err)
