"""Error metric and oracle helpers shared by the GPU parity tests.

Metric (per (batch, head) slice, maxed over slices): max|X - R| / max|R| for
the output [T, dv] and for the final state [dv, dk].  Tolerances are the
ones stated for this path: bf16 inputs (fp32 state) 2e-3 on the output and
1e-3 on the state; fp32 inputs 1e-5 on both.
"""
from __future__ import annotations

import numpy as np

import oracle

TOL = {"bf16": (2e-3, 1e-3), "f32": (1e-5, 1e-5)}


def rel_err(x, r, axes):
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    num = np.abs(x - r).max(axis=axes)
    den = np.abs(r).max(axis=axes)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if num.size else 0.0


def out_err(o, o_ref):
    """o: [B,T,H,dv] -> slices over (T, dv)."""
    if o.shape[1] == 0:
        return 0.0
    return rel_err(o, o_ref, axes=(1, 3))


def state_err(s, s_ref):
    return rel_err(s, s_ref, axes=(2, 3))


def oracle_on(inp: dict, gate: str, order: int, bh=None, threads=0):
    """Run the oracle on all (b, h) pairs, or only on the listed ones.
    Returns (out, state) restricted to those pairs: out [n,T,1,dv]."""
    g = oracle.GATE_SCALAR if gate == "scalar" else oracle.GATE_CHANNEL
    if bh is None:
        return oracle.forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                              inp["state0"], gate=g, order=order, threads=threads)
    outs, states = [], []
    for b, h in bh:
        sl = lambda x: None if x is None else x[b:b + 1, :, h:h + 1]
        s0 = None if inp["state0"] is None else inp["state0"][b:b + 1, h:h + 1]
        o, s = oracle.forward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["alpha"]),
                              sl(inp["beta"]), s0, gate=g, order=order, threads=threads)
        outs.append(o[0])
        states.append(s[0])
    return np.stack(outs), np.stack(states)
