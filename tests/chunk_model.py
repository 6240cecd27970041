"""Chunk-form model of the gated delta rule in fp64 numpy — a test helper.

This is NOT the oracle (the oracle is the token loop in ``oracle/``).  It is
the chunkwise WY/UT algorithm written plainly, one chunk at a time, so that
the tests can (1) pin the oracle against an independent formulation the pages
give, and (2) check the chunk, state-passing and sequence-parallel algebra the
HIP kernels implement, stage by stage, on the CPU.

Sources:
  * DeltaNet illustrated notes (stay-hungry-time.github.io/deltanet), WY/UT
    section: A_tj = -beta_t k_t.k_j for j < t, T = (I - A)^{-1},
    U = T diag(beta) V, W = T diag(beta) K, chunk state passing
    S_[i+1] = S_[i](I - W^T K) + U^T K, output
    O = Q S^T + ((Q K^T) (.) M)(U - W S^T), M lower-triangular with diagonal.
  * same notes, GLA gating section: chunk-local gate prefixes b_t, the gated
    scores (Q (.) B)(K / B)^T, the boundary key K (.) (b_C / B) and the entry
    history read (Q (.) B) S^T.
  * How to Implement Sequence Parallelism in DeltaNet (papercache notes),
    "parallel algorithm" derivation: zero-start increment state S^D, scaling
    matrix M_[i+1] = M_[i](I - W^T K) from M = I, correction S = S^D + S_start M.

With gates the per-chunk transition is Diag(b_C) - W^T Kbar instead of
I - W^T K (it reduces to the pages' form when every gate is 1).
"""
from __future__ import annotations

import numpy as np


def _gate_table(alpha_c, dk):
    """Chunk-local prefix table B (C x dk): row t is prod_{u<=t} alpha_u."""
    a = np.asarray(alpha_c, dtype=np.float64)
    if a.ndim == 1:
        a = np.repeat(a[:, None], dk, axis=1)
    return np.cumprod(a, axis=0)


def chunk_stage(qc, kc, vc, alpha_c, beta_c, order):
    """Per-chunk quantities that do not depend on the entry state.

    Returns dict with B (prefixes), Bp (prefix used by the prediction),
    Tp = T diag(beta), U, W, P (gated causal scores incl. diagonal), Kbar.
    """
    C, dk = kc.shape
    B = _gate_table(alpha_c, dk)
    ones = np.ones((1, dk))
    Bprev = np.vstack([ones, B[:-1]])
    Bp = Bprev if order == 0 else B
    # L_tj = sum_a k_ta b'_ta k_ja / b_ja for j < t
    L = np.tril((kc * Bp) @ (kc / B).T, -1)
    A = np.eye(C) + beta_c[:, None] * L
    T = np.linalg.inv(A)
    Tp = T * beta_c[None, :]
    U = Tp @ vc
    W = Tp @ (kc * Bp)
    P = np.tril((qc * B) @ (kc / B).T)
    Kbar = kc * (B[-1][None, :] / B)
    return dict(B=B, Bp=Bp, Tp=Tp, U=U, W=W, P=P, Kbar=Kbar, L=L)


def chunk_step(st, qc, S):
    """Output of one chunk and the next state, given the entry state S."""
    delta = st["U"] - st["W"] @ S.T
    out = (qc * st["B"]) @ S.T + st["P"] @ delta
    S_next = S * st["B"][-1][None, :] + delta.T @ st["Kbar"]
    return out, S_next, delta


def chunk_transition(st):
    """Affine map of a chunk, S_next = S @ Acal + Bcal."""
    dk = st["W"].shape[1]
    Acal = np.diag(st["B"][-1]) - st["W"].T @ st["Kbar"]
    Bcal = st["U"].T @ st["Kbar"]
    assert Acal.shape == (dk, dk)
    return Acal, Bcal


def forward(q, k, v, alpha, beta, S0, chunk, order=0):
    """Chunkwise forward of one (batch, head) sequence: q,k [T,dk], v [T,dv].

    alpha [T] or [T,dk]; beta [T]; S0 [dv,dk].  The last chunk may be short.
    """
    T = q.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    out = np.zeros((T, v.shape[1]))
    for i0 in range(0, T, chunk):
        sl = slice(i0, min(i0 + chunk, T))
        st = chunk_stage(q[sl], k[sl], v[sl], alpha[sl], beta[sl], order)
        out[sl], S, _ = chunk_step(st, q[sl], S)
    return out, S


def seqpar_forward(q, k, v, alpha, beta, S0, chunk, n_segments, order=0):
    """Increment-and-correct over contiguous, chunk-aligned segments.

    Segment 0 runs from the true start state.  Every later segment runs the
    increment state S^D from zero and the scaling matrix M from I; outputs are
    corrected with R_i S_start^T where R_i = ((Q (.) B) - P W) M_[i]^T, which
    is the output operator applied to S_start M_[i] (outputs are linear in the
    entry state), and the start states are chained
    S_start(g+1) = S^D_end(g) + S_start(g) M_end(g).
    """
    T, dk = k.shape
    dv = v.shape[1]
    nc = T // chunk
    assert nc * chunk == T and nc % n_segments == 0
    per = nc // n_segments
    out = np.zeros((T, dv))
    ends = []
    corr = []
    for g in range(n_segments):
        S = np.array(S0, dtype=np.float64) if g == 0 else np.zeros((dv, dk))
        M = None if g == 0 else np.eye(dk)
        R_list = []
        for i in range(g * per, (g + 1) * per):
            sl = slice(i * chunk, (i + 1) * chunk)
            st = chunk_stage(q[sl], k[sl], v[sl], alpha[sl], beta[sl], order)
            o, S, _ = chunk_step(st, q[sl], S)
            out[sl] = o
            if M is not None:
                R_list.append(((q[sl] * st["B"]) - st["P"] @ st["W"]) @ M.T)
                Acal, _ = chunk_transition(st)
                M = M @ Acal
        ends.append((S, M))
        corr.append(R_list)
    S_start = None
    for g in range(n_segments):
        S_end, M_end = ends[g]
        if g == 0:
            S_start = S_end
            continue
        for j, R in enumerate(corr[g]):
            i = g * per + j
            sl = slice(i * chunk, (i + 1) * chunk)
            out[sl] += R @ S_start.T
        S_start = S_end + S_start @ M_end
    return out, S_start
