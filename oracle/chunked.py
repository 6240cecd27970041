"""Chunk-level backward of the gated delta rule (scalar gate) — TEST
INFRASTRUCTURE ONLY (the same rules as the rest of ``oracle``: only tests may
import it; it shares no code with the HIP library).

The pages fix the forward recurrence and its chunk form (DeltaNet illustrated
notes, WY/UT section: the UT transform, chunk state passing and the output;
GLA gating section: gate prefixes; the scalar gate of the Gated DeltaNet
paragraph); they print no gradient.  ``chunk_backward`` writes out the chain
rule through that chunk form in fp64 numpy, the equations the chunked backward
kernels follow, so that the chunk algebra (every sign, index and triangular
mask) is checked against ``oracle.backward`` (the token-level chain rule,
itself pinned by finite differences) before any kernel runs.

Per chunk of C tokens with entry state S (dv x dk): the log-gate prefix
l_t = sum_{s <= t} log alpha_s (gamma_t = e^{l_t}), the prediction prefix
l'_t (l_{t-1} predict-then-decay, l_t decay-then-predict), R_t = e^{l_{C-1} - l_t}:

    Atilde_tj = e^{l'_t - l_j} k_t.k_j (j < t),   A = diag(beta) Atilde,   T = (I + A)^{-1}
    U = V - diag(gamma') K S^T,   Delta = T diag(beta) U
    O = scale (diag(gamma) Q S^T + P Delta),   P_tj = e^{l_t - l_j} q_t.k_j (j <= t)
    S_end = gamma_{C-1} S + Delta^T diag(R) K

Backward, given dO and dS_end:

    dDelta = scale P^T dO + diag(R) K dS_end^T,   dU' = T^T dDelta,   dv = diag(beta) dU'
    dS = gamma_{C-1} dS_end + scale dO^T diag(gamma) Q - dU'^T diag(gamma' beta) K
    dP = scale dO Delta^T (j <= t),   dT = dDelta U^T diag(beta),   dA = -T^T dT T^T (j < t)
    dq = scale diag(gamma) dO S + (dP o M) K,   M_tj = e^{l_t - l_j} (j <= t)
    dk = (dP o M)^T Q - diag(gamma' beta) dU' S + diag(R) Delta dS_end + (W + W^T) K,
         W_tj = beta_t dA_tj e^{l'_t - l_j}
    dbeta_t = dU'_t . U_t + sum_j dA_tj Atilde_tj

and the gate: every gate product above is a ratio e^{l_b - l_a} over the
tokens a < s <= b (a = -1 for a product from the chunk start), whose
derivative in log alpha_s is the term itself, so dlog alpha_s is the sum of
the terms whose range holds s — the pair terms dP_tj P_tj (range (j, t]) and
dA_tj A_tj (range (j, t']), t' = t or t - 1 by the order) and the boundary
terms q_t . (scale gamma_t dO_t S) (range (-1, t]), k_t . (-gamma'_t beta_t
dU'_t S) (range (-1, t']), R_j k_j . (Delta_j dS_end) (range (j, C - 1]) and
gamma_{C-1} <dS_end, S> (range (-1, C - 1]) — and dalpha_s = dlog alpha_s / alpha_s.
A short last chunk is padded with tokens that neither decay nor write.
"""
from __future__ import annotations

import numpy as np

PREDICT_THEN_DECAY = 0
DECAY_THEN_PREDICT = 1


def _head(q, k, v, a, b, s0, do, dst, order, scale, C):
    """One (batch, head) pair: q, k [T, dk], v, do [T, dv], a, b [T];
    s0, dst [dv, dk] or None."""
    T, dk = q.shape
    dv = v.shape[1]
    nc = (T + C - 1) // C
    S = np.zeros((dv, dk)) if s0 is None else s0.copy()
    chunks = []
    # forward over the chunks: each chunk's entry state and pieces
    for c in range(nc):
        sl = slice(c * C, min(T, (c + 1) * C))
        Q, K, V, al, be = q[sl], k[sl], v[sl], a[sl], b[sl]
        n = len(al)
        l = np.cumsum(np.log(al))
        lp = l if order == DECAY_THEN_PREDICT else np.concatenate([[0.0], l[:-1]])
        strict = np.tril(np.ones((n, n)), -1)
        lower = np.tril(np.ones((n, n)))
        Et = np.exp(lp[:, None] - l[None, :]) * strict
        At = Et * (K @ K.T)
        Tm = np.linalg.inv(np.eye(n) + be[:, None] * At)
        U = V - np.exp(lp)[:, None] * (K @ S.T)
        Dl = Tm @ (be[:, None] * U)
        M = np.exp(l[:, None] - l[None, :]) * lower
        P = M * (Q @ K.T)
        R = np.exp(l[-1] - l)
        chunks.append(dict(sl=sl, Q=Q, K=K, be=be, al=al, l=l, lp=lp, Et=Et, At=At, Tm=Tm,
                           U=U, Dl=Dl, M=M, P=P, R=R, S=S.copy(), n=n))
        S = np.exp(l[-1]) * S + Dl.T @ (R[:, None] * K)
    dq = np.zeros_like(q)
    dkk = np.zeros_like(k)
    dvv = np.zeros_like(v)
    da = np.zeros_like(a)
    db = np.zeros_like(b)
    dS = np.zeros((dv, dk)) if dst is None else dst.copy()
    # backward over the chunks, carrying the state gradient
    for ch in reversed(chunks):
        Q, K, be, l, lp, R, S0, n = ch["Q"], ch["K"], ch["be"], ch["l"], ch["lp"], ch["R"], ch["S"], ch["n"]
        dO = do[ch["sl"]]
        gam, gamp = np.exp(l), np.exp(lp)
        dD = scale * ch["P"].T @ dO + R[:, None] * (K @ dS.T)
        dUp = ch["Tm"].T @ dD
        dU = be[:, None] * dUp
        dP = np.tril(scale * dO @ ch["Dl"].T)
        dPm = dP * ch["M"]
        dT = dD @ (be[:, None] * ch["U"]).T
        dA = np.tril(-ch["Tm"].T @ dT @ ch["Tm"].T, -1)
        W = be[:, None] * dA * ch["Et"]
        dQ_S = scale * gam[:, None] * (dO @ S0)
        dK_S = -(gamp * be)[:, None] * (dUp @ S0)
        dK_dS = R[:, None] * (ch["Dl"] @ dS)
        dq[ch["sl"]] = dQ_S + dPm @ K
        dkk[ch["sl"]] = dPm.T @ Q + dK_S + dK_dS + (W + W.T) @ K
        dvv[ch["sl"]] = dU
        db[ch["sl"]] = np.sum(dUp * ch["U"], axis=1) + np.sum(dA * ch["At"], axis=1)
        # gate terms by range (a, b]: column a + 1 (0 for the chunk start), row b
        V = np.zeros((n, n + 1))
        V[:, 1:] += np.tril(dP * ch["P"], -1)
        VA = dA * (be[:, None] * ch["At"])
        vx = np.sum(K * dK_S, axis=1)
        if order == DECAY_THEN_PREDICT:
            V[:, 1:] += VA
            V[:, 0] += vx
        else:
            V[:-1, 1:] += VA[1:]
            V[:-1, 0] += vx[1:]
        V[:, 0] += np.sum(Q * dQ_S, axis=1)
        V[n - 1, 1:] += np.sum(K * dK_dS, axis=1)
        V[n - 1, 0] += np.exp(l[-1]) * np.sum(dS * S0)
        dlog = np.array([V[s:, :s + 1].sum() for s in range(n)])
        da[ch["sl"]] = dlog / ch["al"]
        dS = np.exp(l[-1]) * dS + scale * dO.T @ (gam[:, None] * Q) - dU.T @ (gamp[:, None] * K)
    return dq, dkk, dvv, da, db, dS


def chunk_backward(q, k, v, alpha, beta, state0, dout, dstate=None, *,
                   order: int = PREDICT_THEN_DECAY, scale: float = 1.0, chunk: int = 64):
    """The gradients ``oracle.backward`` returns (scalar gate), through the
    chunk form: q, k [B,T,H,dk], v, dout [B,T,H,dv], alpha, beta [B,T,H],
    state0, dstate [B,H,dv,dk] or None.  Returns (dq, dk, dv, dalpha, dbeta,
    dstate0) as float64 arrays."""
    f = lambda x: None if x is None else np.asarray(x, dtype=np.float64)
    q, k, v, alpha, beta, dout = (f(x) for x in (q, k, v, alpha, beta, dout))
    s0, dst = f(state0), f(dstate)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(alpha),
           np.zeros_like(beta), np.zeros((B, H, dv, dk))]
    for bb in range(B):
        for h in range(H):
            r = _head(q[bb, :, h], k[bb, :, h], v[bb, :, h], alpha[bb, :, h], beta[bb, :, h],
                      None if s0 is None else s0[bb, h], dout[bb, :, h],
                      None if dst is None else dst[bb, h], order, scale, chunk)
            for i in range(5):
                out[i][bb, :, h] = r[i]
            out[5][bb, h] = r[5]
    return tuple(out)
