"""Pins for the oracle: what the pages and the mathematics fix, independently
of the oracle's own loop.

Each test names the passage it relies on.  A plausible mistake in the oracle
(read before the update, prediction after instead of before the decay, a
transposed state, gates on rows instead of key columns, a dropped beta, a
wrong sign in the correction) fails at least one of them:

* printed worked examples (tests/golden/*.txt, each with its citation);
* closed forms: beta = 0 (pure decay), orthogonal keys (decayed linear
  attention in its parallel form), unit keys (interpolation identity);
* the per-token affine maps and their associative composition;
* the WY product identity for two Householder-like factors;
* the chunkwise WY/UT algorithm (an independent formulation) and the
  increment-and-correct split;
* linearity in (V, S0);
* exact rational arithmetic on tiny dyadic inputs.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from chunk_model import forward as chunk_forward
from chunk_model import seqpar_forward
from conftest import read_golden

PTD = oracle.PREDICT_THEN_DECAY
DTP = oracle.DECAY_THEN_PREDICT


def run1(q, k, v, alpha, beta, S0=None, gate=0, order=PTD):
    """Oracle on one (batch, head) sequence: q,k [T,dk], v [T,dv]."""
    q = np.asarray(q, float)[None, :, None, :]
    k = np.asarray(k, float)[None, :, None, :]
    v = np.asarray(v, float)[None, :, None, :]
    a = np.asarray(alpha, float)
    a = a[None, :, None] if gate == 0 else a[None, :, None, :]
    b = np.asarray(beta, float)[None, :, None]
    s0 = None if S0 is None else np.asarray(S0, float)[None, None]
    o, s = oracle.forward(q, k, v, a, b, s0, gate=gate, order=order)
    return o[0, :, 0, :], s[0, 0]


def rand_seq(rng, T, dk, dv, gate=0, unit=True):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    if unit:
        q /= np.linalg.norm(q, axis=1, keepdims=True)
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    shape = (T,) if gate == 0 else (T, dk)
    alpha = 1.0 / (1.0 + np.exp(-rng.normal(2.0, 0.5, shape)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    S0 = 0.3 * rng.standard_normal((dv, dk))
    return q, k, v, alpha, beta, S0


# --------------------------------------------------------------------------
# printed worked examples
# --------------------------------------------------------------------------

@pytest.mark.parametrize("order", [PTD, DTP])
def test_printed_vector_delta_example(order):
    g = read_golden("delta_rule_vector_example.txt")
    T = 3
    o, _ = run1([g["q"]] * T, [g["k"]] * T, [g["v"]] * T, g["alpha"] * T,
                g["beta"] * T, order=order)
    np.testing.assert_allclose(o, [g["out1"], g["out2"], g["out3"]], rtol=0, atol=1e-15)


def test_printed_scalar_delta_example():
    g = read_golden("delta_rule_scalar_example.txt")
    ones = [[1.0]] * 3
    o, _ = run1(ones, [g["k"]] * 3, [g["v"]] * 3, [1.0] * 3, [0.5] * 3)
    np.testing.assert_allclose(o[:, 0], g["beta_half"], atol=1e-15)
    o, _ = run1(ones, [g["k"]] * 3, [g["v"]] * 3, [1.0] * 3, [1.0] * 3)
    np.testing.assert_allclose(o[:, 0], g["beta_one"], atol=1e-15)


def test_printed_prediction_error_example():
    g = read_golden("prediction_error_example.txt")
    S0 = np.array(g["S0"]).reshape(2, 2)
    k = np.array(g["k"])
    # beta = 0, no forgetting: the read with q = k is the prediction itself
    o, s = run1([k], [k], [g["v"]], [1.0], [0.0], S0=S0)
    np.testing.assert_allclose(o[0], g["prediction"], atol=1e-15)
    # beta = 1, unit key: the state moves by error k^T, so it reads v
    o, s = run1([k], [k], [g["v"]], [1.0], [1.0], S0=S0)
    np.testing.assert_allclose(o[0] - np.array(g["prediction"]), g["error"], atol=1e-15)
    np.testing.assert_allclose(s - S0, np.outer(g["error"], k), atol=1e-15)


def test_printed_gdn_gate_example():
    """Decay-then-predict reproduces 3.7; predict-then-decay (the recurrence
    S_t = a S + b (v - S k) k^T of the Gated DeltaNet blog, section 1.2) gives
    0.8*3 + 0.5*(5-3) = 3.4 on the same numbers."""
    g = read_golden("gdn_gate_example.txt")
    S0 = [[g["old_prediction"][0]]]
    args = ([[1.0]], [[1.0]], [g["target"]], g["alpha"], g["beta"])
    o, _ = run1(*args, S0=S0, order=DTP)
    assert o[0, 0] == pytest.approx(g["new_prediction"][0], abs=1e-14)
    o, _ = run1(*args, S0=S0, order=PTD)
    a, b, p, v = g["alpha"][0], g["beta"][0], g["old_prediction"][0], g["target"][0]
    assert o[0, 0] == pytest.approx(a * p + b * (v - p), abs=1e-14)
    assert abs(o[0, 0] - 3.4) < 1e-14


@pytest.mark.parametrize("order", [PTD, DTP])
def test_printed_kda_forgetting(order):
    g = read_golden("kda_example.txt")
    S0 = np.array(g["S0"]).reshape(2, 2)
    alpha = np.array(g["alpha"])
    qA, qB = [1.0, 0.0], [0.0, 1.0]
    # one step with no write (beta = 0), read with q_A then q_B
    for q, want in ((qA, g["read_qA"]), (qB, g["read_qB"])):
        o, s = run1([q], [[0.0, 1.0]], [[0.0, 0.0]], [alpha], [0.0], S0=S0,
                    gate=1, order=order)
        np.testing.assert_allclose(s, np.array(g["forget_once"]).reshape(2, 2), atol=1e-14)
        np.testing.assert_allclose(o[0], want, atol=1e-14)
    qm = np.array([1.0, 1.0]) / np.sqrt(2.0)
    o, _ = run1([qm], [[0.0, 1.0]], [[0.0, 0.0]], [alpha], [0.0], S0=S0, gate=1, order=order)
    np.testing.assert_allclose(o[0], np.array([9.0, 4.0]) / np.sqrt(2.0), atol=1e-14)
    o, s = run1([qA] * 3, [[0.0, 1.0]] * 3, [[0.0, 0.0]] * 3, [alpha] * 3, [0.0] * 3,
                S0=S0, gate=1, order=order)
    np.testing.assert_allclose(s, np.array(g["forget_thrice"]).reshape(2, 2), atol=1e-13)


def test_printed_kda_update_decay_then_predict():
    g = read_golden("kda_example.txt")
    S0 = np.array(g["S0"]).reshape(2, 2)
    o, s = run1([[0.0, 1.0]], [g["k"]], [g["v"]], [g["alpha"]], g["beta"], S0=S0,
                gate=1, order=DTP)
    np.testing.assert_allclose(s, np.array(g["after_update"]).reshape(2, 2), atol=1e-14)
    assert o[0, 1] == pytest.approx(6.0, abs=1e-14)
    # predict-then-decay on the same numbers predicts from the undecayed
    # column (20), error 8 - 20 = -12, half of it written: diag(9, -2)
    o, s = run1([[0.0, 1.0]], [g["k"]], [g["v"]], [g["alpha"]], g["beta"], S0=S0,
                gate=1, order=PTD)
    np.testing.assert_allclose(s, [[9.0, 0.0], [0.0, -2.0]], atol=1e-14)


@pytest.mark.parametrize("order", [PTD, DTP])
def test_printed_gla_gate_prefix(order):
    """A single write at step 1 read at step 3 carries the gate ratio b3/b1."""
    g = read_golden("gla_gate_prefix_example.txt")
    a = g["alpha_scalar"]
    assert np.prod(a[:1]) == pytest.approx(g["b1"][0])
    assert np.prod(a) == pytest.approx(g["b3"][0])
    q = [[0.0], [0.0], g["q3_scalar"]]
    k = [g["k1_scalar"], [0.0], [0.0]]
    o, _ = run1(q, k, [[1.0], [0.0], [0.0]], a, [1.0, 0.0, 0.0], order=order)
    assert o[2, 0] == pytest.approx(g["score_scalar"][0], abs=1e-15)
    # two channels: gates chosen so that b3/b1 = (0.1, 0.125), b3 = (0.05, 0.1)
    alpha = np.array([[0.5, 0.8], [0.2, 0.25], [0.5, 0.5]])
    np.testing.assert_allclose(alpha.prod(0), g["b3_vec"], atol=1e-15)
    np.testing.assert_allclose(alpha[1:].prod(0), g["ratio_vec"], atol=1e-15)
    q = [[0.0, 0.0], [0.0, 0.0], g["q3"]]
    k = [g["k1"], [0.0, 0.0], [0.0, 0.0]]
    o, _ = run1(q, k, [[1.0], [0.0], [0.0]], alpha, [1.0, 0.0, 0.0], gate=1, order=order)
    assert o[2, 0] == pytest.approx(g["score_vec"][0], abs=1e-14)


def test_printed_wy_example():
    g = read_golden("wy_example.txt")
    args = ([[1.0]], [g["k"]], [g["v"]], [1.0], g["beta"])
    o, s = run1(*args)
    assert s[0, 0] == pytest.approx(g["S1_zero_start"][0], abs=1e-15)
    assert s[0, 0] == pytest.approx(g["u"][0], abs=1e-15)
    o, s = run1(*args, S0=[g["entry"]])
    assert s[0, 0] == pytest.approx(g["S1_from_entry"][0], abs=1e-15)
    assert s[0, 0] == pytest.approx(g["entry"][0] * g["P1"][0] + g["u"][0], abs=1e-15)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("order", [PTD, DTP])
def test_beta_zero_is_pure_decay(gate, order):
    """beta = 0: S_t = S_0 Diag(b_t), o_t = S_0 (b_t (.) q_t) (GLA gating
    section: the entry history read through the gate prefix)."""
    rng = np.random.default_rng(1)
    T, dk, dv = 20, 5, 3
    q, k, v, alpha, beta, S0 = rand_seq(rng, T, dk, dv, gate)
    o, s = run1(q, k, v, alpha, np.zeros(T), S0=S0, gate=gate, order=order)
    a = alpha if gate == 1 else np.repeat(alpha[:, None], dk, 1)
    b = np.cumprod(a, axis=0)
    np.testing.assert_allclose(o, (S0 @ (b * q).T).T, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(s, S0 * b[-1][None, :], rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("order", [PTD, DTP])
def test_axis_keys_give_decayed_linear_attention(gate, order):
    """Zero start and distinct axis-aligned keys: no key predicts another, so
    the delta rule writes beta_t v_t k_t^T and the output is decayed linear
    attention in the parallel form of the GLA gating section:
    O = (((Q (.) B)(K / B)^T) (.) M) diag(beta) V, M lower incl. diagonal."""
    rng = np.random.default_rng(2)
    T = dk = 8
    dv = 3
    q, _, v, alpha, beta, _ = rand_seq(rng, T, dk, dv, gate)
    perm = rng.permutation(dk)
    k = np.eye(dk)[perm] * rng.uniform(0.5, 2.0, (T, 1))
    o, _ = run1(q, k, v, alpha, beta, gate=gate, order=order)
    a = alpha if gate == 1 else np.repeat(alpha[:, None], dk, 1)
    Bt = np.cumprod(a, axis=0)
    scores = np.tril((q * Bt) @ (k / Bt).T)
    np.testing.assert_allclose(o, scores @ (beta[:, None] * v), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("order", [PTD, DTP])
def test_unit_key_interpolation(order):
    """DeltaNet section: with ||k|| = 1, S_t k_t = (1 - beta) vhat + beta v,
    vhat the prediction; with beta = 1 the key reads v exactly."""
    rng = np.random.default_rng(3)
    dk, dv = 6, 4
    for _ in range(10):
        q, k, v, alpha, beta, S0 = rand_seq(rng, 1, dk, dv)
        a = alpha[0]
        vhat = (a * S0 if order == DTP else S0) @ k[0]
        o, s = run1(k, k, v, alpha, beta, S0=S0, order=order)
        keep = a * S0 @ k[0] if order == PTD else vhat
        want = keep + beta[0] * (v[0] - vhat)
        np.testing.assert_allclose(o[0], want, rtol=1e-13, atol=1e-14)
        o, s = run1(k, k, v, [1.0], [1.0], S0=S0, order=order)
        np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-13)


def test_unit_keys_overwrite_along_sequence():
    """alpha = beta = 1 and unit keys: after every token S_t k_t = v_t."""
    rng = np.random.default_rng(4)
    T, dk, dv = 40, 8, 5
    q, k, v, _, _, S0 = rand_seq(rng, T, dk, dv)
    o, _ = run1(k, k, v, np.ones(T), np.ones(T), S0=S0)
    np.testing.assert_allclose(o, v, atol=1e-12)


def test_wy_two_factor_identity():
    """WY/UT section: H1 H2 = I - w1 k1^T - w2 k2^T with w1 = b1 k1,
    w2 = b2 (k2 - (k1.k2) w1), H_t = I - b_t k_t k_t^T; the old state is
    multiplied on the right, so from S_0 = I with zero values S_2 = H1 H2."""
    rng = np.random.default_rng(5)
    d = 5
    k = rng.standard_normal((2, d))
    b = np.array([0.3, 0.9])
    w1 = b[0] * k[0]
    w2 = b[1] * (k[1] - (k[0] @ k[1]) * w1)
    want = np.eye(d) - np.outer(w1, k[0]) - np.outer(w2, k[1])
    _, s = run1(np.zeros((2, d)), k, np.zeros((2, d)), [1.0, 1.0], b, S0=np.eye(d))
    np.testing.assert_allclose(s, want, rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------
# affine maps and their composition (Gated DeltaNet blog, sections 2.2-2.3, 3.3)
# --------------------------------------------------------------------------

def token_map(alpha_t, beta_t, k_t, v_t, order):
    """Blog section 2.2 in the d_k x d_v orientation: X_t = A_t X_{t-1} + B_t
    with X = S^T.  Predict-then-decay: A_t = D_t - beta k k^T (D_t =
    alpha_t.diag(), section 3.3 allows a vector alpha); decay-then-predict:
    A_t = (I - beta k k^T) D_t.  B_t = beta k v^T."""
    dk = k_t.shape[0]
    D = np.diag(np.broadcast_to(alpha_t, (dk,)).astype(float))
    kk = np.outer(k_t, k_t)
    A = D - beta_t * kk if order == PTD else (np.eye(dk) - beta_t * kk) @ D
    return A, beta_t * np.outer(k_t, v_t)


def compose(nxt, prv):
    """compose((A_n, B_n), (A_p, B_p)) = (A_n A_p, A_n B_p + B_n)."""
    return nxt[0] @ prv[0], nxt[0] @ prv[1] + nxt[1]


@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("order", [PTD, DTP])
def test_chunk_affine_maps_compose_to_token_loop(gate, order):
    rng = np.random.default_rng(6)
    T, dk, dv, C = 48, 6, 4, 8
    q, k, v, alpha, beta, S0 = rand_seq(rng, T, dk, dv, gate)
    chunks = []
    for i0 in range(0, T, C):
        acc = (np.eye(dk), np.zeros((dk, dv)))
        for t in range(i0, i0 + C):
            acc = compose(token_map(alpha[t], beta[t], k[t], v[t], order), acc)
        chunks.append(acc)
    # sequential scan of chunk maps: state at every chunk boundary
    acc = None
    for i, ch in enumerate(chunks):
        acc = ch if acc is None else compose(ch, acc)
        X = acc[0] @ S0.T + acc[1]
        T_i = (i + 1) * C
        _, s = run1(q[:T_i], k[:T_i], v[:T_i], alpha[:T_i], beta[:T_i], S0=S0,
                    gate=gate, order=order)
        np.testing.assert_allclose(X.T, s, rtol=1e-11, atol=1e-12)
    # associativity: a tree-ordered reduction gives the same total map
    level = list(chunks)
    while len(level) > 1:
        level = [compose(level[i + 1], level[i]) if i + 1 < len(level) else level[i]
                 for i in range(0, len(level), 2)]
    np.testing.assert_allclose(level[0][0], acc[0], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(level[0][1], acc[1], rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------
# chunkwise WY/UT algorithm and the increment-and-correct split
# --------------------------------------------------------------------------

@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("order", [PTD, DTP])
@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_chunk_form_matches_token_loop(gate, order, C):
    """WY/UT section (chunk state passing and output) and GLA gating section
    (gate prefixes): C = 1 is the token recurrence, C = T the parallel form."""
    rng = np.random.default_rng(7 + C)
    T, dk, dv = 64, 8, 5
    q, k, v, alpha, beta, S0 = rand_seq(rng, T, dk, dv, gate)
    o_ref, s_ref = run1(q, k, v, alpha, beta, S0=S0, gate=gate, order=order)
    o, s = chunk_forward(q, k, v, alpha, beta, S0, C, order)
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(s, s_ref, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_increment_and_correct_matches_token_loop(gate, G):
    """Sequence parallelism notes: S = S^D + S_start M with M from I."""
    rng = np.random.default_rng(30 + G)
    T, dk, dv, C = 128, 6, 4, 8
    q, k, v, alpha, beta, S0 = rand_seq(rng, T, dk, dv, gate)
    o_ref, s_ref = run1(q, k, v, alpha, beta, S0=S0, gate=gate)
    o, s = seqpar_forward(q, k, v, alpha, beta, S0, C, G)
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(s, s_ref, rtol=1e-10, atol=1e-12)


def test_seqpar_difference_identity():
    """S_[i+k] - S^D_[i+k] = (S_[i] - S^D_[i]) prod (I - W^T K): with all gates 1
    the per-chunk factor is exactly the pages' I - W^T K."""
    from chunk_model import chunk_stage, chunk_step
    rng = np.random.default_rng(8)
    T, dk, dv, C = 64, 5, 3, 8
    q, k, v, _, beta, S0 = rand_seq(rng, T, dk, dv)
    alpha = np.ones(T)
    S, SD, prod = S0.copy(), np.zeros_like(S0), np.eye(dk)
    for i0 in range(0, T, C):
        sl = slice(i0, i0 + C)
        st = chunk_stage(q[sl], k[sl], v[sl], alpha[sl], beta[sl], 0)
        fac = np.eye(dk) - st["W"].T @ k[sl]
        prod = prod @ fac
        _, S, _ = chunk_step(st, q[sl], S)
        _, SD, _ = chunk_step(st, q[sl], SD)
        np.testing.assert_allclose(S - SD, S0 @ prod, rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------------------
# linearity and exact arithmetic
# --------------------------------------------------------------------------

@pytest.mark.parametrize("gate", [0, 1])
def test_linear_in_values_and_start_state(gate):
    rng = np.random.default_rng(9)
    T, dk, dv = 30, 6, 4
    q, k, v1, alpha, beta, S01 = rand_seq(rng, T, dk, dv, gate)
    v2 = rng.standard_normal((T, dv))
    S02 = rng.standard_normal((dv, dk))
    c = -1.7
    o1, s1 = run1(q, k, v1, alpha, beta, S0=S01, gate=gate)
    o2, s2 = run1(q, k, v2, alpha, beta, S0=S02, gate=gate)
    o3, s3 = run1(q, k, v1 + c * v2, alpha, beta, S0=S01 + c * S02, gate=gate)
    np.testing.assert_allclose(o3, o1 + c * o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s3, s1 + c * s2, rtol=1e-12, atol=1e-12)


def _exact_run(q, k, v, alpha, beta, S0, order, gate):
    """Exact rational arithmetic, matrix form: e = v - Sbar k (Sbar the state
    the prediction reads), S <- S D + beta e k^T, o = S q."""
    dk = len(k[0])
    S = [[Fraction(x) for x in row] for row in S0]
    outs = []
    for t in range(len(q)):
        a = [Fraction(alpha[t][c] if gate else alpha[t]) for c in range(dk)]
        Sd = [[row[c] * a[c] for c in range(dk)] for row in S]
        Sp = Sd if order == DTP else S
        kt = [Fraction(x) for x in k[t]]
        e = [Fraction(v[t][r]) - sum(Sp[r][c] * kt[c] for c in range(dk))
             for r in range(len(S))]
        bt = Fraction(beta[t])
        S = [[Sd[r][c] + bt * e[r] * kt[c] for c in range(dk)] for r in range(len(S))]
        outs.append([sum(S[r][c] * Fraction(q[t][c]) for c in range(dk))
                     for r in range(len(S))])
    return outs, S


@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("order", [PTD, DTP])
def test_exact_rationals_tiny(gate, order):
    """T <= 32 on dyadic inputs: fp64 agrees with exact arithmetic."""
    rng = np.random.default_rng(10)
    T, dk, dv = 24, 3, 2
    dy = lambda shape: rng.integers(-8, 9, shape) / 8.0
    q, k, v = dy((T, dk)), dy((T, dk)), dy((T, dv))
    alpha = rng.integers(4, 9, (T, dk) if gate else (T,)) / 8.0
    beta = rng.integers(0, 9, T) / 8.0
    S0 = dy((dv, dk))
    o, s = run1(q, k, v, alpha, beta, S0=S0, gate=gate, order=order)
    oe, se = _exact_run(q, k, v, alpha, beta, S0, order, gate)
    scale = max(1.0, float(np.abs(o).max()))
    np.testing.assert_allclose(o, np.array(oe, dtype=float), rtol=0, atol=1e-12 * scale)
    np.testing.assert_allclose(s, np.array(se, dtype=float), rtol=0, atol=1e-12 * scale)


def test_batch_head_layout_and_threads():
    """[B,T,H,d] layout: every (b, h) slice equals its own single run."""
    rng = np.random.default_rng(11)
    B, T, H, dk, dv = 2, 17, 3, 4, 5
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk)) / 2
    v = rng.standard_normal((B, T, H, dv))
    alpha = rng.uniform(0.5, 1.0, (B, T, H))
    beta = rng.uniform(0.0, 1.0, (B, T, H))
    S0 = rng.standard_normal((B, H, dv, dk))
    o, s = oracle.forward(q, k, v, alpha, beta, S0, threads=3)
    for b in range(B):
        for h in range(H):
            o1, s1 = run1(q[b, :, h], k[b, :, h], v[b, :, h], alpha[b, :, h],
                          beta[b, :, h], S0=S0[b, h])
            np.testing.assert_array_equal(o[b, :, h], o1)
            np.testing.assert_array_equal(s[b, h], s1)


def test_empty_sequence_returns_start_state():
    rng = np.random.default_rng(12)
    S0 = rng.standard_normal((1, 2, 3, 4))
    z = lambda *s: np.zeros(s)
    o, s = oracle.forward(z(1, 0, 2, 4), z(1, 0, 2, 4), z(1, 0, 2, 3), z(1, 0, 2),
                          z(1, 0, 2), S0)
    assert o.shape == (1, 0, 2, 3)
    np.testing.assert_array_equal(s, S0)


@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("order", [PTD, DTP])
def test_one_token_calls_thread_the_state(gate, order):
    """The recurrence carries nothing but S between tokens (the fixed-size
    state of the linear-attention-as-RNN reading): T calls of one token each,
    each starting from the previous call's state, equal one call over the T
    tokens.  This is what makes the oracle the reference for chains of
    single-token decode steps."""
    rng = np.random.default_rng(21 + gate + 2 * order)
    q, k, v, alpha, beta, S0 = rand_seq(rng, 9, 6, 5, gate=gate)
    o, s = run1(q, k, v, alpha, beta, S0=S0, gate=gate, order=order)
    st = S0
    for t in range(9):
        o1, st = run1(q[t:t + 1], k[t:t + 1], v[t:t + 1], alpha[t:t + 1], beta[t:t + 1],
                      S0=st, gate=gate, order=order)
        np.testing.assert_array_equal(o1[0], o[t])
    np.testing.assert_array_equal(st, s)


def test_prologue_printed_l2_example_and_sigmoid():
    """The notes' worked L2 example, (3, 4) -> (0.6, 0.8), per (token, head)
    and never across tokens ((30, 40) beside it has its own length 50); the
    sigmoid against the library's logistic function and its fixed point."""
    from scipy.special import expit
    q = np.array([[[3.0, 4.0]], [[30.0, 40.0]]])      # [T=2, H=1, d=2]
    k = np.array([[[0.0, 0.0]], [[-6.0, 8.0]]])       # a zero key stays zero
    logits = np.array([[-3.0, 0.0, 2.5], [40.0, -40.0, 1e-3]])
    qn, kn, a, b = oracle.prologue(q, k, logits, logits[0])
    np.testing.assert_allclose(qn[0, 0], [0.6, 0.8], rtol=0, atol=1e-15)
    np.testing.assert_allclose(qn[1, 0], [0.6, 0.8], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(kn[0, 0], [0.0, 0.0])
    np.testing.assert_allclose(kn[1, 0], [-0.6, 0.8], rtol=0, atol=1e-15)
    np.testing.assert_allclose(a, expit(logits), rtol=1e-15, atol=0)
    np.testing.assert_allclose(b, expit(logits[0]), rtol=1e-15, atol=0)
    assert a[0, 1] == 0.5
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 3, 5, 16)) * rng.uniform(0.1, 10, (4, 3, 5, 1))
    xn = oracle.prologue(x, x, 0.0, 0.0)[0]
    np.testing.assert_allclose(np.linalg.norm(xn, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(xn * np.linalg.norm(x, axis=-1, keepdims=True), x, rtol=1e-13)
