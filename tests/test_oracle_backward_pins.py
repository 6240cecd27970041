"""Pins for the oracle's backward pass (``oracle.backward``).

The pages give no gradient formulas; the oracle derives them by the chain
rule through the forward token loop.  They are pinned here against the
oracle's forward pass alone, by central finite differences in fp64:

* every input element on tiny shapes (all four gate kinds x orderings, a
  scale other than one, a start state and a gradient on the final state);
* random directions on larger shapes (long-memory gates, unequal dk and dv);
* special cases that fix single terms: beta = 0 makes v irrelevant (dv = 0),
  a zero dout and dstate give zero gradients everywhere, and with T = 0 the
  start-state gradient is the final-state gradient itself;
* and by a second, independent route: PyTorch's reverse mode through a plain
  fp64 token loop written in the test from the recurrence (agreement to
  1e-12).

A dropped term, a wrong sign, a transposed state or a gate on the wrong axis
in the backward changes at least one of these derivatives by far more than
the finite-difference error (about 1e-9 relative here).
"""
import numpy as np
import pytest

import oracle

PTD = oracle.PREDICT_THEN_DECAY
DTP = oracle.DECAY_THEN_PREDICT
SC, CH = oracle.GATE_SCALAR, oracle.GATE_CHANNEL


def inputs(rng, B, T, H, dk, dv, gate, alpha_mean=2.0):
    q = rng.normal(size=(B, T, H, dk))
    k = rng.normal(size=(B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(size=(B, T, H, dv))
    ash = (B, T, H) if gate == SC else (B, T, H, dk)
    a = 1.0 / (1.0 + np.exp(-rng.normal(alpha_mean, 0.5, size=ash)))
    b = 1.0 / (1.0 + np.exp(-rng.normal(size=(B, T, H))))
    s0 = rng.normal(size=(B, H, dv, dk)) * 0.5
    do = rng.normal(size=(B, T, H, dv))
    ds = rng.normal(size=(B, H, dv, dk))
    return [q, k, v, a, b, s0], do, ds


def loss(x, do, ds, gate, order, scale):
    o, s = oracle.forward(*x, gate=gate, order=order, scale=scale)
    return float((o * do).sum() + (s * ds).sum())


@pytest.mark.parametrize("gate", [SC, CH])
@pytest.mark.parametrize("order", [PTD, DTP])
def test_every_element_by_central_differences(gate, order):
    rng = np.random.default_rng(10 + 2 * gate + order)
    x, do, ds = inputs(rng, B=1, T=6, H=2, dk=4, dv=3, gate=gate)
    scale = 0.7
    g = oracle.backward(*x, do, ds, gate=gate, order=order, scale=scale)
    eps = 1e-6
    for i, name in enumerate(["q", "k", "v", "alpha", "beta", "state0"]):
        num = np.zeros_like(x[i])
        for idx in np.ndindex(x[i].shape):
            xp = list(x)
            xx = x[i].copy()
            xx[idx] += eps
            xp[i] = xx
            lp = loss(xp, do, ds, gate, order, scale)
            xx[idx] -= 2 * eps
            lm = loss(xp, do, ds, gate, order, scale)
            num[idx] = (lp - lm) / (2 * eps)
        err = np.abs(num - g[i]).max() / np.abs(num).max()
        assert err < 1e-7, (name, err)


@pytest.mark.parametrize("gate,order,dk,dv,alpha_mean", [
    (SC, PTD, 16, 8, 2.0), (CH, DTP, 8, 16, 2.0), (SC, DTP, 12, 12, 6.0), (CH, PTD, 16, 16, 6.0)])
def test_random_directions(gate, order, dk, dv, alpha_mean):
    """<grad, u> against (L(x + eps u) - L(x - eps u)) / 2 eps for random u,
    on 40 tokens and two batches, one input at a time."""
    rng = np.random.default_rng(100 + dk + dv)
    x, do, ds = inputs(rng, B=2, T=40, H=2, dk=dk, dv=dv, gate=gate, alpha_mean=alpha_mean)
    g = oracle.backward(*x, do, ds, gate=gate, order=order)
    eps = 1e-6
    for i in range(6):
        for _ in range(3):
            u = rng.normal(size=x[i].shape)
            xp, xm = list(x), list(x)
            xp[i] = x[i] + eps * u
            xm[i] = x[i] - eps * u
            num = (loss(xp, do, ds, gate, order, 1.0) - loss(xm, do, ds, gate, order, 1.0)) / (2 * eps)
            ana = float((g[i] * u).sum())
            assert abs(num - ana) <= 1e-7 * max(1.0, abs(num)), (i, num, ana)


def test_special_cases():
    rng = np.random.default_rng(7)
    x, do, ds = inputs(rng, B=1, T=9, H=2, dk=8, dv=8, gate=SC)
    # beta = 0: the update never reads v
    x0 = list(x)
    x0[4] = np.zeros_like(x[4])
    g = oracle.backward(*x0, do, ds)
    assert np.all(g[2] == 0.0)
    assert np.abs(g[4]).max() > 0  # but the loss does depend on beta
    # no upstream gradient: every gradient vanishes
    g = oracle.backward(*x, np.zeros_like(do), None)
    assert all(np.all(a == 0.0) for a in g)
    # T = 0: dS0 is dS_T and nothing else is touched
    xe = [a[:, :0] if a.ndim >= 3 and i < 5 else a for i, a in enumerate(x)]
    g = oracle.backward(*xe, do[:, :0], ds)
    assert np.array_equal(g[5], ds)


@pytest.mark.parametrize("gate", [SC, CH])
@pytest.mark.parametrize("order", [PTD, DTP])
def test_against_autograd_of_a_plain_loop(gate, order):
    """A second, independent route to the same gradients: PyTorch's reverse
    mode through a plain fp64 token loop written here from the recurrence
    (the update as the pages state it, not the oracle's code), on every input
    at once."""
    import torch
    rng = np.random.default_rng(30 + 2 * gate + order)
    x, do, ds = inputs(rng, B=1, T=24, H=2, dk=6, dv=5, gate=gate)
    scale = 1.3
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in x]
    q, k, v, al, be, s0 = t
    B, T, H, dk = q.shape
    outs = []
    states = []
    for h in range(H):
        S = s0[0, h]
        o_h = []
        for tt in range(T):
            kt, qt, vt, b = k[0, tt, h], q[0, tt, h], v[0, tt, h], be[0, tt, h]
            d = al[0, tt, h] * torch.ones(dk, dtype=torch.float64) if gate == SC else al[0, tt, h]
            if order == PTD:
                S = S * d + b * torch.outer(vt - S @ kt, kt)
            else:
                Sb = S * d
                S = Sb + b * torch.outer(vt - Sb @ kt, kt)
            o_h.append(scale * (S @ qt))
        outs.append(torch.stack(o_h))
        states.append(S)
    out = torch.stack(outs, dim=1)[None]   # [1, T, H, dv]
    st = torch.stack(states)[None]         # [1, H, dv, dk]
    L = (out * torch.tensor(do)).sum() + (st * torch.tensor(ds)).sum()
    L.backward()
    g = oracle.backward(*x, do, ds, gate=gate, order=order, scale=scale)
    for name, a, ref in zip(["q", "k", "v", "alpha", "beta", "state0"], g, t):
        r = ref.grad.numpy()
        assert np.abs(a - r).max() <= 1e-12 * max(1.0, np.abs(r).max()), name
