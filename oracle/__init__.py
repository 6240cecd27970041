"""Oracle for the gated delta rule forward pass — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``gated_delta_rule_12_amd``) and never imports it.

``forward`` is the plain definition of the method: a double-precision
token-by-token loop (``gdn_oracle.c``), one (batch, head) pair at a time.
The recurrence, the two gate orderings and the two gate kinds it follows are
stated, with the passages of the pages they come from, in the header of
``gdn_oracle.c``.

``backward`` is the reverse mode of ``forward``: the chain rule through the
same token loop, run backwards over stored states (``gdn_oracle.c``, second
half; the pages give no gradient formulas, so its header derives them).

``prologue`` forms the core's inputs from raw projections (per-head L2 norm of
q and k, sigmoid gates), the step before the core in the DeltaNet block.

``chunked.chunk_backward`` (``oracle/chunked.py``, fp64 numpy) writes the same
gradients (scalar gate) through the chunk form of the forward, the equations
the chunked backward kernels follow; it is pinned to ``backward`` by
``tests/test_oracle_chunk_backward.py``.

Every function here is pinned by ``tests/test_oracle_pins.py`` against what
the pages and the mathematics fix (printed worked examples, closed forms,
affine composition, the WY identity, linearity, exact rational arithmetic on
tiny inputs); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

PREDICT_THEN_DECAY = 0
DECAY_THEN_PREDICT = 1
GATE_SCALAR = 0
GATE_CHANNEL = 1


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (OpenMP).  Building is not using it."""
    if (not force and os.path.exists(_LIB_PATH)
            and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC)):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c99",
           "-o", tmp, _SRC]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            i64, dp = ctypes.c_int64, ctypes.c_void_p
            lib.gdn_oracle_forward.argtypes = [
                i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                ctypes.c_double, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
            lib.gdn_oracle_forward.restype = ctypes.c_int
            lib.gdn_oracle_backward.argtypes = [
                i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                ctypes.c_double] + [dp] * 14 + [ctypes.c_int]
            lib.gdn_oracle_backward.restype = ctypes.c_int
            lib.gdn_oracle_max_threads.argtypes = []
            lib.gdn_oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().gdn_oracle_max_threads())


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def forward(q, k, v, alpha, beta, state0=None, *, gate: int = GATE_SCALAR,
            order: int = PREDICT_THEN_DECAY, scale: float = 1.0,
            threads: int = 0):
    """Token-by-token fp64 gated delta rule.

    q, k: [B, T, H, dk]; v: [B, T, H, dv]; alpha: [B, T, H] (scalar gate) or
    [B, T, H, dk] (channel gate); beta: [B, T, H]; state0: [B, H, dv, dk] or
    None (zero start).  Inputs are read exactly as given (upcast to fp64).
    Returns (out [B, T, H, dv], state [B, H, dv, dk]) as float64 arrays.
    """
    q, k, v, alpha, beta = (_f64(a) for a in (q, k, v, alpha, beta))
    if q.ndim != 4 or k.shape != q.shape or v.ndim != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,T,H,dk] and v [B,T,H,dv]")
    B, T, H, dk = q.shape
    dv = v.shape[3]
    want_alpha = (B, T, H) if gate == GATE_SCALAR else (B, T, H, dk)
    if alpha.shape != want_alpha:
        raise ValueError(f"alpha must have shape {want_alpha}, got {alpha.shape}")
    if beta.shape != (B, T, H):
        raise ValueError("beta must be [B,T,H]")
    s0 = None
    if state0 is not None:
        s0 = _f64(state0)
        if s0.shape != (B, H, dv, dk):
            raise ValueError("state0 must be [B,H,dv,dk]")
    out = np.zeros((B, T, H, dv), dtype=np.float64)
    st = np.zeros((B, H, dv, dk), dtype=np.float64)
    rc = _load().gdn_oracle_forward(B, T, H, dk, dv, int(gate), int(order),
                                    float(scale), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(alpha), _ptr(beta), _ptr(s0),
                                    _ptr(out), _ptr(st), int(threads))
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_forward failed with status {rc}")
    return out, st


def backward(q, k, v, alpha, beta, state0, dout, dstate=None, *,
             gate: int = GATE_SCALAR, order: int = PREDICT_THEN_DECAY,
             scale: float = 1.0, threads: int = 0):
    """Gradients of a loss L through ``forward``: given dout = dL/dout
    [B, T, H, dv] and dstate = dL/dS_T [B, H, dv, dk] (None: zero), returns
    (dq, dk, dv, dalpha, dbeta, dstate0) as float64 arrays shaped like
    q, k, v, alpha, beta and the state.  fp64, token by token in reverse
    over the states of a forward sweep.
    """
    q, k, v, alpha, beta, dout = (_f64(a) for a in (q, k, v, alpha, beta, dout))
    B, T, H, dk = q.shape
    dv = v.shape[3]
    want_alpha = (B, T, H) if gate == GATE_SCALAR else (B, T, H, dk)
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or alpha.shape != want_alpha \
            or beta.shape != (B, T, H) or dout.shape != v.shape:
        raise ValueError("backward: inconsistent shapes")
    s0 = None if state0 is None else _f64(state0)
    dst = None if dstate is None else _f64(dstate)
    for x in (s0, dst):
        if x is not None and x.shape != (B, H, dv, dk):
            raise ValueError("states must be [B,H,dv,dk]")
    dq = np.zeros_like(q)
    dkk = np.zeros_like(k)
    dvv = np.zeros_like(v)
    dal = np.zeros_like(alpha)
    dbe = np.zeros_like(beta)
    ds0 = np.zeros((B, H, dv, dk), dtype=np.float64)
    rc = _load().gdn_oracle_backward(B, T, H, dk, dv, int(gate), int(order), float(scale),
                                     _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                     _ptr(s0), _ptr(dout), _ptr(dst), _ptr(dq), _ptr(dkk),
                                     _ptr(dvv), _ptr(dal), _ptr(dbe), _ptr(ds0), int(threads))
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_backward failed with status {rc}")
    return dq, dkk, dvv, dal, dbe, ds0


def prologue(q, k, alpha_logit, beta_logit):
    """The inputs of the delta-rule core from the model's raw projections, as
    the DeltaNet block forms them (DeltaNet illustrated notes, block
    description): q and k divided by their L2 length along the feature axis,
    separately for every (batch, token, head) (a zero vector stays zero);
    beta = sigmoid(beta_logit) with sigmoid(z) = 1 / (1 + exp(-z)); the gate
    alpha through the same sigmoid.  fp64 throughout.

    q, k: [..., d]; alpha_logit, beta_logit: any shape.  Returns
    (q, k, alpha, beta) as float64 arrays of the same shapes.
    """
    def l2(x):
        x = np.asarray(x, dtype=np.float64)
        n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        return np.divide(x, n, out=np.zeros_like(x), where=n > 0)

    def sigmoid(z):
        return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))

    return l2(q), l2(k), sigmoid(alpha_logit), sigmoid(beta_logit)
