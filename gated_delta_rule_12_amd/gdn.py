"""Thin Python binding of libgdn.so (include/gdn.h).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of libgdn.so.  PyTorch supplies device memory and the stream.  There
is no fallback: if the library is missing or no GPU is present, calls raise.

Low-level names mirror the C ABI (gdn_chunk_fwd, gdn_recurrent_ref,
gdn_seqpar_fwd, gdn_decode_step, ...); chunk_fwd / seqpar_fwd / recurrent_ref /
decode_step are the same calls taking torch tensors and allocating the
outputs and the workspace.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
GDN_GATE_SCALAR, GDN_GATE_CHANNEL = 0, 1
GDN_PREDICT_THEN_DECAY, GDN_DECAY_THEN_PREDICT = 0, 1
GDN_OK, GDN_E_ARG, GDN_E_SHAPE, GDN_E_UNSUPPORTED, GDN_E_WORKSPACE, GDN_E_HIP = 0, -1, -2, -3, -4, -5
GDN_E_SCRATCH = -6
GDN_NOALLOC_SCRATCH_BYTES = 128 << 20
GDN_PATH_VALU, GDN_PATH_MFMA = 0, 1
GDN_BWD_TOKEN, GDN_BWD_CHUNKED = 0, 1

# every symbol include/gdn.h declares
EXPORTS = ("gdn_chunk_fwd", "gdn_recurrent_ref", "gdn_seqpar_fwd", "gdn_decode_step",
           "gdn_decode_step_raw", "gdn_backward", "gdn_backward_workspace_bytes",
           "gdn_workspace_bytes",
           "gdn_validate", "gdn_chunk_path", "gdn_chunk_segments", "gdn_seqpar_segments",
           "gdn_status_str", "gdn_abi_version",
           "gdn_timer_create", "gdn_timer_destroy", "gdn_timer_read", "gdn_chunk_fwd_timed",
           "gdn_seqpar_fwd_timed", "gdn_decode_step_timed", "gdn_backward_timed",
           "gdn_chunk_fwd_noalloc", "gdn_chunk_fwd_raw", "gdn_chunk_fwd_raw_timed",
           "gdn_raw_workspace_bytes", "gdn_backward_path")

_lib = None


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} ({status})")
        self.status = status


def lib():
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, f32, vp, sz = (ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                             ctypes.c_void_p, ctypes.c_size_t)
    shape = [i64, i64, i64, i64, i64]
    tens = [vp] * 8
    L.gdn_chunk_fwd.argtypes = shape + [i32, i32, i32, i32, f32] + tens + [vp, sz, vp]
    L.gdn_chunk_fwd.restype = ctypes.c_int
    L.gdn_chunk_fwd_raw.argtypes = shape + [i32, i32, i32, i32, f32] + tens + [vp, sz, vp]
    L.gdn_chunk_fwd_raw.restype = ctypes.c_int
    L.gdn_raw_workspace_bytes.argtypes = shape + [i32, i32, i32]
    L.gdn_raw_workspace_bytes.restype = sz
    L.gdn_chunk_fwd_noalloc.argtypes = shape + [i32, i32, i32, i32, f32] + tens + [vp]
    L.gdn_chunk_fwd_noalloc.restype = ctypes.c_int
    L.gdn_seqpar_fwd.argtypes = shape + [i32, i32, i32, i32, f32, i32] + tens + [vp, sz, vp]
    L.gdn_seqpar_fwd.restype = ctypes.c_int
    L.gdn_recurrent_ref.argtypes = shape + [i32, i32, i32, f32] + tens + [vp]
    L.gdn_recurrent_ref.restype = ctypes.c_int
    L.gdn_decode_step.argtypes = [i64] * 4 + [i32, i32, i32, f32] + tens + [vp]
    L.gdn_decode_step.restype = ctypes.c_int
    L.gdn_decode_step_raw.argtypes = [i64] * 4 + [i32, i32, i32, f32] + tens + [vp]
    L.gdn_decode_step_raw.restype = ctypes.c_int
    L.gdn_backward.argtypes = shape + [i32, i32, i32, f32] + [vp] * 14 + [vp, sz, vp]
    L.gdn_backward.restype = ctypes.c_int
    L.gdn_backward_workspace_bytes.argtypes = shape + [i32]
    L.gdn_backward_workspace_bytes.restype = sz
    L.gdn_workspace_bytes.argtypes = shape + [i32, i32, i32, i32]
    L.gdn_workspace_bytes.restype = sz
    L.gdn_validate.argtypes = shape + [i32, i32, i32, i32, i32]
    L.gdn_validate.restype = ctypes.c_int
    L.gdn_chunk_path.argtypes = [i64, i64, i32, i32, i32]
    L.gdn_chunk_path.restype = ctypes.c_int
    L.gdn_backward_path.argtypes = [i64, i64, i32]
    L.gdn_backward_path.restype = ctypes.c_int
    L.gdn_chunk_segments.argtypes = shape + [i32, i32, i32]
    L.gdn_chunk_segments.restype = ctypes.c_int
    L.gdn_seqpar_segments.argtypes = shape + [i32, i32, i32, i32]
    L.gdn_seqpar_segments.restype = ctypes.c_int
    L.gdn_status_str.argtypes = [ctypes.c_int]
    L.gdn_status_str.restype = ctypes.c_char_p
    L.gdn_abi_version.argtypes = []
    L.gdn_abi_version.restype = ctypes.c_int
    L.gdn_timer_create.argtypes = [ctypes.POINTER(vp)]
    L.gdn_timer_create.restype = ctypes.c_int
    L.gdn_timer_destroy.argtypes = [vp]
    L.gdn_timer_destroy.restype = ctypes.c_int
    L.gdn_timer_read.argtypes = [vp, ctypes.c_int, ctypes.c_char_p, sz,
                                 ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    L.gdn_timer_read.restype = ctypes.c_int
    # the *_timed variants: the same arguments plus the timer
    for name in ("gdn_chunk_fwd", "gdn_chunk_fwd_raw", "gdn_seqpar_fwd", "gdn_decode_step",
                 "gdn_backward"):
        f = getattr(L, name + "_timed")
        f.argtypes = getattr(L, name).argtypes + [vp]
        f.restype = ctypes.c_int
    _lib = L
    return L


# ---- raw C ABI ---------------------------------------------------------------

def gdn_chunk_fwd(*args):
    return lib().gdn_chunk_fwd(*args)


def gdn_seqpar_fwd(*args):
    return lib().gdn_seqpar_fwd(*args)


def gdn_recurrent_ref(*args):
    return lib().gdn_recurrent_ref(*args)


def gdn_decode_step(*args):
    return lib().gdn_decode_step(*args)


def gdn_decode_step_raw(*args):
    return lib().gdn_decode_step_raw(*args)


def gdn_backward(*args):
    return lib().gdn_backward(*args)


def gdn_backward_workspace_bytes(B, T, H, dk, dv, gate=GDN_GATE_SCALAR) -> int:
    return int(lib().gdn_backward_workspace_bytes(B, T, H, dk, dv, gate))


def gdn_workspace_bytes(B, T, H, dk, dv, chunk, dtype, gate, n_segments=1) -> int:
    return int(lib().gdn_workspace_bytes(B, T, H, dk, dv, chunk, dtype, gate, n_segments))


def gdn_validate(B, T, H, dk, dv, chunk, dtype, gate, order, n_segments=1) -> int:
    return int(lib().gdn_validate(B, T, H, dk, dv, chunk, dtype, gate, order, n_segments))


def gdn_chunk_path(dk, dv, chunk, dtype, gate) -> int:
    return int(lib().gdn_chunk_path(dk, dv, chunk, dtype, gate))


def gdn_backward_path(dk, dv, gate) -> int:
    return int(lib().gdn_backward_path(dk, dv, gate))


def gdn_chunk_segments(B, T, H, dk, dv, chunk, dtype, gate) -> int:
    return int(lib().gdn_chunk_segments(B, T, H, dk, dv, chunk, dtype, gate))


def gdn_seqpar_segments(B, T, H, dk, dv, chunk, dtype, gate, n_segments) -> int:
    return int(lib().gdn_seqpar_segments(B, T, H, dk, dv, chunk, dtype, gate, n_segments))


def gdn_status_str(status: int) -> str:
    return lib().gdn_status_str(int(status)).decode()


status_str = gdn_status_str


def gdn_abi_version() -> int:
    return int(lib().gdn_abi_version())


class Timer:
    """A caller-owned per-kernel timer (gdn_timer_create / gdn_timer_read /
    gdn_timer_destroy).  Pass it as timer= to the torch-level helpers; they
    then call the *_timed entry points, which bracket each kernel with HIP
    events on the launch stream."""

    def __init__(self):
        h = ctypes.c_void_p()
        rc = lib().gdn_timer_create(ctypes.byref(h))
        if rc != GDN_OK:
            raise GdnError(rc, "gdn_timer_create")
        self.handle = h

    def read(self):
        """Every kernel timed so far: {name: (total ms, launches)}."""
        res = {}
        buf = ctypes.create_string_buffer(128)
        i = 0
        while True:
            ms, cnt = ctypes.c_double(), ctypes.c_int64()
            if lib().gdn_timer_read(self.handle, i, buf, 128, ctypes.byref(ms),
                                    ctypes.byref(cnt)) != GDN_OK:
                break
            res[buf.value.decode()] = (ms.value, cnt.value)
            i += 1
        return res

    def close(self):
        if self.handle is not None:
            lib().gdn_timer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _call(name, args, timer):
    """The entry point `name`, or its *_timed variant with the timer."""
    if timer is None:
        return getattr(lib(), name)(*args)
    return getattr(lib(), name + "_timed")(*args, timer.handle)


# ---- torch-level helpers -------------------------------------------------------

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _check(q, k, v, alpha, beta, state0):
    import torch
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,T,H,dk] and v [B,T,H,dv]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    tensors = [q, k, v, alpha, beta] + ([state0] if state0 is not None else [])
    for t in tensors:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    for t in tensors[3:]:
        if t.dtype != torch.float32:
            raise TypeError("alpha, beta, state0 must be float32")
    B, T, H, dk = q.shape
    dv = v.shape[3]
    if alpha.shape == (B, T, H):
        gate = GDN_GATE_SCALAR
    elif alpha.shape == (B, T, H, dk):
        gate = GDN_GATE_CHANNEL
    else:
        raise ValueError("alpha must be [B,T,H] or [B,T,H,dk]")
    if beta.shape != (B, T, H):
        raise ValueError("beta must be [B,T,H]")
    if state0 is not None and state0.shape != (B, H, dv, dk):
        raise ValueError("state0 must be [B,H,dv,dk]")
    return B, T, H, dk, dv, gate


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspace_for(q, v, alpha, chunk=64, n_segments=None):
    import torch
    B, T, H, dk = q.shape
    gate = GDN_GATE_SCALAR if alpha.dim() == 3 else GDN_GATE_CHANNEL
    n = gdn_workspace_bytes(B, T, H, dk, v.shape[3], chunk, _dtype_code(q), gate,
                            1 if n_segments is None else n_segments)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)


def chunk_fwd(q, k, v, alpha, beta, state0=None, *, chunk=64,
              order=GDN_PREDICT_THEN_DECAY, scale=1.0, n_segments=None,
              out=None, state_out=None, workspace=None, timer=None):
    """Chunkwise forward: gdn_chunk_fwd (the library's schedule) when
    n_segments is None, else gdn_seqpar_fwd with that many segments (1: a
    single stream).  timer: a Timer (the *_timed entry point) or None.
    Returns (out [B,T,H,dv] fp32, final state [B,H,dv,dk] fp32)."""
    import torch
    B, T, H, dk, dv, gate = _check(q, k, v, alpha, beta, state0)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=q.device)
    if state_out is None:
        state_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = workspace_for(q, v, alpha, chunk, n_segments)
    args = [B, T, H, dk, dv, chunk, _dtype_code(q), gate, order, scale]
    tens = [_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state0),
            _ptr(out), _ptr(state_out)]
    tail = [_ptr(workspace), workspace.numel(), _stream()]
    if n_segments is None:
        where = "gdn_chunk_fwd"
        rc = _call(where, [*args, *tens, *tail], timer)
    else:
        where = "gdn_seqpar_fwd"
        rc = _call(where, [*args, n_segments, *tens, *tail], timer)
    if rc != GDN_OK:
        raise GdnError(rc, where)
    return out, state_out


def chunk_fwd_raw(q, k, v, alpha_logit, beta_logit, state0=None, *, chunk=64,
                  order=GDN_PREDICT_THEN_DECAY, scale=1.0, out=None, state_out=None,
                  workspace=None, timer=None):
    """gdn_chunk_fwd_raw: the forward on raw projections q, k (L2-normalised
    in the kernels) and gate / beta logits (through a sigmoid in the
    kernels); timer: a Timer (gdn_chunk_fwd_raw_timed) or None.
    Returns (out [B,T,H,dv] fp32, final state [B,H,dv,dk])."""
    import torch
    B, T, H, dk, dv, gate = _check(q, k, v, alpha_logit, beta_logit, state0)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=q.device)
    if state_out is None:
        state_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    if workspace is None:
        n = int(lib().gdn_raw_workspace_bytes(B, T, H, dk, dv, chunk, _dtype_code(q), gate))
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    rc = _call("gdn_chunk_fwd_raw",
               [B, T, H, dk, dv, chunk, _dtype_code(q), gate, order, scale,
                _ptr(q), _ptr(k), _ptr(v), _ptr(alpha_logit), _ptr(beta_logit),
                _ptr(state0), _ptr(out), _ptr(state_out), _ptr(workspace),
                workspace.numel(), _stream()], timer)
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_chunk_fwd_raw")
    return out, state_out


def chunk_fwd_noalloc(q, k, v, alpha, beta, state0=None, *, chunk=64,
                      order=GDN_PREDICT_THEN_DECAY, scale=1.0, out=None, state_out=None):
    """gdn_chunk_fwd_noalloc: the forward with the library's static device
    scratch as its workspace (the call itself allocates nothing; out and
    state_out are allocated here when not given)."""
    import torch
    B, T, H, dk, dv, gate = _check(q, k, v, alpha, beta, state0)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=q.device)
    if state_out is None:
        state_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    rc = lib().gdn_chunk_fwd_noalloc(B, T, H, dk, dv, chunk, _dtype_code(q), gate, order, scale,
                                     _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                     _ptr(state0), _ptr(out), _ptr(state_out), _stream())
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_chunk_fwd_noalloc")
    return out, state_out


def seqpar_fwd(q, k, v, alpha, beta, state0=None, *, n_segments=8, **kw):
    return chunk_fwd(q, k, v, alpha, beta, state0, n_segments=n_segments, **kw)


def recurrent_ref(q, k, v, alpha, beta, state0=None, *, order=GDN_PREDICT_THEN_DECAY,
                  scale=1.0, out=None, state_out=None):
    import torch
    B, T, H, dk, dv, gate = _check(q, k, v, alpha, beta, state0)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=q.device)
    if state_out is None:
        state_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    rc = gdn_recurrent_ref(B, T, H, dk, dv, _dtype_code(q), gate, order, scale,
                           _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state0),
                           _ptr(out), _ptr(state_out), _stream())
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_recurrent_ref")
    return out, state_out


def backward(q, k, v, alpha, beta, state0, grad_out, grad_state_out=None, *,
             order=GDN_PREDICT_THEN_DECAY, scale=1.0, want_grad_state0=True, workspace=None,
             timer=None):
    """Gradients through the forward pass: gdn_backward.
    grad_out [B,T,H,dv] fp32 = dL/d out; grad_state_out [B,H,dv,dk] fp32 =
    dL/d S_T or None (zero).  Returns (dq, dk, dv, dalpha, dbeta, dstate0),
    fp32, shaped like q, k, v, alpha, beta and the state (dstate0 None when
    not wanted)."""
    import torch
    B, T, H, dk, dv, gate = _check(q, k, v, alpha, beta, state0)
    for t in (grad_out, grad_state_out):
        if t is not None and (not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float32):
            raise ValueError("gradients must be contiguous float32 GPU tensors")
    if grad_out.shape != (B, T, H, dv):
        raise ValueError("grad_out must be [B,T,H,dv]")
    if grad_state_out is not None and grad_state_out.shape != (B, H, dv, dk):
        raise ValueError("grad_state_out must be [B,H,dv,dk]")
    dev = q.device
    f32 = torch.float32
    dq = torch.empty((B, T, H, dk), dtype=f32, device=dev)
    dkk = torch.empty((B, T, H, dk), dtype=f32, device=dev)
    dvv = torch.empty((B, T, H, dv), dtype=f32, device=dev)
    dal = torch.empty(alpha.shape, dtype=f32, device=dev)
    dbe = torch.empty((B, T, H), dtype=f32, device=dev)
    ds0 = torch.empty((B, H, dv, dk), dtype=f32, device=dev) if want_grad_state0 else None
    if workspace is None:
        n = gdn_backward_workspace_bytes(B, T, H, dk, dv, gate)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    rc = _call("gdn_backward",
               [B, T, H, dk, dv, _dtype_code(q), gate, order, scale,
                _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state0),
                _ptr(grad_out), _ptr(grad_state_out), _ptr(dq), _ptr(dkk), _ptr(dvv),
                _ptr(dal), _ptr(dbe), _ptr(ds0), _ptr(workspace), workspace.numel(),
                _stream()], timer)
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_backward")
    return dq, dkk, dvv, dal, dbe, ds0


def decode_step(q, k, v, alpha, beta, state=None, *, order=GDN_PREDICT_THEN_DECAY,
                scale=1.0, out=None, state_out=None, inplace=False, raw=False, timer=None):
    """One token on a persistent state: gdn_decode_step.
    q, k [B,H,dk], v [B,H,dv] (bf16 or fp32), alpha [B,H] or [B,H,dk], beta
    [B,H] fp32, state [B,H,dv,dk] fp32 or None (zero).  inplace=True writes the
    new state over `state`.  raw=True calls gdn_decode_step_raw: q, k are raw
    projections (L2-normalised in the kernel) and alpha, beta are logits
    (passed through a sigmoid in the kernel).
    Returns (out [B,H,dv] fp32, new state)."""
    import torch
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k must be [B,H,dk] and v [B,H,dv]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    B, H, dk = q.shape
    dv = v.shape[2]
    tensors = [q, k, v, alpha, beta] + ([state] if state is not None else [])
    for t in tensors:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous and on the GPU")
    for t in tensors[3:]:
        if t.dtype != torch.float32:
            raise TypeError("alpha, beta, state must be float32")
    if alpha.shape == (B, H):
        gate = GDN_GATE_SCALAR
    elif alpha.shape == (B, H, dk):
        gate = GDN_GATE_CHANNEL
    else:
        raise ValueError("alpha must be [B,H] or [B,H,dk]")
    if beta.shape != (B, H):
        raise ValueError("beta must be [B,H]")
    if state is not None and state.shape != (B, H, dv, dk):
        raise ValueError("state must be [B,H,dv,dk]")
    if inplace:
        if state is None:
            raise ValueError("inplace needs a state")
        state_out = state
    if out is None:
        out = torch.empty((B, H, dv), dtype=torch.float32, device=q.device)
    if state_out is None:
        state_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    if raw and timer is not None:
        raise ValueError("the raw decode step has no timed variant")
    name = "gdn_decode_step_raw" if raw else "gdn_decode_step"
    rc = _call(name, [B, H, dk, dv, _dtype_code(q), gate, order, scale,
                      _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state),
                      _ptr(out), _ptr(state_out), _stream()], timer)
    if rc != GDN_OK:
        raise GdnError(rc, name)
    return out, state_out
