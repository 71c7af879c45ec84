"""Python binding of libjscan (selective state-space scan on MI355X).

Argument marshalling only: every step of the scan runs in the HIP kernels of
``libjscan.so``.  torch supplies device memory and the current HIP stream.
The library must be built (``python -m selective_state_space_11_amd.build`` or
``__graft_entry__.build()``); importing works without it, but every call then
raises ``JscanUnavailable`` -- there is no fallback implementation.

Entry points mirror the C ABI in ``include/jscan.h``:

* ``prefill(x, delta, A, B, C, D, z, h0=None)`` -> ``(y, hT)``
* ``prefill_noalloc(x, delta, A, B, C, D, z, h0=None, y=..., hT=...)``: the
  same through jscan_prefill_noalloc (no allocation anywhere)
* ``step(state, x, delta, A, B, C, D, z)`` -> ``y`` (state updated in place)
* ``step_batch(state, x, delta, A, B, C, D, z)`` -> ``y`` (states updated in place)
* ``prefill_fused`` / ``step_batch_fused``: the same with the layer's input
  prologue (causal depthwise conv + SiLU on x, softplus(delta + dt_bias))
  applied inside the scan kernels
* ``prefill_trap`` / ``step_batch_trap``: the exponential-trapezoidal
  recurrence (Mamba-3's discretisation as read from the pages)
* ``backward(x, delta, A, B, C, D, z, dy, h0=None, dhT=None)`` -> dict of the
  gradients dx, ddelta, dz, dA, dB, dC, dD, dh0
* ``selective_scan(x, delta, A, B, C, D, z, h0=None)`` -> ``(y, hT)`` with
  torch autograd support: forward through jscan_prefill, backward through
  jscan_backward_saved (the forward's workspace is kept for its chunk states)
* ``workspace_size``, ``step_workspace_size``, ``plan``, ``set_plan_override``,
  ``time_next_prefill``, ``prefill_stats``
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libjscan.so")
D_STATE = 16

JSCAN_OK = 0
STATUS_NAMES = {0: "JSCAN_OK", 1: "JSCAN_ERR_NULL", 2: "JSCAN_ERR_SHAPE", 3: "JSCAN_ERR_UNSUPPORTED",
                4: "JSCAN_ERR_ALIGN", 5: "JSCAN_ERR_ALIAS", 6: "JSCAN_ERR_WORKSPACE", 7: "JSCAN_ERR_HIP"}
IO_F32, IO_BF16 = 0, 1

EXPORTS = ("jscan_prefill_workspace_size", "jscan_prefill", "jscan_prefill_noalloc", "jscan_step", "jscan_step_batch",
           "jscan_status_string", "jscan_last_error", "jscan_prefill_plan",
           "jscan_set_plan_override", "jscan_time_next_prefill", "jscan_prefill_fused",
           "jscan_step_batch_fused", "jscan_backward_workspace_size", "jscan_backward", "jscan_prefill_trap",
           "jscan_step_batch_trap", "jscan_backward_saved", "jscan_prefill_stats", "jscan_step_workspace_size",
           "jscan_step_batch_fused_ws")


class Trap(ctypes.Structure):
    """struct jscan_trap (device pointers as integers)."""
    _fields_ = [("lam", ctypes.c_void_p), ("x_prev", ctypes.c_void_p), ("B_prev", ctypes.c_void_p)]


class Prologue(ctypes.Structure):
    """struct jscan_prologue (device pointers as integers)."""
    _fields_ = [("conv_weight", ctypes.c_void_p), ("conv_bias", ctypes.c_void_p),
                ("conv_state_in", ctypes.c_void_p), ("conv_state_out", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p), ("conv_width", ctypes.c_int32), ("dt_softplus", ctypes.c_int32),
                ("rms_dt_weight", ctypes.c_void_p), ("rms_B_weight", ctypes.c_void_p),
                ("rms_C_weight", ctypes.c_void_p), ("rms_eps", ctypes.c_float)]


class JscanUnavailable(RuntimeError):
    """libjscan.so is not built or cannot be loaded."""


class JscanError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


_lock = threading.Lock()
_lib = None


def load_library(path: str = LIB_PATH):
    """Load libjscan.so and declare its C signatures (no GPU work)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise JscanUnavailable(f"{path} is not built; run `python -m selective_state_space_11_amd.build`")
        try:
            lib = ctypes.CDLL(path)
        except OSError as e:
            raise JscanUnavailable(f"cannot load {path}: {e}") from e
        i64, vp, sz, st = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        fp = ctypes.c_void_p
        lib.jscan_prefill_workspace_size.argtypes = [i64, i64, i64, i64, st]
        lib.jscan_prefill_workspace_size.restype = sz
        lib.jscan_prefill.argtypes = [i64, i64, i64, i64, st, vp, vp, fp, vp, vp, fp, vp, fp, vp, fp, vp, sz, vp]
        lib.jscan_prefill.restype = st
        lib.jscan_prefill_noalloc.argtypes = [i64, i64, i64, i64, st, vp, vp, fp, vp, vp, fp, vp, fp, vp, fp, vp]
        lib.jscan_prefill_noalloc.restype = st
        lib.jscan_step.argtypes = [i64, i64, st, fp, vp, vp, fp, vp, vp, fp, vp, vp, vp]
        lib.jscan_step.restype = st
        lib.jscan_step_batch.argtypes = [i64, i64, i64, st, fp, vp, vp, fp, vp, vp, fp, vp, vp, vp]
        lib.jscan_step_batch.restype = st
        lib.jscan_status_string.argtypes = [st]
        lib.jscan_status_string.restype = ctypes.c_char_p
        lib.jscan_last_error.argtypes = []
        lib.jscan_last_error.restype = ctypes.c_char_p
        lib.jscan_prefill_plan.argtypes = [i64, i64, i64, i64, ctypes.POINTER(ctypes.c_int),
                                           ctypes.POINTER(ctypes.c_int)]
        lib.jscan_prefill_plan.restype = st
        lib.jscan_set_plan_override.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.jscan_set_plan_override.restype = st
        lib.jscan_time_next_prefill.argtypes = [vp, vp]
        lib.jscan_time_next_prefill.restype = None
        lib.jscan_prefill_stats.argtypes = [vp, sz, i64, i64, i64, ctypes.POINTER(ctypes.c_double), vp]
        lib.jscan_prefill_stats.restype = st
        pp = ctypes.POINTER(Prologue)
        lib.jscan_prefill_fused.argtypes = [i64, i64, i64, i64, st, vp, vp, fp, vp, vp, fp, vp, fp, vp, fp, pp, vp,
                                            sz, vp]
        lib.jscan_prefill_fused.restype = st
        lib.jscan_step_batch_fused.argtypes = [i64, i64, i64, st, fp, vp, vp, fp, vp, vp, fp, vp, vp, pp, vp]
        lib.jscan_step_batch_fused.restype = st
        lib.jscan_step_workspace_size.argtypes = [i64, i64, i64, st, pp]
        lib.jscan_step_workspace_size.restype = sz
        lib.jscan_step_batch_fused_ws.argtypes = [i64, i64, i64, st, fp, vp, vp, fp, vp, vp, fp, vp, vp, pp, vp, sz,
                                                  vp]
        lib.jscan_step_batch_fused_ws.restype = st
        tp = ctypes.POINTER(Trap)
        lib.jscan_prefill_trap.argtypes = [i64, i64, i64, i64, st, vp, vp, fp, vp, vp, fp, vp, fp, vp, fp, tp, pp, vp,
                                           sz, vp]
        lib.jscan_prefill_trap.restype = st
        lib.jscan_step_batch_trap.argtypes = [i64, i64, i64, st, fp, vp, vp, fp, vp, vp, fp, vp, vp, tp, pp, vp]
        lib.jscan_step_batch_trap.restype = st
        lib.jscan_backward_workspace_size.argtypes = [i64, i64, i64, i64, st]
        lib.jscan_backward_workspace_size.restype = sz
        lib.jscan_backward.argtypes = [i64, i64, i64, i64, st] + [vp] * 18 + [vp, sz, vp]
        lib.jscan_backward.restype = st
        lib.jscan_backward_saved.argtypes = [i64, i64, i64, i64, st] + [vp] * 18 + [vp, sz, vp, sz, vp]
        lib.jscan_backward_saved.restype = st
        _lib = lib
        return lib


def _check(status):
    if status != JSCAN_OK:
        msg = load_library().jscan_last_error().decode()
        raise JscanError(status, msg)


def _torch():
    import torch
    return torch


def _io_of(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return IO_BF16
    if t.dtype == torch.float32:
        return IO_F32
    raise TypeError(f"I/O tensors must be bfloat16 or float32, got {t.dtype}")


def _dev(t, name, dtype=None, shape=None):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def workspace_size(batch, L, d_inner, d_state=D_STATE, io=IO_BF16) -> int:
    return int(load_library().jscan_prefill_workspace_size(batch, L, d_inner, d_state, io))


def plan(batch, L, d_inner, d_state=D_STATE):
    k, c = ctypes.c_int(), ctypes.c_int()
    _check(load_library().jscan_prefill_plan(batch, L, d_inner, d_state, ctypes.byref(k), ctypes.byref(c)))
    return k.value, c.value


def set_plan_override(waves_per_group=0, chunks=0):
    """Force the prefill's launch plan on this thread; (0, 0) restores the automatic one."""
    _check(load_library().jscan_set_plan_override(int(waves_per_group), int(chunks)))


def prefill_stats(workspace, batch, L, d_inner, stream=None):
    """(state-only fraction of pass 1, rescanned fraction of pass 2, chunks) of
    the last chunked prefill of these sizes that used ``workspace`` (a device
    uint8 tensor); the fractions are of the tokens of the chunks after the first."""
    out = (ctypes.c_double * 3)()
    _dev(workspace, "workspace")
    _check(load_library().jscan_prefill_stats(_ptr(workspace), workspace.numel() * workspace.element_size(), batch,
                                              L, d_inner, out, _stream(stream)))
    return out[0], out[1], int(out[2])


def time_next_prefill(before, after):
    """Record HIP events around the next prefill's main scan kernel (torch.cuda.Event
    created with enable_timing=True).  torch creates the underlying hipEvent_t
    lazily, at its first record(); record each once so the handle exists."""
    for ev in (before, after):
        if not ev.cuda_event:
            ev.record()
    load_library().jscan_time_next_prefill(ctypes.c_void_p(before.cuda_event), ctypes.c_void_p(after.cuda_event))


def prefill(x, delta, A, B, C, D, z, h0=None, *, y=None, hT=None, want_state=True,
            workspace=None, stream=None):
    """Selective scan over [batch, L, d_inner] inputs.  Returns (y, hT); hT is None
    when want_state is False and no hT buffer is given.  hT may be h0 (in place)."""
    torch = _torch()
    lib = load_library()
    _dev(x, "x")
    batch, L, d_inner = x.shape
    io = _io_of(x)
    _dev(delta, "delta", x.dtype, x.shape)
    _dev(z, "z", x.dtype, x.shape)
    _dev(B, "B", x.dtype, (batch, L, D_STATE))
    _dev(C, "C", x.dtype, (batch, L, D_STATE))
    _dev(A, "A", torch.float32, (d_inner, D_STATE))
    _dev(D, "D", torch.float32, (d_inner,))
    _dev(h0, "h0", torch.float32, (batch, d_inner, D_STATE))
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", x.dtype, x.shape)
    if hT is None and want_state:
        hT = torch.empty((batch, d_inner, D_STATE), dtype=torch.float32, device=x.device)
    _dev(hT, "hT", torch.float32, (batch, d_inner, D_STATE))
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.jscan_prefill(batch, L, d_inner, D_STATE, io, _ptr(x), _ptr(delta), _ptr(A), _ptr(B),
                             _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(hT), _ptr(workspace),
                             ws_bytes, _stream(stream)))
    return y, hT


def prefill_noalloc(x, delta, A, B, C, D, z, h0=None, *, y, hT=None, stream=None):
    """jscan_prefill_noalloc: the prefill with its chunk records in the
    library's own per-GPU scratch array, for callers that cannot allocate.
    The caller passes every output buffer (y, and hT or None); nothing is
    allocated here either."""
    torch = _torch()
    lib = load_library()
    _dev(x, "x")
    batch, L, d_inner = x.shape
    io = _io_of(x)
    _dev(delta, "delta", x.dtype, x.shape)
    _dev(z, "z", x.dtype, x.shape)
    _dev(B, "B", x.dtype, (batch, L, D_STATE))
    _dev(C, "C", x.dtype, (batch, L, D_STATE))
    _dev(A, "A", torch.float32, (d_inner, D_STATE))
    _dev(D, "D", torch.float32, (d_inner,))
    _dev(h0, "h0", torch.float32, (batch, d_inner, D_STATE))
    _dev(y, "y", x.dtype, x.shape)
    _dev(hT, "hT", torch.float32, (batch, d_inner, D_STATE))
    _check(lib.jscan_prefill_noalloc(batch, L, d_inner, D_STATE, io, _ptr(x), _ptr(delta), _ptr(A), _ptr(B),
                                     _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(hT), _stream(stream)))
    return y, hT


def step_batch(state, x, delta, A, B, C, D, z, *, y=None, stream=None):
    """One decode token for n_seq sequences; state [n_seq, d_inner, 16] is updated in place."""
    torch = _torch()
    lib = load_library()
    _dev(state, "state", torch.float32)
    n_seq, d_inner, _ = state.shape
    _dev(state, "state", torch.float32, (n_seq, d_inner, D_STATE))
    _dev(x, "x", None, (n_seq, d_inner))
    io = _io_of(x)
    _dev(delta, "delta", x.dtype, x.shape)
    _dev(z, "z", x.dtype, x.shape)
    _dev(B, "B", x.dtype, (n_seq, D_STATE))
    _dev(C, "C", x.dtype, (n_seq, D_STATE))
    _dev(A, "A", torch.float32, (d_inner, D_STATE))
    _dev(D, "D", torch.float32, (d_inner,))
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", x.dtype, x.shape)
    _check(lib.jscan_step_batch(n_seq, d_inner, D_STATE, io, _ptr(state), _ptr(x), _ptr(delta), _ptr(A),
                                _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y), _stream(stream)))
    return y


def step(state, x, delta, A, B, C, D, z, *, y=None, stream=None):
    """One decode token for one sequence; state [d_inner, 16] is updated in place."""
    torch = _torch()
    lib = load_library()
    _dev(state, "state", torch.float32)
    d_inner = state.shape[0]
    _dev(state, "state", torch.float32, (d_inner, D_STATE))
    _dev(x, "x", None, (d_inner,))
    io = _io_of(x)
    _dev(delta, "delta", x.dtype, x.shape)
    _dev(z, "z", x.dtype, x.shape)
    _dev(B, "B", x.dtype, (D_STATE,))
    _dev(C, "C", x.dtype, (D_STATE,))
    _dev(A, "A", torch.float32, (d_inner, D_STATE))
    _dev(D, "D", torch.float32, (d_inner,))
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", x.dtype, x.shape)
    _check(lib.jscan_step(d_inner, D_STATE, io, _ptr(state), _ptr(x), _ptr(delta), _ptr(A), _ptr(B),
                          _ptr(C), _ptr(D), _ptr(z), _ptr(y), _stream(stream)))
    return y


def _prologue(nseq, d_inner, conv_weight, conv_bias, conv_state_in, conv_state_out, dt_bias, softplus,
              rms=None):
    """rms: None or (w_dt [d_inner] or None, w_B [16] or None, w_C [16] or None, eps)."""
    torch = _torch()
    width = 1
    if conv_weight is not None:
        _dev(conv_weight, "conv_weight", torch.float32)
        if conv_weight.dim() != 2 or conv_weight.shape[0] != d_inner:
            raise ValueError(f"conv_weight must be [{d_inner}, width], got {tuple(conv_weight.shape)}")
        width = conv_weight.shape[1]
        _dev(conv_bias, "conv_bias", torch.float32, (d_inner,))
        _dev(conv_state_in, "conv_state_in", torch.float32, (nseq, width - 1, d_inner))
        _dev(conv_state_out, "conv_state_out", torch.float32, (nseq, width - 1, d_inner))
    _dev(dt_bias, "dt_bias", torch.float32, (d_inner,))
    p = Prologue()
    p.conv_weight = None if conv_weight is None else conv_weight.data_ptr()
    p.conv_bias = None if conv_bias is None else conv_bias.data_ptr()
    p.conv_state_in = None if conv_state_in is None else conv_state_in.data_ptr()
    p.conv_state_out = None if conv_state_out is None else conv_state_out.data_ptr()
    p.dt_bias = None if dt_bias is None else dt_bias.data_ptr()
    p.conv_width = width
    p.dt_softplus = 1 if softplus else 0
    if rms is not None:
        w_dt, w_B, w_C, eps = rms
        _dev(w_dt, "rms_dt_weight", torch.float32, (d_inner,))
        _dev(w_B, "rms_B_weight", torch.float32, (D_STATE,))
        _dev(w_C, "rms_C_weight", torch.float32, (D_STATE,))
        p.rms_dt_weight = None if w_dt is None else w_dt.data_ptr()
        p.rms_B_weight = None if w_B is None else w_B.data_ptr()
        p.rms_C_weight = None if w_C is None else w_C.data_ptr()
        p.rms_eps = float(eps)
    return p


def prefill_fused(x, delta, A, B, C, D, z, h0=None, *, conv_weight=None, conv_bias=None, conv_state_in=None,
                  conv_state_out=None, dt_bias=None, softplus=False, rms=None, y=None, hT=None, want_state=True,
                  workspace=None, stream=None):
    """prefill with the input prologue: x -> SiLU(causal depthwise conv(x) + conv_bias)
    (conv_weight [d_inner, width], width 1..4; conv_state_in/out [batch, width-1, d_inner],
    may be one tensor) and, with softplus, delta -> softplus(delta + dt_bias); rms =
    (w_dt, w_B, w_C, eps) first applies RMSNorm to delta (over d_inner) and to the B, C rows
    (over 16), a None weight skipping that tensor.  Returns (y, hT)."""
    torch = _torch()
    lib = load_library()
    _dev(x, "x")
    batch, L, d_inner = x.shape
    io = _io_of(x)
    _dev(delta, "delta", x.dtype, x.shape)
    _dev(z, "z", x.dtype, x.shape)
    _dev(B, "B", x.dtype, (batch, L, D_STATE))
    _dev(C, "C", x.dtype, (batch, L, D_STATE))
    _dev(A, "A", torch.float32, (d_inner, D_STATE))
    _dev(D, "D", torch.float32, (d_inner,))
    _dev(h0, "h0", torch.float32, (batch, d_inner, D_STATE))
    pro = _prologue(batch, d_inner, conv_weight, conv_bias, conv_state_in, conv_state_out, dt_bias, softplus, rms)
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", x.dtype, x.shape)
    if hT is None and want_state:
        hT = torch.empty((batch, d_inner, D_STATE), dtype=torch.float32, device=x.device)
    _dev(hT, "hT", torch.float32, (batch, d_inner, D_STATE))
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.jscan_prefill_fused(batch, L, d_inner, D_STATE, io, _ptr(x), _ptr(delta), _ptr(A), _ptr(B),
                                   _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(hT), ctypes.byref(pro),
                                   _ptr(workspace), ws_bytes, _stream(stream)))
    return y, hT


def step_workspace_size(n_seq, d_inner, rms=None, io=IO_BF16) -> int:
    """Bytes of workspace step_batch_fused needs with this RMSNorm argument (0 without one)."""
    pro = _prologue(n_seq, d_inner, None, None, None, None, None, False, rms)
    return int(load_library().jscan_step_workspace_size(n_seq, d_inner, D_STATE, io, ctypes.byref(pro)))


def step_batch_fused(state, x, delta, A, B, C, D, z, *, conv_weight=None, conv_bias=None, conv_state=None,
                     dt_bias=None, softplus=False, rms=None, y=None, workspace=None, stream=None):
    """step_batch with the input prologue; conv_state [n_seq, width-1, d_inner] holds the last
    width-1 raw x of each sequence and is updated in place, like state.  With RMSNorm, a
    workspace of step_workspace_size() bytes keeps the step free of allocations."""
    torch = _torch()
    lib = load_library()
    _dev(state, "state", torch.float32)
    n_seq, d_inner, _ = state.shape
    _dev(state, "state", torch.float32, (n_seq, d_inner, D_STATE))
    _dev(x, "x", None, (n_seq, d_inner))
    io = _io_of(x)
    _dev(delta, "delta", x.dtype, x.shape)
    _dev(z, "z", x.dtype, x.shape)
    _dev(B, "B", x.dtype, (n_seq, D_STATE))
    _dev(C, "C", x.dtype, (n_seq, D_STATE))
    _dev(A, "A", torch.float32, (d_inner, D_STATE))
    _dev(D, "D", torch.float32, (d_inner,))
    pro = _prologue(n_seq, d_inner, conv_weight, conv_bias, conv_state, conv_state, dt_bias, softplus, rms)
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", x.dtype, x.shape)
    if workspace is None:
        _check(lib.jscan_step_batch_fused(n_seq, d_inner, D_STATE, io, _ptr(state), _ptr(x), _ptr(delta), _ptr(A),
                                          _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y), ctypes.byref(pro),
                                          _stream(stream)))
    else:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
        _check(lib.jscan_step_batch_fused_ws(n_seq, d_inner, D_STATE, io, _ptr(state), _ptr(x), _ptr(delta),
                                             _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y),
                                             ctypes.byref(pro), _ptr(workspace), ws_bytes, _stream(stream)))
    return y


def backward_workspace_size(batch, L, d_inner, d_state=D_STATE, io=IO_BF16) -> int:
    return int(load_library().jscan_backward_workspace_size(batch, L, d_inner, d_state, io))


def backward(x, delta, A, B, C, D, z, dy, h0=None, dhT=None, *, want_dh0=True, out=None, workspace=None,
             prefill_workspace=None, stream=None):
    """Gradients of prefill for output gradients dy (like y) and dhT ([batch, d_inner, 16]
    fp32 or None).  Returns a dict: dx, ddelta, dz (like x), dA [d_inner, 16], dB, dC
    [batch, L, 16], dD [d_inner] (fp32) and dh0 ([batch, d_inner, 16] fp32, or None when
    want_dh0 is False).  ``out`` may supply any of these tensors.  ``prefill_workspace``:
    the workspace a prefill call over the same inputs used (jscan_backward_saved reads the
    chunk starting states from it instead of recomputing them)."""
    torch = _torch()
    lib = load_library()
    _dev(x, "x")
    batch, L, d_inner = x.shape
    io = _io_of(x)
    for name, t in (("delta", delta), ("z", z), ("dy", dy)):
        _dev(t, name, x.dtype, x.shape)
    _dev(B, "B", x.dtype, (batch, L, D_STATE))
    _dev(C, "C", x.dtype, (batch, L, D_STATE))
    _dev(A, "A", torch.float32, (d_inner, D_STATE))
    _dev(D, "D", torch.float32, (d_inner,))
    _dev(h0, "h0", torch.float32, (batch, d_inner, D_STATE))
    _dev(dhT, "dhT", torch.float32, (batch, d_inner, D_STATE))
    out = dict(out or {})
    shapes = {"dx": (x.shape, x.dtype), "ddelta": (x.shape, x.dtype), "dz": (x.shape, x.dtype),
              "dA": ((d_inner, D_STATE), torch.float32), "dB": ((batch, L, D_STATE), torch.float32),
              "dC": ((batch, L, D_STATE), torch.float32), "dD": ((d_inner,), torch.float32),
              "dh0": ((batch, d_inner, D_STATE), torch.float32)}
    for name, (shape, dtype) in shapes.items():
        if name == "dh0" and not want_dh0 and out.get(name) is None:
            out[name] = None
            continue
        if out.get(name) is None:
            out[name] = torch.empty(shape, dtype=dtype, device=x.device)
        _dev(out[name], name, dtype, shape)
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    args = (batch, L, d_inner, D_STATE, io, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(h0), _ptr(dy), _ptr(dhT), _ptr(out["dx"]), _ptr(out["ddelta"]), _ptr(out["dz"]), _ptr(out["dA"]),
            _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dh0"]))
    if prefill_workspace is None:
        _check(lib.jscan_backward(*args, _ptr(workspace), ws_bytes, _stream(stream)))
    else:
        _dev(prefill_workspace, "prefill_workspace")
        pws_bytes = prefill_workspace.numel() * prefill_workspace.element_size()
        _check(lib.jscan_backward_saved(*args, _ptr(prefill_workspace), pws_bytes, _ptr(workspace), ws_bytes,
                                        _stream(stream)))
    return out


def _trap(x, nseq, L, d_inner, lam, x_prev, B_prev):
    _dev(lam, "lam", x.dtype, (nseq, L, d_inner) if L is not None else (nseq, d_inner))
    _dev(x_prev, "x_prev", x.dtype, (nseq, d_inner))
    _dev(B_prev, "B_prev", x.dtype, (nseq, D_STATE))
    t = Trap()
    t.lam = None if lam is None else lam.data_ptr()
    t.x_prev = None if x_prev is None else x_prev.data_ptr()
    t.B_prev = None if B_prev is None else B_prev.data_ptr()
    return t


def prefill_trap(x, delta, A, B, C, D, z, h0=None, *, lam=None, x_prev=None, B_prev=None, dt_bias=None,
                 softplus=False, y=None, hT=None, want_state=True, workspace=None, stream=None):
    """Exponential-trapezoidal prefill: h_t = a_t h_{t-1} + dt_t ((1 - lam_t) a_t B_{t-1} x_{t-1}
    + lam_t B_t x_t).  lam like x (None: 1/2); x_prev [batch, d_inner] and B_prev [batch, 16]
    (like x, None: zero) give the token before the first.  Returns (y, hT)."""
    torch = _torch()
    lib = load_library()
    _dev(x, "x")
    batch, L, d_inner = x.shape
    io = _io_of(x)
    _dev(delta, "delta", x.dtype, x.shape)
    _dev(z, "z", x.dtype, x.shape)
    _dev(B, "B", x.dtype, (batch, L, D_STATE))
    _dev(C, "C", x.dtype, (batch, L, D_STATE))
    _dev(A, "A", torch.float32, (d_inner, D_STATE))
    _dev(D, "D", torch.float32, (d_inner,))
    _dev(h0, "h0", torch.float32, (batch, d_inner, D_STATE))
    tr = _trap(x, batch, L, d_inner, lam, x_prev, B_prev)
    pro = _prologue(batch, d_inner, None, None, None, None, dt_bias, softplus)
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", x.dtype, x.shape)
    if hT is None and want_state:
        hT = torch.empty((batch, d_inner, D_STATE), dtype=torch.float32, device=x.device)
    _dev(hT, "hT", torch.float32, (batch, d_inner, D_STATE))
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.jscan_prefill_trap(batch, L, d_inner, D_STATE, io, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                  _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(hT), ctypes.byref(tr),
                                  ctypes.byref(pro), _ptr(workspace), ws_bytes, _stream(stream)))
    return y, hT


def step_batch_trap(state, x, delta, A, B, C, D, z, *, lam=None, x_prev=None, B_prev=None, dt_bias=None,
                    softplus=False, y=None, stream=None):
    """step_batch with the exponential-trapezoidal recurrence; x_prev and B_prev are the
    previous step's x [n_seq, d_inner] and B [n_seq, 16] (None: zero), lam like x."""
    torch = _torch()
    lib = load_library()
    _dev(state, "state", torch.float32)
    n_seq, d_inner, _ = state.shape
    _dev(state, "state", torch.float32, (n_seq, d_inner, D_STATE))
    _dev(x, "x", None, (n_seq, d_inner))
    io = _io_of(x)
    _dev(delta, "delta", x.dtype, x.shape)
    _dev(z, "z", x.dtype, x.shape)
    _dev(B, "B", x.dtype, (n_seq, D_STATE))
    _dev(C, "C", x.dtype, (n_seq, D_STATE))
    _dev(A, "A", torch.float32, (d_inner, D_STATE))
    _dev(D, "D", torch.float32, (d_inner,))
    tr = _trap(x, n_seq, None, d_inner, lam, x_prev, B_prev)
    pro = _prologue(n_seq, d_inner, None, None, None, None, dt_bias, softplus)
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", x.dtype, x.shape)
    _check(lib.jscan_step_batch_trap(n_seq, d_inner, D_STATE, io, _ptr(state), _ptr(x), _ptr(delta), _ptr(A),
                                     _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y), ctypes.byref(tr),
                                     ctypes.byref(pro), _stream(stream)))
    return y


_ScanFn = None


def _scan_fn():
    """torch.autograd.Function pairing jscan_prefill with jscan_backward (built
    on first use so that importing this module does not import torch)."""
    global _ScanFn
    if _ScanFn is not None:
        return _ScanFn
    torch = _torch()

    class ScanFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, delta, A, B, C, D, z, h0):
            # The prefill's workspace is kept: it holds the chunk starting
            # states, which the backward then does not recompute.
            nb = workspace_size(*x.shape, io=_io_of(x))
            ws = torch.empty(nb, dtype=torch.uint8, device=x.device) if nb else None
            y, hT = prefill(x, delta, A, B, C, D, z, h0, workspace=ws)
            ctx.save_for_backward(x, delta, A, B, C, D, z, h0)
            ctx.has_h0 = h0 is not None
            ctx.prefill_ws = ws
            ctx.plan = (plan(*x.shape), nb)
            return y, hT

        @staticmethod
        def backward(ctx, dy, dhT):
            x, delta, A, B, C, D, z, h0 = ctx.saved_tensors
            if dy is None:
                dy = torch.zeros_like(x)
            # The plan is per thread and autograd may run this on another
            # thread: the saved states are used only under the same plan.
            saved = ctx.prefill_ws if (plan(*x.shape), workspace_size(*x.shape, io=_io_of(x))) == ctx.plan else None
            g = backward(x, delta, A, B, C, D, z, dy.contiguous(), h0 if ctx.has_h0 else None,
                         None if dhT is None else dhT.contiguous(), want_dh0=ctx.has_h0,
                         prefill_workspace=saved)
            ctx.prefill_ws = None
            return (g["dx"], g["ddelta"], g["dA"], g["dB"].to(B.dtype), g["dC"].to(C.dtype), g["dD"], g["dz"],
                    g["dh0"] if ctx.has_h0 else None)

    _ScanFn = ScanFn
    return ScanFn


def selective_scan(x, delta, A, B, C, D, z, h0=None):
    """Differentiable prefill: (y, hT) = prefill(...), with gradients for every
    input from jscan_backward_saved (the forward's workspace is kept until the
    backward).  dB and dC are returned in B's and C's dtype."""
    return _scan_fn().apply(x, delta, A, B, C, D, z, h0)
