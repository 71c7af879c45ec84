"""fp64 CPU oracle for the selective state-space scan.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  Nothing in the product package imports
this module, and this module imports nothing from the product package.

Two implementations of the same definition live here:

* ``jscan_oracle.c`` (loaded through ctypes): the sequential fp64 loop, threaded
  over independent (batch, channel) pairs.  ``prefill`` and ``step`` are written
  separately in C.
* ``backward`` (C, ``oracle_backward``): the gradient of the prefill by the
  adjoint recurrence, every forward state kept, for training.
* ``prefill_trap`` (C, ``oracle_prefill_trap``): the exponential-trapezoidal
  variant of the recurrence (Mamba-3's discretisation as read from the pages).
* ``rmsnorm_inputs`` (C, ``oracle_rmsnorm_inputs``): RMSNorm of the time step
  and the B, C rows before the scan (Jamba's stabilising normalisation).
* ``twin.py``: the same loop in numpy, vectorised over channels only, for
  small shapes and as a cross-check of the C code.

The definition they follow (see the header of ``jscan_oracle.c``) is the
state-space recurrence of the "AI Engineering from Scratch" Jamba lesson,
section "一页讲完 SSM", with data-dependent (selective) parameters, a real
diagonal A per (channel, state) as in Mamba-1, exp(delta*A) decay, the
delta*B*x input term, the D skip and the SiLU(z) gate on the whole output.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "jscan_oracle.c")
_LIB = os.path.join(_HERE, "libjscan_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
               "-shared", "-fPIC", "-std=c11", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            dp = ctypes.POINTER(ctypes.c_double)
            i64 = ctypes.c_int64
            lib.oracle_prefill.argtypes = [i64, i64, i64, i64] + [dp] * 10
            lib.oracle_prefill.restype = None
            lib.oracle_step.argtypes = [i64, i64, i64] + [dp] * 9
            lib.oracle_step.restype = None
            lib.oracle_prologue.argtypes = [i64, i64, i64, i64] + [dp] * 6 + [dp, dp, ctypes.c_int, dp]
            lib.oracle_prologue.restype = None
            lib.oracle_backward.argtypes = [i64, i64, i64, i64] + [dp] * 18
            lib.oracle_backward.restype = ctypes.c_int
            lib.oracle_prefill_trap.argtypes = [i64, i64, i64, i64] + [dp] * 15
            lib.oracle_prefill_trap.restype = None
            lib.oracle_rmsnorm_inputs.argtypes = [i64, i64, i64, i64] + [dp] * 6 + [ctypes.c_double] + [dp] * 3
            lib.oracle_rmsnorm_inputs.restype = None
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = ctypes.c_int
            lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
            lib.oracle_set_num_threads.restype = None
            _lib = lib
    return _lib


def _f64(a, shape, name):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {a.shape}, expected {shape}")
    return a


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def prefill(x, delta, A, B, C, D, z, h0=None, want_state=True):
    """Sequential fp64 scan.

    x, delta, z: [batch, L, d_inner]; B, C: [batch, L, d_state];
    A: [d_inner, d_state]; D: [d_inner]; h0: [batch, d_inner, d_state] or None.
    Returns (y [batch, L, d_inner], hT [batch, d_inner, d_state] or None), float64.
    """
    x = np.asarray(x)
    batch, L, d_inner = x.shape
    d_state = np.asarray(A).shape[1]
    if d_state > 256:
        raise ValueError("oracle supports d_state <= 256")
    x = _f64(x, (batch, L, d_inner), "x")
    delta = _f64(delta, (batch, L, d_inner), "delta")
    z = _f64(z, (batch, L, d_inner), "z")
    A = _f64(A, (d_inner, d_state), "A")
    B = _f64(B, (batch, L, d_state), "B")
    C = _f64(C, (batch, L, d_state), "C")
    D = _f64(D, (d_inner,), "D")
    h0 = None if h0 is None else _f64(h0, (batch, d_inner, d_state), "h0")
    y = np.empty((batch, L, d_inner), dtype=np.float64)
    hT = np.empty((batch, d_inner, d_state), dtype=np.float64) if want_state else None
    _load().oracle_prefill(batch, L, d_inner, d_state, _ptr(x), _ptr(delta), _ptr(A),
                           _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(hT))
    return y, hT


def step(state, x, delta, A, B, C, D, z):
    """One decode token for n_seq sequences.

    state: [n_seq, d_inner, d_state] (not modified; the updated state is returned);
    x, delta, z: [n_seq, d_inner]; B, C: [n_seq, d_state].
    Returns (y [n_seq, d_inner], new_state), float64.
    """
    state = np.array(state, dtype=np.float64, copy=True, order="C")
    n_seq, d_inner, d_state = state.shape
    x = _f64(x, (n_seq, d_inner), "x")
    delta = _f64(delta, (n_seq, d_inner), "delta")
    z = _f64(z, (n_seq, d_inner), "z")
    A = _f64(A, (d_inner, d_state), "A")
    B = _f64(B, (n_seq, d_state), "B")
    C = _f64(C, (n_seq, d_state), "C")
    D = _f64(D, (d_inner,), "D")
    y = np.empty((n_seq, d_inner), dtype=np.float64)
    _load().oracle_step(n_seq, d_inner, d_state, _ptr(state), _ptr(x), _ptr(delta), _ptr(A),
                        _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y))
    return y, state


def prologue(x, delta, conv_weight=None, conv_bias=None, conv_state=None, dt_bias=None, softplus=False):
    """Input prologue of a Mamba layer (see jscan_oracle.c): causal depthwise
    convolution of x + SiLU, and delta -> softplus(delta + dt_bias).

    x, delta: [batch, L, d_inner]; conv_weight: [d_inner, width] or None (no
    convolution); conv_bias, dt_bias: [d_inner] or None; conv_state:
    [batch, width-1, d_inner] or None (zeros).
    Returns (xc, delta_out, conv_state_out or None), float64.
    """
    x = np.asarray(x)
    batch, L, d_inner = x.shape
    x = _f64(x, (batch, L, d_inner), "x")
    delta = _f64(delta, (batch, L, d_inner), "delta")
    width = 1
    w = bias = st = None
    if conv_weight is not None:
        width = np.asarray(conv_weight).shape[1]
        w = _f64(conv_weight, (d_inner, width), "conv_weight")
        bias = None if conv_bias is None else _f64(conv_bias, (d_inner,), "conv_bias")
        st = None if conv_state is None else _f64(conv_state, (batch, width - 1, d_inner), "conv_state")
    dtb = None if dt_bias is None else _f64(dt_bias, (d_inner,), "dt_bias")
    xc = np.empty_like(x)
    dout = np.empty_like(delta)
    st_out = np.empty((batch, width - 1, d_inner)) if w is not None else None
    _load().oracle_prologue(batch, L, d_inner, width, _ptr(x), _ptr(w), _ptr(bias), _ptr(st), _ptr(xc),
                            _ptr(st_out), _ptr(delta), _ptr(dtb), 1 if softplus else 0, _ptr(dout))
    return xc, dout, st_out


def backward(x, delta, A, B, C, D, z, dy, h0=None, dhT=None):
    """Gradients of the prefill for output gradients dy [batch, L, d_inner] and
    dhT [batch, d_inner, d_state] (None: zero), by the adjoint recurrence (see
    jscan_oracle.c).  Returns a dict of float64 arrays dx, ddelta, dz
    [batch, L, d_inner], dA [d_inner, d_state], dB, dC [batch, L, d_state],
    dD [d_inner] and dh0 [batch, d_inner, d_state]."""
    x = np.asarray(x)
    batch, L, d_inner = x.shape
    d_state = np.asarray(A).shape[1]
    if d_state > 256:
        raise ValueError("oracle supports d_state <= 256")
    x = _f64(x, (batch, L, d_inner), "x")
    delta = _f64(delta, (batch, L, d_inner), "delta")
    z = _f64(z, (batch, L, d_inner), "z")
    dy = _f64(dy, (batch, L, d_inner), "dy")
    A = _f64(A, (d_inner, d_state), "A")
    B = _f64(B, (batch, L, d_state), "B")
    C = _f64(C, (batch, L, d_state), "C")
    D = _f64(D, (d_inner,), "D")
    h0 = None if h0 is None else _f64(h0, (batch, d_inner, d_state), "h0")
    dhT = None if dhT is None else _f64(dhT, (batch, d_inner, d_state), "dhT")
    out = {k: np.empty((batch, L, d_inner)) for k in ("dx", "ddelta", "dz")}
    out["dA"] = np.empty((d_inner, d_state))
    out["dB"] = np.empty((batch, L, d_state))
    out["dC"] = np.empty((batch, L, d_state))
    out["dD"] = np.empty((d_inner,))
    out["dh0"] = np.empty((batch, d_inner, d_state))
    rc = _load().oracle_backward(batch, L, d_inner, d_state, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                 _ptr(D), _ptr(z), _ptr(h0), _ptr(dy), _ptr(dhT), _ptr(out["dx"]),
                                 _ptr(out["ddelta"]), _ptr(out["dz"]), _ptr(out["dA"]), _ptr(out["dB"]),
                                 _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dh0"]))
    if rc:
        raise MemoryError("oracle_backward: out of memory")
    return out


def prefill_trap(x, delta, A, B, C, D, z, h0=None, lam=None, x_prev=None, B_prev=None, want_state=True):
    """Exponential-trapezoidal prefill (see jscan_oracle.c):
    h_t = a_t h_{t-1} + dt_t ((1 - lam_t) a_t B_{t-1} x_{t-1} + lam_t B_t x_t).
    lam: [batch, L, d_inner] or None (1/2); x_prev [batch, d_inner], B_prev
    [batch, d_state] or None (0).  Returns (y, hT, x_last, B_last), float64."""
    x = np.asarray(x)
    batch, L, d_inner = x.shape
    d_state = np.asarray(A).shape[1]
    if d_state > 256:
        raise ValueError("oracle supports d_state <= 256")
    x = _f64(x, (batch, L, d_inner), "x")
    delta = _f64(delta, (batch, L, d_inner), "delta")
    z = _f64(z, (batch, L, d_inner), "z")
    A = _f64(A, (d_inner, d_state), "A")
    B = _f64(B, (batch, L, d_state), "B")
    C = _f64(C, (batch, L, d_state), "C")
    D = _f64(D, (d_inner,), "D")
    h0 = None if h0 is None else _f64(h0, (batch, d_inner, d_state), "h0")
    lam = None if lam is None else _f64(lam, (batch, L, d_inner), "lam")
    x_prev = None if x_prev is None else _f64(x_prev, (batch, d_inner), "x_prev")
    B_prev = None if B_prev is None else _f64(B_prev, (batch, d_state), "B_prev")
    y = np.empty((batch, L, d_inner))
    hT = np.empty((batch, d_inner, d_state)) if want_state else None
    x_last = np.empty((batch, d_inner))
    B_last = np.empty((batch, d_state))
    _load().oracle_prefill_trap(batch, L, d_inner, d_state, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                _ptr(D), _ptr(z), _ptr(h0), _ptr(lam), _ptr(x_prev), _ptr(B_prev), _ptr(y),
                                _ptr(hT), _ptr(x_last), _ptr(B_last))
    return y, hT, x_last, B_last


def rmsnorm_inputs(delta, B, C, w_dt=None, w_B=None, w_C=None, eps=1e-6):
    """RMSNorm of delta over d_inner and of the B, C rows over d_state, per token
    (see jscan_oracle.c).  A None weight leaves that tensor unchanged.
    Returns (delta_out, B_out, C_out), float64, unrounded."""
    delta = np.asarray(delta)
    batch, L, d_inner = delta.shape
    d_state = np.asarray(B).shape[2]
    delta = _f64(delta, (batch, L, d_inner), "delta")
    B = _f64(B, (batch, L, d_state), "B")
    C = _f64(C, (batch, L, d_state), "C")
    w_dt = None if w_dt is None else _f64(w_dt, (d_inner,), "w_dt")
    w_B = None if w_B is None else _f64(w_B, (d_state,), "w_B")
    w_C = None if w_C is None else _f64(w_C, (d_state,), "w_C")
    outs = (np.empty_like(delta), np.empty_like(B), np.empty_like(C))
    _load().oracle_rmsnorm_inputs(batch, L, d_inner, d_state, _ptr(delta), _ptr(B), _ptr(C), _ptr(w_dt), _ptr(w_B),
                                  _ptr(w_C), float(eps), _ptr(outs[0]), _ptr(outs[1]),
                                  _ptr(outs[2]))
    return outs
