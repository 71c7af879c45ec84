"""Seeded synthetic inputs for the selective-scan workloads.

This module is shared by the tests, the benchmark and the smoke check: it is
the only code the oracle and the HIP path have in common, and it holds none of
the scan's arithmetic.  It draws random numbers, rounds them to the I/O dtype
and hands out numpy arrays.

Recipe (Jamba-shaped inputs: hidden 4096, d_inner 8192, d_state 16):

* Token tensors are drawn per block of ``CHUNK`` = 4096 tokens from
  ``numpy.random.Generator(PCG64([seed, block]))`` in the fixed order
  x, delta, z (each [batch, block, d_inner]), then B, C (each [batch, block,
  d_state]); all draws are float64.
  - x, z ~ N(0, 1)
  - delta = softplus(N(0, 1) - 2), so delta > 0 with a median of about 0.13
  - B, C ~ N(0, 1) / 4
* Per-layer parameters come from ``PCG64([seed, PARAM_STREAM])`` in the order
  A, D, h0:
  - A[d, n] = -exp(U(log 1, log 16)), fp32
  - D[d] ~ N(0, 1), fp32
  - h0 ~ N(0, 1) fp32 when requested, else absent (zero state)
* Input-prologue parameters (causal depthwise conv of width W, time-step
  bias) come from ``PCG64([seed, PROLOGUE_STREAM])`` in the order
  conv_weight [d_inner, W] ~ N(0, 1) / sqrt(W), conv_bias [d_inner] ~
  N(0, 1) / 4, conv_state [batch, W-1, d_inner] ~ N(0, 1), dt_bias
  [d_inner] = log(expm1(dt0)) with log dt0 ~ U(log 1e-3, log 1e-1), all fp32.
  RMSNorm weights (time step [d_inner], B and C rows [d_state]) ~ U(0.5, 1.5)
  come from ``PCG64([seed, PROLOGUE_STREAM, 2])``.
  Raw (pre-softplus) time steps for tokens [0, L) come from
  ``PCG64([seed, PROLOGUE_STREAM, 1])`` as N(0, 1) [batch, L, d_inner] in the
  I/O dtype.
* Output gradients for the backward scan come from ``PCG64([seed,
  GRAD_STREAM, block])`` per block of ``CHUNK`` tokens as dy ~ N(0, 1)
  [batch, block, d_inner] in the I/O dtype, and dhT ~ N(0, 1) [batch, d_inner,
  d_state] fp32 from ``PCG64([seed, GRAD_STREAM])``.
* Trapezoidal-recurrence inputs come from ``PCG64([seed, TRAP_STREAM])``:
  lam ~ U(0, 1) [batch, L, d_inner], then the token before the first,
  x_prev ~ N(0, 1) [batch, d_inner] and B_prev ~ N(0, 1) / 4 [batch,
  d_state], all in the I/O dtype.
* Decode inputs for step k of a run seeded ``seed`` come from
  ``PCG64([seed, DECODE_STREAM, k])`` in the order x, delta, z ([n_seq,
  d_inner]), B, C ([n_seq, d_state]); the initial decode state (~N(0, 1)) from
  ``PCG64([seed, STATE_STREAM])``.

bf16 values are produced from float64 by rounding to float32 (nearest-even)
and then to bf16 (nearest-even on the float32 bit pattern) and are stored as
uint16 bit patterns.  Both consumers read the same rounded values: the oracle
widens them exactly to float64 (``widen``), the GPU reads the bit patterns.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

CHUNK = 4096
PARAM_STREAM = 1_000_003
DECODE_STREAM = 2_000_003
STATE_STREAM = 3_000_017
PROLOGUE_STREAM = 4_000_037
GRAD_STREAM = 5_000_011
TRAP_STREAM = 6_000_013

IO_BF16 = "bf16"
IO_F32 = "f32"


def _threads(requested=None):
    if requested:
        return int(requested)
    return max(1, min(8, os.cpu_count() or 1))


def to_bf16_bits(a) -> np.ndarray:
    """float (any width) -> bf16 bit patterns (uint16), round to nearest even.

    Inputs here are finite; NaN handling is not needed by the recipe.
    """
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def widen(arr) -> np.ndarray:
    """Exact float64 view of an I/O array (uint16 bf16 bits or float32)."""
    arr = np.asarray(arr)
    if arr.dtype == np.uint16:
        return bf16_bits_to_f32(arr).astype(np.float64)
    return arr.astype(np.float64)


def _round(a, io):
    if io == IO_BF16:
        return to_bf16_bits(a)
    if io == IO_F32:
        return a.astype(np.float32)
    raise ValueError(f"unknown io dtype {io!r}")


def _io_dtype(io):
    return np.uint16 if io == IO_BF16 else np.float32


def _softplus(u):
    return np.logaddexp(0.0, u)


def params(d_inner, d_state=16, seed=0, h0=False, batch=1):
    """Per-layer A [d_inner, d_state] fp32, D [d_inner] fp32, optional h0."""
    g = np.random.Generator(np.random.PCG64([seed, PARAM_STREAM]))
    A = (-np.exp(g.uniform(np.log(1.0), np.log(16.0), size=(d_inner, d_state)))).astype(np.float32)
    D = g.standard_normal(size=(d_inner,)).astype(np.float32)
    h = g.standard_normal(size=(batch, d_inner, d_state)).astype(np.float32) if h0 else None
    return A, D, h


def prefill_inputs(batch, L, d_inner, d_state=16, seed=0, io=IO_BF16, h0=False,
                   threads=None, t_begin=0, t_end=None):
    """Token tensors for tokens [t_begin, t_end) of the stream seeded ``seed``.

    Returns a dict with x, delta, z ([batch, T, d_inner]), B, C ([batch, T,
    d_state]) in the I/O dtype (uint16 bf16 bits or float32), plus A, D (fp32)
    and h0 (fp32 or None).  t_begin and t_end must be multiples of CHUNK unless
    they are 0 and L.
    """
    t_end = L if t_end is None else t_end
    T = t_end - t_begin
    dt = _io_dtype(io)
    out = {
        "x": np.empty((batch, T, d_inner), dt),
        "delta": np.empty((batch, T, d_inner), dt),
        "z": np.empty((batch, T, d_inner), dt),
        "B": np.empty((batch, T, d_state), dt),
        "C": np.empty((batch, T, d_state), dt),
    }
    blocks = []
    t = t_begin
    while t < t_end:
        blk = t // CHUNK
        lo = t
        hi = min(t_end, (blk + 1) * CHUNK, L)
        blocks.append((blk, lo, hi))
        t = hi

    def fill(job):
        blk, lo, hi = job
        g = np.random.Generator(np.random.PCG64([seed, blk]))
        full = min(CHUNK, L - blk * CHUNK)       # block length in the stream
        skip = lo - blk * CHUNK
        take = hi - lo
        sl = slice(lo - t_begin, hi - t_begin)
        # The block is always drawn whole and in the fixed order, so a token's
        # values do not depend on which slice was requested.
        for name in ("x", "delta", "z"):
            v = g.standard_normal(size=(batch, full, d_inner))
            if name == "delta":
                v = _softplus(v - 2.0)
            out[name][:, sl, :] = _round(v[:, skip:skip + take, :], io)
            del v
        for name in ("B", "C"):
            v = g.standard_normal(size=(batch, full, d_state)) / 4.0
            out[name][:, sl, :] = _round(v[:, skip:skip + take, :], io)

    n = _threads(threads)
    if n == 1 or len(blocks) == 1:
        for j in blocks:
            fill(j)
    else:
        with _cf.ThreadPoolExecutor(n) as ex:
            list(ex.map(fill, blocks))
    A, D, h = params(d_inner, d_state, seed, h0=h0, batch=batch)
    out["A"], out["D"], out["h0"] = A, D, h
    return out


def prologue_params(d_inner, width, seed=0, batch=1):
    """conv_weight [d_inner, width], conv_bias [d_inner], conv_state
    [batch, width-1, d_inner] and dt_bias [d_inner], all fp32."""
    g = np.random.Generator(np.random.PCG64([seed, PROLOGUE_STREAM]))
    w = (g.standard_normal(size=(d_inner, width)) / np.sqrt(width)).astype(np.float32)
    b = (g.standard_normal(size=(d_inner,)) / 4.0).astype(np.float32)
    st = g.standard_normal(size=(batch, width - 1, d_inner)).astype(np.float32)
    dt0 = np.exp(g.uniform(np.log(1e-3), np.log(1e-1), size=(d_inner,)))
    dtb = np.log(np.expm1(dt0)).astype(np.float32)
    return {"conv_weight": w, "conv_bias": b, "conv_state": st, "dt_bias": dtb}


def rms_weights(d_inner, d_state=16, seed=0):
    """RMSNorm weights for the time step [d_inner] and the B, C rows [d_state],
    ~ U(0.5, 1.5) fp32, from PCG64([seed, PROLOGUE_STREAM, 2])."""
    g = np.random.Generator(np.random.PCG64([seed, PROLOGUE_STREAM, 2]))
    return tuple(g.uniform(0.5, 1.5, size=(n,)).astype(np.float32) for n in (d_inner, d_state, d_state))


def raw_time_steps(batch, L, d_inner, seed=0, io=IO_BF16):
    """Pre-softplus time steps ~ N(0, 1), [batch, L, d_inner] in the I/O dtype."""
    g = np.random.Generator(np.random.PCG64([seed, PROLOGUE_STREAM, 1]))
    return _round(g.standard_normal(size=(batch, L, d_inner)), io)


def output_grads(batch, L, d_inner, d_state=16, seed=0, io=IO_BF16, t_begin=0, t_end=None):
    """dy [batch, T, d_inner] (I/O dtype) for tokens [t_begin, t_end) and dhT
    [batch, d_inner, d_state] fp32.  t_begin, t_end: multiples of CHUNK unless 0, L."""
    t_end = L if t_end is None else t_end
    dy = np.empty((batch, t_end - t_begin, d_inner), _io_dtype(io))
    t = t_begin
    while t < t_end:
        blk = t // CHUNK
        hi = min(t_end, (blk + 1) * CHUNK, L)
        g = np.random.Generator(np.random.PCG64([seed, GRAD_STREAM, blk]))
        full = min(CHUNK, L - blk * CHUNK)
        v = g.standard_normal(size=(batch, full, d_inner))
        dy[:, t - t_begin:hi - t_begin, :] = _round(v[:, t - blk * CHUNK:hi - blk * CHUNK, :], io)
        t = hi
    g = np.random.Generator(np.random.PCG64([seed, GRAD_STREAM]))
    dhT = g.standard_normal(size=(batch, d_inner, d_state)).astype(np.float32)
    return dy, dhT


def trap_inputs(batch, L, d_inner, d_state=16, seed=0, io=IO_BF16):
    """lam [batch, L, d_inner], x_prev [batch, d_inner], B_prev [batch, d_state] (I/O dtype)."""
    g = np.random.Generator(np.random.PCG64([seed, TRAP_STREAM]))
    lam = _round(g.uniform(0.0, 1.0, size=(batch, L, d_inner)), io)
    x_prev = _round(g.standard_normal(size=(batch, d_inner)), io)
    B_prev = _round(g.standard_normal(size=(batch, d_state)) / 4.0, io)
    return lam, x_prev, B_prev


def decode_state(n_seq, d_inner, d_state=16, seed=3):
    g = np.random.Generator(np.random.PCG64([seed, STATE_STREAM]))
    return g.standard_normal(size=(n_seq, d_inner, d_state)).astype(np.float32)


def decode_inputs(n_seq, d_inner, d_state=16, seed=3, step=0, io=IO_BF16):
    """One decode token for each of n_seq sequences (step ``step`` of the run)."""
    g = np.random.Generator(np.random.PCG64([seed, DECODE_STREAM, step]))
    out = {}
    for name in ("x", "delta", "z"):
        v = g.standard_normal(size=(n_seq, d_inner))
        if name == "delta":
            v = _softplus(v - 2.0)
        out[name] = _round(v, io)
    for name in ("B", "C"):
        out[name] = _round(g.standard_normal(size=(n_seq, d_state)) / 4.0, io)
    return out


def channel_slice(inp, channels):
    """The sub-problem made of a subset of channels (channels are independent).

    Returns float64 arrays x, delta, z [batch, T, k], B, C, A [k, N], D [k],
    h0 [batch, k, N] or None, ready for the oracle.
    """
    ch = np.asarray(channels)
    res = {name: widen(inp[name][:, :, ch]) for name in ("x", "delta", "z")}
    res["B"] = widen(inp["B"])
    res["C"] = widen(inp["C"])
    res["A"] = inp["A"][ch].astype(np.float64)
    res["D"] = inp["D"][ch].astype(np.float64)
    res["h0"] = None if inp.get("h0") is None else inp["h0"][:, ch, :].astype(np.float64)
    return res
