"""Helpers for the GPU parity tests: moving seeded inputs to the device and the
tolerance checks.

Tolerance (the reading used throughout): the output y must match the fp64
oracle with max |y_gpu - y_ref| <= 2e-3 * max |y_ref|.  For bf16 output the
rounding of a perfect result to bf16 alone can reach half a bf16 ulp, which is
between 1.95e-3 and 3.9e-3 of max |y_ref| depending on where max |y_ref|
falls in its binade, so for bf16 each element's error is first reduced by
half a bf16 ulp of that element.  States (hT, decode state) are fp32 and are
held to 2e-3 * max |ref| as stated.
"""
from __future__ import annotations

import numpy as np
import torch

import synth

REL_TOL = 2e-3


def dev_io(a, device="cuda"):
    """numpy I/O array (uint16 bf16 bits or float32) -> device tensor (bf16 or f32)."""
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a)
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device)


def dev_f32(a, device="cuda"):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)


def to_device(inp, device="cuda"):
    out = {k: dev_io(inp[k], device) for k in ("x", "delta", "z", "B", "C")}
    out["A"] = dev_f32(inp["A"], device)
    out["D"] = dev_f32(inp["D"], device)
    out["h0"] = dev_f32(inp.get("h0"), device)
    return out


def host64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_half_ulp(v):
    """Half a bf16 ulp at |v| (normal range): 2^(floor(log2|v|) - 8)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 8)


def y_error(y_gpu, y_ref, bf16: bool):
    """Return (criterion ratio, raw ratio): both must be <= REL_TOL to pass the
    criterion (raw is reported, not required for bf16)."""
    yg = y_gpu if isinstance(y_gpu, np.ndarray) else host64(y_gpu)
    scale = max(float(np.max(np.abs(y_ref))), 1e-30)
    err = np.abs(yg - y_ref)
    raw = float(np.max(err)) / scale if err.size else 0.0
    if bf16:
        # half a bf16 ulp of the reference: a correctly rounded result is
        # within it, also where it rounds up to the next power of two
        err = np.maximum(err - bf16_half_ulp(y_ref), 0.0)
    crit = float(np.max(err)) / scale if err.size else 0.0
    return crit, raw


def assert_y(y_gpu, y_ref, bf16: bool, what="y"):
    crit, raw = y_error(y_gpu, y_ref, bf16)
    assert np.all(np.isfinite(host64(y_gpu) if not isinstance(y_gpu, np.ndarray) else y_gpu)), f"{what}: non-finite"
    assert crit <= REL_TOL, f"{what}: error {crit:.3e} (raw {raw:.3e}) of max|ref| > {REL_TOL}"
    return crit, raw


def assert_state(h_gpu, h_ref, what="state"):
    hg = h_gpu if isinstance(h_gpu, np.ndarray) else host64(h_gpu)
    scale = max(float(np.max(np.abs(h_ref))), 1e-30)
    err = float(np.max(np.abs(hg - h_ref))) / scale if hg.size else 0.0
    assert err <= REL_TOL, f"{what}: error {err:.3e} of max|ref| > {REL_TOL}"
    return err


def oracle_inputs(inp):
    """All channels of a (small) problem as float64 for the oracle."""
    return {"x": synth.widen(inp["x"]), "delta": synth.widen(inp["delta"]), "z": synth.widen(inp["z"]),
            "B": synth.widen(inp["B"]), "C": synth.widen(inp["C"]), "A": inp["A"].astype(np.float64),
            "D": inp["D"].astype(np.float64),
            "h0": None if inp.get("h0") is None else inp["h0"].astype(np.float64)}


def n_star(t):
    """Hash of a token index into 0..15 (not t mod 16, so offsets that are
    multiples of 16 tokens are distinguished)."""
    t = torch.as_tensor(t)
    return ((t * 7) + (t >> 4) * 5 + (t >> 8) * 3 + (t >> 12)) & 15
