"""numpy twin of the fp64 oracle, for small shapes.

TEST INFRASTRUCTURE ONLY.  Same definition as ``jscan_oracle.c``: the selective
state-space recurrence (decay exp(delta*A), input delta*B*x, output C.h plus the
D skip, times SiLU(z)), from the "AI Engineering from Scratch" Jamba lesson,
section "一页讲完 SSM".  The only difference is that the channel loop is a
numpy axis; the token loop and the order of the sum over states are the same.
"""
from __future__ import annotations

import numpy as np


def prefill(x, delta, A, B, C, D, z, h0=None):
    x = np.asarray(x, np.float64)
    delta = np.asarray(delta, np.float64)
    z = np.asarray(z, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    D = np.asarray(D, np.float64)
    batch, L, d_inner = x.shape
    d_state = A.shape[1]
    h = np.zeros((batch, d_inner, d_state)) if h0 is None else np.array(h0, np.float64)
    y = np.empty((batch, L, d_inner))
    for t in range(L):
        dt = delta[:, t, :, None]                       # [batch, d_inner, 1]
        xv = x[:, t, :, None]
        h = np.exp(dt * A[None]) * h + dt * B[:, t, None, :] * xv
        acc = np.zeros((batch, d_inner))
        for n in range(d_state):                         # same summation order as the C loop
            acc = acc + C[:, t, None, n] * h[:, :, n]
        zv = z[:, t, :]
        y[:, t, :] = (acc + D[None] * x[:, t, :]) * zv / (1.0 + np.exp(-zv))
    return y, h
