"""Pins for the fp64 oracle: checks against brute force, closed forms, a library
IIR filter and invariants -- never against the oracle itself.

The recurrence under test is the selective state-space scan of the
"AI Engineering from Scratch" Jamba lesson (section "一页讲完 SSM"):
h_t = exp(delta_t*A) h_{t-1} + delta_t*B_t*x_t, y_t = C_t.h_t, plus the D skip,
gated by SiLU(z_t).  Each test below is chosen so that a plausible mistake in the
oracle (a dropped term, a sign, an off-by-one token index, a transposed A, the
gate in the wrong place) breaks at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.signal
import torch
from hypothesis import given, settings, strategies as st

import oracle
from oracle import twin


def silu_lib(z):
    """SiLU from torch (an independent library implementation), in float64."""
    return torch.nn.functional.silu(torch.as_tensor(np.asarray(z, np.float64))).numpy()


def rand_problem(rng, batch, L, d_inner, d_state, h0=True):
    x = rng.standard_normal((batch, L, d_inner))
    delta = np.logaddexp(0.0, rng.standard_normal((batch, L, d_inner)) - 2.0)
    z = rng.standard_normal((batch, L, d_inner))
    A = -np.exp(rng.uniform(0.0, np.log(16.0), (d_inner, d_state)))
    B = rng.standard_normal((batch, L, d_state)) / 4
    C = rng.standard_normal((batch, L, d_state)) / 4
    D = rng.standard_normal(d_inner)
    h = rng.standard_normal((batch, d_inner, d_state)) if h0 else None
    return dict(x=x, delta=delta, A=A, B=B, C=C, D=D, z=z, h0=h)


def run_oracle(p):
    return oracle.prefill(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["h0"])


def brute_force(p):
    """Unrolled sums: every decay product is ONE exp of a summed delta.

    y_t = silu(z_t) * [ sum_n C_tn ( exp(A_n S(0,t)) h0_n
                                     + sum_{s<=t} exp(A_n S(s,t)) delta_s B_sn x_s )
                        + D x_t ]
    with S(s,t) = sum_{s<r<=t} delta_r and S(0,t) = sum_{r<=t} delta_r.
    """
    x, dl, A, B, C, D, z, h0 = (p[k] for k in ("x", "delta", "A", "B", "C", "D", "z", "h0"))
    batch, L, d_inner = x.shape
    N = A.shape[1]
    y = np.zeros((batch, L, d_inner))
    hT = np.zeros((batch, d_inner, N))
    for b in range(batch):
        for d in range(d_inner):
            cum = np.concatenate([[0.0], np.cumsum(dl[b, :, d])])    # cum[t+1] = sum_{r<=t}
            for t in range(L):
                tot = 0.0
                for n in range(N):
                    hv = 0.0 if h0 is None else math.exp(A[d, n] * cum[t + 1]) * h0[b, d, n]
                    for s in range(t + 1):
                        hv += math.exp(A[d, n] * (cum[t + 1] - cum[s + 1])) * dl[b, s, d] * B[b, s, n] * x[b, s, d]
                    tot += C[b, t, n] * hv
                    if t == L - 1:
                        hT[b, d, n] = hv
                y[b, t, d] = tot + D[d] * x[b, t, d]
            y[b, :, d] *= silu_lib(z[b, :, d])
    return y, hT


def rel_err(a, b):
    scale = max(np.max(np.abs(b)), 1e-300)
    return np.max(np.abs(a - b)) / scale


@settings(max_examples=20, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), batch=st.integers(1, 2), L=st.integers(1, 14),
       d_inner=st.integers(1, 3), d_state=st.sampled_from([1, 3, 16]), h0=st.booleans())
def test_oracle_matches_brute_force(seed, batch, L, d_inner, d_state, h0):
    p = rand_problem(np.random.default_rng(seed), batch, L, d_inner, d_state, h0)
    y, hT = run_oracle(p)
    yb, hb = brute_force(p)
    assert rel_err(y, yb) < 1e-12
    assert rel_err(hT, hb) < 1e-12


def test_oracle_brute_force_jamba_state_width():
    """d_state 16 and d_inner 5 != 16, so a transposed A cannot pass."""
    p = rand_problem(np.random.default_rng(7), 2, 24, 5, 16, True)
    y, hT = run_oracle(p)
    yb, hb = brute_force(p)
    assert rel_err(y, yb) < 1e-12
    assert rel_err(hT, hb) < 1e-12


def lti_problem(rng, L, d_inner, N):
    p = rand_problem(rng, 1, L, d_inner, N, True)
    # delta, B, C constant over time: the scan is a linear time-invariant filter
    p["delta"] = np.broadcast_to(p["delta"][:, :1, :], p["delta"].shape).copy()
    p["B"] = np.broadcast_to(p["B"][:, :1, :], p["B"].shape).copy()
    p["C"] = np.broadcast_to(p["C"][:, :1, :], p["C"].shape).copy()
    return p


def test_lti_matches_scipy_lfilter():
    """Constant delta, B, C: per (d, n) the state is the first-order IIR filter
    h_t = abar h_{t-1} + (delta B) x_t, run here by scipy.signal.lfilter with the
    initial condition set from h0."""
    rng = np.random.default_rng(11)
    L, d_inner, N = 300, 4, 16
    p = lti_problem(rng, L, d_inner, N)
    y, hT = run_oracle(p)
    for d in range(d_inner):
        dt = p["delta"][0, 0, d]
        yp = np.zeros(L)
        for n in range(N):
            abar = math.exp(dt * p["A"][d, n])
            beta = dt * p["B"][0, 0, n]
            h, _ = scipy.signal.lfilter([beta], [1.0, -abar], p["x"][0, :, d], zi=[abar * p["h0"][0, d, n]])
            np.testing.assert_allclose(hT[0, d, n], h[-1], rtol=1e-11, atol=1e-14)
            yp += p["C"][0, 0, n] * h
        yp = (yp + p["D"][d] * p["x"][0, :, d]) * silu_lib(p["z"][0, :, d])
        assert rel_err(y[0, :, d], yp) < 1e-11


def test_lti_matches_long_convolution():
    """The S4 view of the same lesson: an LTI SSM is a long convolution with kernel
    K_k = sum_n C_n abar_n^k delta B_n, plus the free response of h0."""
    rng = np.random.default_rng(12)
    L, d_inner, N = 257, 3, 16
    p = lti_problem(rng, L, d_inner, N)
    y, _ = run_oracle(p)
    k = np.arange(L)
    for d in range(d_inner):
        dt = p["delta"][0, 0, d]
        abar = np.exp(dt * p["A"][d])                      # [N]
        Cn, Bn = p["C"][0, 0], p["B"][0, 0]
        K = (Cn[None, :] * abar[None, :] ** k[:, None] * dt * Bn[None, :]).sum(1)
        yp = np.convolve(p["x"][0, :, d], K)[:L]
        free = (Cn[None, :] * abar[None, :] ** (k[:, None] + 1) * p["h0"][0, d][None, :]).sum(1)
        yp = (yp + free + p["D"][d] * p["x"][0, :, d]) * silu_lib(p["z"][0, :, d])
        assert rel_err(y[0, :, d], yp) < 1e-11


def test_zero_input_pure_decay():
    """x = 0 with time-varying delta: h_T = exp(A * sum_t delta_t) h0."""
    rng = np.random.default_rng(13)
    p = rand_problem(rng, 2, 97, 6, 16, True)
    p["x"][:] = 0.0
    y, hT = run_oracle(p)
    S = p["delta"].sum(axis=1)                            # [batch, d_inner]
    expect = np.exp(S[:, :, None] * p["A"][None]) * p["h0"]
    np.testing.assert_allclose(hT, expect, rtol=1e-12, atol=1e-300)


def test_impulse_and_step_closed_forms():
    """Constant delta and B, h0 = 0.  Impulse x = e_0: h_t = abar^t delta B.
    Unit step x = 1: h_t = delta B (1 - abar^(t+1)) / (1 - abar)."""
    L, N = 40, 16
    rng = np.random.default_rng(14)
    A = -np.exp(rng.uniform(0.0, np.log(16.0), (1, N)))
    dt = 0.07
    Bv = rng.standard_normal(N) / 4
    base = dict(delta=np.full((1, L, 1), dt), A=A, B=np.tile(Bv, (1, L, 1)),
                C=np.zeros((1, L, N)), D=np.zeros(1), z=np.full((1, L, 1), 50.0), h0=None)
    abar = np.exp(dt * A[0])
    for t_end in (1, 17, L):
        imp = dict(base, x=np.zeros((1, t_end, 1)))
        imp["x"][0, 0, 0] = 1.0
        for key in ("delta", "B", "C", "z"):
            imp[key] = base[key][:, :t_end]
        _, hT = run_oracle(imp)
        np.testing.assert_allclose(hT[0, 0], abar ** (t_end - 1) * dt * Bv, rtol=1e-13)
        stp = dict(imp, x=np.ones((1, t_end, 1)))
        _, hT = run_oracle(stp)
        np.testing.assert_allclose(hT[0, 0], dt * Bv * (1 - abar ** t_end) / (1 - abar), rtol=1e-12)


def test_output_reads_state_through_C_and_D_skip():
    """Impulse response read out through a one-hot C, with the D skip and a
    saturated gate (z = 50: SiLU(z) = z exactly in float64)."""
    L, N = 12, 16
    rng = np.random.default_rng(15)
    A = -np.exp(rng.uniform(0.0, np.log(16.0), (1, N)))
    dt, Bv, Dd = 0.3, rng.standard_normal(N), 0.75
    C = np.zeros((1, L, N))
    picks = [(3 * t + 5) % N for t in range(L)]
    for t, n in enumerate(picks):
        C[0, t, n] = 1.0
    x = np.zeros((1, L, 1)); x[0, 0, 0] = 2.0
    y, _ = oracle.prefill(x, np.full((1, L, 1), dt), A, np.tile(Bv, (1, L, 1)), C,
                          np.array([Dd]), np.full((1, L, 1), 50.0))
    abar = np.exp(dt * A[0])
    for t, n in enumerate(picks):
        expect = abar[n] ** t * dt * Bv[n] * 2.0 + (Dd * 2.0 if t == 0 else 0.0)
        assert abs(y[0, t, 0] - 50.0 * expect) <= 1e-13 * max(1.0, abs(50.0 * expect))


def test_gate_zero_and_saturated():
    p = rand_problem(np.random.default_rng(16), 1, 30, 4, 16, True)
    p["z"][:] = 0.0
    y, _ = run_oracle(p)
    assert np.all(y == 0.0)
    # z = 40: 1 + exp(-40) rounds to 1 in float64, so y = z * (C.h + D x) exactly
    p["z"][:] = 40.0
    y40, _ = run_oracle(p)
    p["z"][:] = 1.0
    y1, _ = run_oracle(p)
    s1 = silu_lib(np.array([1.0]))[0]
    np.testing.assert_allclose(y40 / 40.0, y1 / s1, rtol=1e-13)


def test_silu_matches_library():
    """The gate value for a range of z against torch's SiLU (C = 0, D = 1, x = 1)."""
    zs = np.linspace(-30, 30, 241)
    L = zs.size
    y, _ = oracle.prefill(np.ones((1, L, 1)), np.full((1, L, 1), 0.1), -np.ones((1, 16)),
                          np.zeros((1, L, 16)), np.zeros((1, L, 16)), np.ones(1), zs.reshape(1, L, 1))
    np.testing.assert_allclose(y[0, :, 0], silu_lib(zs), rtol=1e-14, atol=1e-300)


def test_prefill_final_state_equals_chained_steps():
    """The lesson's point that inference costs O(1) per token with a fixed-size
    state: the prefill's final state equals T chained decode steps, bitwise (the
    two C functions update the state with the same operations in the same
    order); the outputs agree to rounding (the step groups the gate product as
    (C.h + D x) * SiLU(z))."""
    rng = np.random.default_rng(17)
    batch, L, d_inner, N = 3, 50, 7, 16
    p = rand_problem(rng, batch, L, d_inner, N, True)
    y, hT = run_oracle(p)
    state = p["h0"].copy()
    for t in range(L):
        ys, state = oracle.step(state, p["x"][:, t], p["delta"][:, t], p["A"], p["B"][:, t],
                                p["C"][:, t], p["D"], p["z"][:, t])
        np.testing.assert_allclose(ys, y[:, t], rtol=1e-15, atol=1e-300)
    np.testing.assert_array_equal(state, hT)


def test_chunked_prefill_equals_single_call():
    """Carrying hT into h0 across calls is the same sequential arithmetic."""
    rng = np.random.default_rng(18)
    p = rand_problem(rng, 2, 96, 5, 16, True)
    y, hT = run_oracle(p)
    h = p["h0"]
    ys = []
    for lo, hi in ((0, 31), (31, 64), (64, 96)):
        sl = slice(lo, hi)
        yc, h = oracle.prefill(p["x"][:, sl], p["delta"][:, sl], p["A"], p["B"][:, sl], p["C"][:, sl],
                               p["D"], p["z"][:, sl], h)
        ys.append(yc)
    np.testing.assert_array_equal(np.concatenate(ys, axis=1), y)
    np.testing.assert_array_equal(h, hT)


def test_linearity_in_input_and_initial_state():
    rng = np.random.default_rng(19)
    p1 = rand_problem(rng, 1, 40, 4, 16, True)
    p2 = dict(p1, x=rng.standard_normal(p1["x"].shape), h0=rng.standard_normal(p1["h0"].shape))
    a, b = 0.7, -1.3
    p3 = dict(p1, x=a * p1["x"] + b * p2["x"], h0=a * p1["h0"] + b * p2["h0"])
    y1, h1 = run_oracle(p1)
    y2, h2 = run_oracle(p2)
    y3, h3 = run_oracle(p3)
    assert rel_err(y3, a * y1 + b * y2) < 1e-12
    assert rel_err(h3, a * h1 + b * h2) < 1e-12


def test_causality_and_channel_independence():
    rng = np.random.default_rng(20)
    p = rand_problem(rng, 2, 60, 6, 16, True)
    y, _ = run_oracle(p)
    q = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
    q["x"][1, 33, 4] += 1.0
    yq, _ = run_oracle(q)
    np.testing.assert_array_equal(yq[:, :33], y[:, :33])
    changed = yq != y
    assert changed[1, 33:, 4].all()
    changed[1, 33:, 4] = False
    assert not changed.any()


def test_batch_permutation_and_nan_locality():
    rng = np.random.default_rng(21)
    p = rand_problem(rng, 3, 25, 4, 16, True)
    y, hT = run_oracle(p)
    perm = [2, 0, 1]
    q = {k: (v[perm] if k in ("x", "delta", "z", "B", "C", "h0") else v) for k, v in p.items()}
    yq, hq = run_oracle(q)
    np.testing.assert_array_equal(yq, y[perm])
    np.testing.assert_array_equal(hq, hT[perm])
    q = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
    q["x"][1, 10, 2] = np.nan
    yn, hn = run_oracle(q)
    bad = np.isnan(yn)
    assert bad[1, 10:, 2].all()
    bad[1, 10:, 2] = False
    assert not bad.any()
    mask = np.ones_like(y, bool); mask[1, 10:, 2] = False
    np.testing.assert_array_equal(yn[mask], y[mask])


def test_numpy_twin_agrees_with_c_oracle():
    rng = np.random.default_rng(22)
    p = rand_problem(rng, 2, 70, 9, 16, True)
    y, hT = run_oracle(p)
    yt, ht = twin.prefill(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["h0"])
    assert rel_err(yt, y) < 1e-14
    assert rel_err(ht, hT) < 1e-14


def test_empty_sequence_keeps_state():
    rng = np.random.default_rng(23)
    p = rand_problem(rng, 2, 0, 3, 16, True)
    y, hT = run_oracle(p)
    assert y.shape == (2, 0, 3)
    np.testing.assert_array_equal(hT, p["h0"])


def test_thread_count_does_not_change_result():
    rng = np.random.default_rng(24)
    p = rand_problem(rng, 2, 64, 33, 16, True)
    n0 = oracle.num_threads()
    try:
        oracle.set_num_threads(1)
        y1, h1 = run_oracle(p)
        oracle.set_num_threads(max(2, n0))
        y2, h2 = run_oracle(p)
    finally:
        oracle.set_num_threads(n0)
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_array_equal(h1, h2)


# ------------------------------------------------------------ input prologue
def prologue_problem(rng, batch, L, d_inner, width):
    x = rng.standard_normal((batch, L, d_inner))
    delta = rng.standard_normal((batch, L, d_inner)) - 2.0
    w = rng.standard_normal((d_inner, width)) / width
    bias = rng.standard_normal(d_inner) / 4
    state = rng.standard_normal((batch, width - 1, d_inner))
    dt_bias = rng.standard_normal(d_inner) / 2
    return x, delta, w, bias, state, dt_bias


@pytest.mark.parametrize("width", [1, 2, 4])
def test_prologue_conv_matches_scipy_fir(width):
    """Causal depthwise convolution = an FIR filter per channel (scipy.signal.lfilter
    with taps reversed), run over the history prepended to the sequence."""
    rng = np.random.default_rng(30 + width)
    x, delta, w, bias, state, _ = prologue_problem(rng, 2, 57, 5, width)
    xc, _, st_out = oracle.prologue(x, delta, w, bias, state)
    for b in range(2):
        for d in range(5):
            seq = np.concatenate([state[b, :, d], x[b, :, d]])
            pre = scipy.signal.lfilter(w[d, ::-1], [1.0], seq)[width - 1:] + bias[d]
            np.testing.assert_allclose(xc[b, :, d], silu_lib(pre), rtol=1e-13, atol=1e-15)
            np.testing.assert_array_equal(st_out[b, :, d], seq[len(seq) - (width - 1):])


def test_prologue_conv_zero_history_and_no_conv():
    rng = np.random.default_rng(34)
    x, delta, w, bias, _, _ = prologue_problem(rng, 1, 20, 3, 4)
    xc, dout, st = oracle.prologue(x, delta, w, None, None)
    for d in range(3):
        pre = np.convolve(x[0, :, d], w[d, ::-1])[:20]          # zero history, no bias
        np.testing.assert_allclose(xc[0, :, d], silu_lib(pre), rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(dout, delta)                   # softplus off: delta passes through
    xc2, _, st2 = oracle.prologue(x, delta)                       # no convolution: x passes through
    np.testing.assert_array_equal(xc2, x)
    assert st2 is None


def test_prologue_softplus_matches_library():
    rng = np.random.default_rng(35)
    x, delta, _, _, _, dt_bias = prologue_problem(rng, 2, 40, 6, 4)
    delta[0, 0, 0], delta[0, 1, 0] = -40.0, 15.0               # far tails of softplus
    _, dout, _ = oracle.prologue(x, delta, dt_bias=dt_bias, softplus=True)
    v = torch.as_tensor(delta + dt_bias[None, None, :])
    ref = torch.nn.functional.softplus(v, threshold=50.0).numpy()
    np.testing.assert_allclose(dout, ref, rtol=1e-13, atol=0)
    assert np.all(dout > 0)


def test_prologue_state_carry_equals_one_call():
    """Splitting the sequence and carrying the conv state gives the same bits."""
    rng = np.random.default_rng(36)
    x, delta, w, bias, state, dt_bias = prologue_problem(rng, 2, 61, 4, 4)
    xc, dout, st = oracle.prologue(x, delta, w, bias, state, dt_bias, True)
    xa, da, sa = oracle.prologue(x[:, :2], delta[:, :2], w, bias, state, dt_bias, True)   # shorter than the window
    xb, db, sb = oracle.prologue(x[:, 2:30], delta[:, 2:30], w, bias, sa, dt_bias, True)
    xz, dz, sz = oracle.prologue(x[:, 30:], delta[:, 30:], w, bias, sb, dt_bias, True)
    np.testing.assert_array_equal(np.concatenate([xa, xb, xz], axis=1), xc)
    np.testing.assert_array_equal(np.concatenate([da, db, dz], axis=1), dout)
    np.testing.assert_array_equal(sz, st)


# ------------------------------------------------------------ input RMSNorm
def test_rmsnorm_inputs_matches_torch_rms_norm():
    """Against torch.nn.functional.rms_norm (float64) over the last dimension."""
    import torch
    rng = np.random.default_rng(70)
    delta = rng.standard_normal((2, 7, 40))
    B = rng.standard_normal((2, 7, 16)) / 4
    C = rng.standard_normal((2, 7, 16)) * 3
    w_dt, w_B, w_C = rng.uniform(0.5, 2, 40), rng.uniform(0.5, 2, 16), rng.uniform(0.5, 2, 16)
    eps = 1e-5
    d2, B2, C2 = oracle.rmsnorm_inputs(delta, B, C, w_dt, w_B, w_C, eps)
    ref = lambda v, w: torch.nn.functional.rms_norm(torch.tensor(v), (v.shape[-1],), torch.tensor(w), eps).numpy()
    np.testing.assert_allclose(d2, ref(delta, w_dt), rtol=1e-13)
    np.testing.assert_allclose(B2, ref(B, w_B), rtol=1e-13)
    np.testing.assert_allclose(C2, ref(C, w_C), rtol=1e-13)


def test_rmsnorm_inputs_properties():
    """Unit weights give unit root-mean-square (eps = 0); a positive scale of the
    input does not change the output; a missing weight leaves the tensor as is."""
    rng = np.random.default_rng(71)
    delta = rng.standard_normal((1, 5, 33))
    B = rng.standard_normal((1, 5, 16))
    C = rng.standard_normal((1, 5, 16))
    d2, B2, _ = oracle.rmsnorm_inputs(delta, B, C, np.ones(33), np.ones(16), None, eps=0.0)
    np.testing.assert_allclose(np.sqrt((d2 ** 2).mean(-1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(np.sqrt((B2 ** 2).mean(-1)), 1.0, rtol=1e-14)
    d3, B3, C3 = oracle.rmsnorm_inputs(7.5 * delta, 0.01 * B, C, np.ones(33), np.ones(16), None, eps=0.0)
    np.testing.assert_allclose(d3, d2, rtol=1e-13)
    np.testing.assert_allclose(B3, B2, rtol=1e-13)
    assert np.array_equal(C3, C)
