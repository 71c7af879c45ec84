"""Pins of the oracle's exponential-trapezoidal variant (Mamba-3's
discretisation as read from the pages), against things other than its own
formula:

* lam = 1 is the Euler recurrence of the main oracle;
* on a linear time-invariant system driven by a smooth input, the final
  state converges to the exact solution of h' = A h + B x(t) (closed form)
  with order 2 in the step (error ratio 4 when the step halves), while the
  Euler form converges with order 1;
* a constant input drives the state to the fixed point of the recurrence;
* a sequence split in two calls, the second fed the first's final state and
  last token, gives the single call's result bit for bit.
"""
import numpy as np
import pytest

import oracle


def problem(seed, batch=2, L=11, d=3, N=16):
    rng = np.random.default_rng(seed)
    return dict(x=rng.standard_normal((batch, L, d)),
                delta=np.log1p(np.exp(rng.standard_normal((batch, L, d)) - 2.0)),
                A=-np.exp(rng.uniform(0.0, np.log(16.0), (d, N))),
                B=rng.standard_normal((batch, L, N)) / 4, C=rng.standard_normal((batch, L, N)) / 4,
                D=rng.standard_normal(d), z=rng.standard_normal((batch, L, d)),
                h0=rng.standard_normal((batch, d, N))), rng


def test_lambda_one_is_euler():
    p, rng = problem(0)
    y1, h1 = oracle.prefill(**p)
    lam = np.ones_like(p["x"])
    y2, h2, _, _ = oracle.prefill_trap(**p, lam=lam, x_prev=rng.standard_normal((2, 3)),
                                       B_prev=rng.standard_normal((2, 16)))
    np.testing.assert_allclose(y2, y1, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(h2, h1, rtol=1e-13, atol=1e-15)


def lti_final_state(L, T, lam_value, omega=3.0):
    """One channel, 16 states, A_n in [-4, -0.5], B_n = 1: sample x(t) = sin(omega t)
    at t_k = (k+1) T / L for token k, with the token before the first at t = 0."""
    A = -np.linspace(0.5, 4.0, 16)[None, :]
    dt = T / L
    t = (np.arange(L) + 1) * dt
    x = np.sin(omega * t)[None, :, None]
    B = np.ones((1, L, 16))
    zeros = np.zeros((1, L, 1))
    lam = np.full((1, L, 1), lam_value)
    _, hT, _, _ = oracle.prefill_trap(x, np.full((1, L, 1), dt), A, B, B, np.zeros(1), zeros, lam=lam,
                                      x_prev=np.zeros((1, 1)), B_prev=np.ones((1, 16)))
    a = A[0]
    exact = (-a * np.sin(omega * T) - omega * np.cos(omega * T) + omega * np.exp(a * T)) / (a * a + omega * omega)
    return np.abs(hT[0, 0] - exact).max()


def test_trapezoid_converges_with_order_two_euler_with_order_one():
    T = 2.0
    e_trap = [lti_final_state(L, T, 0.5) for L in (200, 400, 800)]
    e_euler = [lti_final_state(L, T, 1.0) for L in (200, 400, 800)]
    for k in range(2):
        r_trap = e_trap[k] / e_trap[k + 1]
        r_euler = e_euler[k] / e_euler[k + 1]
        assert 3.6 < r_trap < 4.4, (e_trap, r_trap)
        assert 1.7 < r_euler < 2.3, (e_euler, r_euler)
    assert e_trap[-1] < 1e-4 < e_euler[-1]


@pytest.mark.parametrize("lam_value", [0.5, 0.25, 1.0])
def test_constant_input_reaches_the_fixed_point(lam_value):
    """Delta, B, x constant: h -> dt B x (lam + (1 - lam) a) / (1 - a)."""
    L, dt, xv = 4000, 0.05, 0.7
    A = -np.linspace(0.5, 4.0, 16)[None, :]
    Bv = np.linspace(-1, 1, 16)
    x = np.full((1, L, 1), xv)
    B = np.tile(Bv, (1, L, 1))
    _, hT, _, _ = oracle.prefill_trap(x, np.full((1, L, 1), dt), A, B, B, np.zeros(1), np.zeros((1, L, 1)),
                                      lam=np.full((1, L, 1), lam_value), x_prev=np.full((1, 1), xv),
                                      B_prev=Bv[None, :])
    a = np.exp(dt * A[0])
    fixed = dt * Bv * xv * (lam_value + (1 - lam_value) * a) / (1 - a)
    np.testing.assert_allclose(hT[0, 0], fixed, rtol=1e-10, atol=1e-14)


@pytest.mark.parametrize("split", [1, 5, 10])
def test_split_sequence_carries_state_and_last_token(split):
    p, rng = problem(1)
    lam = rng.uniform(0, 1, p["x"].shape)
    xp, Bp = rng.standard_normal((2, 3)), rng.standard_normal((2, 16))
    y, hT, xl, Bl = oracle.prefill_trap(**p, lam=lam, x_prev=xp, B_prev=Bp)
    first = {k: (v[:, :split] if k in ("x", "delta", "B", "C", "z") else v) for k, v in p.items()}
    second = {k: (v[:, split:] if k in ("x", "delta", "B", "C", "z") else v) for k, v in p.items()}
    y1, h1, xl1, Bl1 = oracle.prefill_trap(**first, lam=lam[:, :split], x_prev=xp, B_prev=Bp)
    second["h0"] = h1
    y2, h2, xl2, Bl2 = oracle.prefill_trap(**second, lam=lam[:, split:], x_prev=xl1, B_prev=Bl1)
    assert np.array_equal(np.concatenate([y1, y2], 1), y)
    assert np.array_equal(h2, hT) and np.array_equal(xl2, xl) and np.array_equal(Bl2, Bl)
    np.testing.assert_array_equal(xl, p["x"][:, -1])
    np.testing.assert_array_equal(Bl, p["B"][:, -1])
