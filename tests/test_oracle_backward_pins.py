"""Pins of the oracle's backward (gradient) scan, each against something other
than the backward's own formulas:

* central finite differences of the oracle's forward, along random directions
  in each input separately (a dropped or mis-signed term in any gradient
  shows up in its own direction);
* reverse-mode automatic differentiation (torch.autograd, float64) of a plain
  token-by-token forward loop written here from the recurrence;
* special cases with closed forms (no input term, no state);
* the chain rule across a split sequence: the gradient of the first part's
  final state is the second part's dh0.
"""
import numpy as np
import pytest
import torch

import oracle

NAMES = {"x": "dx", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz", "h0": "dh0"}


def problem(seed, batch=2, L=9, d=3, N=16):
    rng = np.random.default_rng(seed)
    p = dict(x=rng.standard_normal((batch, L, d)),
             delta=np.log1p(np.exp(rng.standard_normal((batch, L, d)) - 2.0)),
             A=-np.exp(rng.uniform(0.0, np.log(16.0), (d, N))),
             B=rng.standard_normal((batch, L, N)) / 4, C=rng.standard_normal((batch, L, N)) / 4,
             D=rng.standard_normal(d), z=rng.standard_normal((batch, L, d)),
             h0=rng.standard_normal((batch, d, N)))
    dy = rng.standard_normal((batch, L, d))
    dhT = rng.standard_normal((batch, d, N))
    return p, dy, dhT, rng


def loss(p, dy, dhT):
    y, hT = oracle.prefill(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["h0"])
    return float((y * dy).sum() + (0.0 if dhT is None else (hT * dhT).sum()))


def grads(p, dy, dhT):
    return oracle.backward(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], dy, p["h0"], dhT)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("with_dhT", [True, False])
def test_backward_matches_finite_differences(seed, with_dhT):
    p, dy, dhT, rng = problem(seed)
    dhT = dhT if with_dhT else None
    g = grads(p, dy, dhT)
    for name in NAMES:
        for _ in range(2):
            v = rng.standard_normal(p[name].shape)
            eps = 1e-6
            hi = dict(p); hi[name] = p[name] + eps * v
            lo = dict(p); lo[name] = p[name] - eps * v
            fd = (loss(hi, dy, dhT) - loss(lo, dy, dhT)) / (2 * eps)
            an = float((g[NAMES[name]] * v).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def torch_forward(p):
    """Plain float64 loop over tokens and states, written from the recurrence."""
    x, dl, A, B, C, D, z, h0 = (p[k] for k in ("x", "delta", "A", "B", "C", "D", "z", "h0"))
    batch, L, d = x.shape
    ys = []
    h = h0
    for t in range(L):
        dt = dl[:, t, :]                                   # [batch, d]
        a = torch.exp(dt[:, :, None] * A[None])            # [batch, d, N]
        h = a * h + (dt * x[:, t, :])[:, :, None] * B[:, t, None, :]
        yt = (h * C[:, t, None, :]).sum(-1) + D[None] * x[:, t, :]
        ys.append(yt * torch.nn.functional.silu(z[:, t, :]))
    return torch.stack(ys, 1), h


@pytest.mark.parametrize("seed", [3, 4])
def test_backward_matches_autograd(seed):
    p, dy, dhT, _ = problem(seed, batch=2, L=6, d=4)
    tp = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in p.items()}
    y, hT = torch_forward(tp)
    (y * torch.tensor(dy)).sum().add((hT * torch.tensor(dhT)).sum()).backward()
    g = grads(p, dy, dhT)
    for name, gname in NAMES.items():
        ref = tp[name].grad.numpy()
        np.testing.assert_allclose(g[gname], ref, rtol=1e-10, atol=1e-12, err_msg=name)


def test_backward_without_input_term_or_state():
    """B = 0 and h0 = 0 leave the state at zero: y = D x SiLU(z), so dx, dz and
    dD have closed forms and dA, dC, ddelta, dh0 (with dhT = 0) vanish."""
    p, dy, _, _ = problem(5)
    p["B"][:] = 0.0
    p["h0"][:] = 0.0
    g = grads(p, dy, None)
    s = 1.0 / (1.0 + np.exp(-p["z"]))
    silu = p["z"] * s
    np.testing.assert_allclose(g["dx"], p["D"] * silu * dy, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(g["dD"], (p["x"] * silu * dy).sum(axis=(0, 1)), rtol=1e-12)
    np.testing.assert_allclose(g["dz"], dy * p["D"] * p["x"] * s * (1 + p["z"] * (1 - s)), rtol=1e-12, atol=1e-15)
    for k in ("dA", "dC", "ddelta"):
        assert np.all(g[k] == 0.0), k
    # the adjoint still flows (it does not depend on B), so dh0 = a_0 * lambda_0 is not zero
    assert np.any(g["dh0"] != 0.0)


@pytest.mark.parametrize("split", [1, 4, 8])
def test_backward_chain_rule_across_a_split(split):
    """Gradients of one call over L tokens equal those of two calls over
    [0, split) and [split, L), where the second call's dh0 is the first call's
    dhT: per-token gradients concatenate, parameter gradients add."""
    p, dy, dhT, _ = problem(6, L=9)
    full = grads(p, dy, dhT)
    first = {k: (v[:, :split] if k in ("x", "delta", "B", "C", "z") else v) for k, v in p.items()}
    second = {k: (v[:, split:] if k in ("x", "delta", "B", "C", "z") else v) for k, v in p.items()}
    _, hmid = oracle.prefill(first["x"], first["delta"], p["A"], first["B"], first["C"], p["D"], first["z"], p["h0"])
    second["h0"] = hmid
    g2 = grads(second, dy[:, split:], dhT)
    g1 = grads(first, dy[:, :split], g2["dh0"])
    for k in ("dx", "ddelta", "dz", "dB", "dC"):
        np.testing.assert_allclose(np.concatenate([g1[k], g2[k]], 1), full[k], rtol=1e-11, atol=1e-13, err_msg=k)
    for k in ("dA", "dD"):
        np.testing.assert_allclose(g1[k] + g2[k], full[k], rtol=1e-11, atol=1e-13, err_msg=k)
    np.testing.assert_allclose(g1["dh0"], full["dh0"], rtol=1e-11, atol=1e-13)


def test_backward_thread_count_does_not_change_results():
    p, dy, dhT, _ = problem(7, batch=3, L=40, d=13)
    n = oracle.num_threads()
    try:
        oracle.set_num_threads(1)
        g1 = grads(p, dy, dhT)
        oracle.set_num_threads(max(2, n))
        g2 = grads(p, dy, dhT)
    finally:
        oracle.set_num_threads(n)
    for k in g1:
        # per-channel outputs are bitwise; cross-channel sums may be added in another order
        np.testing.assert_allclose(g1[k], g2[k], rtol=1e-13, atol=1e-15, err_msg=k)
