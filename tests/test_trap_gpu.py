"""GPU parity of the exponential-trapezoidal recurrence (Mamba-3's
discretisation as read from the pages) against the fp64 oracle's
``prefill_trap``.

Inputs: the scan's seeded recipe (``synth.prefill_inputs``) plus lam ~ U(0, 1)
and the token before the first (x_prev, B_prev) from ``synth.trap_inputs``;
with softplus, raw time steps from ``synth.raw_time_steps``.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import selective_state_space_11_amd as js
from gpu_util import assert_state, assert_y, dev_f32, dev_io, host64, oracle_inputs, to_device

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only machines, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)


def print_case(msg):
    print(f"[case] {msg}", flush=True)


def with_plan(chunks, fn):
    try:
        js.set_plan_override(1, chunks)
        return fn()
    finally:
        js.set_plan_override(0, 0)


def problem(batch, L, d, seed, io, h0=True, softplus=False):
    inp = synth.prefill_inputs(batch, L, d, seed=seed, io=io, h0=h0)
    if softplus:
        inp["delta"] = synth.raw_time_steps(batch, L, d, seed=seed, io=io)
    lam, xp, Bp = synth.trap_inputs(batch, L, d, seed=seed, io=io)
    dtb = synth.prologue_params(d, 4, seed=seed)["dt_bias"] if softplus else None
    return inp, lam, xp, Bp, dtb


def oracle_trap(inp, lam, xp, Bp, dtb, use_lam=True, use_prev=True):
    o = oracle_inputs(inp)
    dt = o["delta"]
    if dtb is not None:
        _, dt, _ = oracle.prologue(o["x"], o["delta"], dt_bias=dtb, softplus=True)
    y, hT, _, _ = oracle.prefill_trap(o["x"], dt, o["A"], o["B"], o["C"], o["D"], o["z"], o["h0"],
                                      lam=synth.widen(lam) if use_lam else None,
                                      x_prev=synth.widen(xp) if use_prev else None,
                                      B_prev=synth.widen(Bp) if use_prev else None)
    return y, hT


def gpu_trap(t, lam, xp, Bp, dtb, use_lam=True, use_prev=True, **kw):
    y, hT = js.prefill_trap(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"],
                            lam=dev_io(lam) if use_lam else None, x_prev=dev_io(xp) if use_prev else None,
                            B_prev=dev_io(Bp) if use_prev else None,
                            dt_bias=dev_f32(dtb) if dtb is not None else None, softplus=dtb is not None, **kw)
    torch.cuda.synchronize()
    return y, hT


@pytest.mark.parametrize("chunks", [1, 3, 7])
def test_trap_tiny_f32(chunks):
    print_case(f"trap tiny f32 chunks={chunks}")
    inp, lam, xp, Bp, dtb = problem(1, 256, 64, seed=40, io=synth.IO_F32)
    yr, hr = oracle_trap(inp, lam, xp, Bp, dtb)
    y, hT = with_plan(chunks, lambda: gpu_trap(to_device(inp), lam, xp, Bp, dtb))
    assert_y(y, yr, bf16=False)
    assert_state(hT, hr, "hT")


@pytest.mark.parametrize("chunks", [0, 1, 5])
@pytest.mark.parametrize("use_lam,use_prev,softplus", [(True, True, False), (False, False, False),
                                                       (True, False, True), (False, True, True)])
def test_trap_ragged_bf16(chunks, use_lam, use_prev, softplus):
    """Two sequences, L 777, d_inner 200, h0; lam / token-before given or not,
    with and without softplus(delta + dt_bias); automatic (0) and forced plans."""
    print_case(f"trap ragged bf16 chunks={chunks} lam={use_lam} prev={use_prev} softplus={softplus}")
    inp, lam, xp, Bp, dtb = problem(2, 777, 200, seed=41, io=synth.IO_BF16, softplus=softplus)
    yr, hr = oracle_trap(inp, lam, xp, Bp, dtb, use_lam, use_prev)
    t = to_device(inp)
    run = lambda: gpu_trap(t, lam, xp, Bp, dtb, use_lam, use_prev)
    y, hT = with_plan(chunks, run) if chunks else run()
    assert_y(y, yr, bf16=True)
    assert_state(hT, hr, "hT")


def test_trap_lambda_one_matches_the_euler_scan():
    """lam = 1 everywhere is jscan_prefill's recurrence."""
    print_case("trap lam=1 vs prefill")
    inp, lam, xp, Bp, _ = problem(1, 500, 128, seed=42, io=synth.IO_BF16)
    t = to_device(inp)
    ones = np.full_like(lam, synth.to_bf16_bits(np.ones(1))[0])
    y1, h1 = gpu_trap(t, ones, xp, Bp, None)
    y0, h0 = js.prefill(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"])
    torch.cuda.synchronize()
    yr, hr = oracle.prefill(*(oracle_inputs(inp)[k] for k in ("x", "delta", "A", "B", "C", "D", "z", "h0")))
    assert_y(y1, yr, bf16=True)
    assert_state(h1, hr, "hT")
    assert_y(y0, yr, bf16=True)


def test_trap_chained_calls_and_decode():
    """A sequence as two prefill calls (the second given the first's state and
    its last x and B row) and then decode steps, against one oracle call."""
    print_case("trap chained prefill + decode")
    L0, L1, T, d = 300, 200, 6, 136
    inp, lam, xp, Bp, dtb = problem(1, L0 + L1 + T, d, seed=43, io=synth.IO_BF16, softplus=True)
    yr, hr = oracle_trap(inp, lam, xp, Bp, dtb)
    t = to_device(inp)
    tl = dev_io(lam)
    sl = lambda v, a, b: v[:, a:b].contiguous()
    kw = dict(dt_bias=dev_f32(dtb), softplus=True)
    y_a, h_a = js.prefill_trap(sl(t["x"], 0, L0), sl(t["delta"], 0, L0), t["A"], sl(t["B"], 0, L0),
                               sl(t["C"], 0, L0), t["D"], sl(t["z"], 0, L0), t["h0"], lam=sl(tl, 0, L0),
                               x_prev=dev_io(xp), B_prev=dev_io(Bp), **kw)
    e = L0 + L1
    y_b, state = js.prefill_trap(sl(t["x"], L0, e), sl(t["delta"], L0, e), t["A"], sl(t["B"], L0, e),
                                 sl(t["C"], L0, e), t["D"], sl(t["z"], L0, e), h_a, lam=sl(tl, L0, e),
                                 x_prev=t["x"][:, L0 - 1].contiguous(), B_prev=t["B"][:, L0 - 1].contiguous(),
                                 **kw)
    ys = []
    for k in range(e, e + T):
        ys.append(js.step_batch_trap(state, t["x"][:, k].contiguous(), t["delta"][:, k].contiguous(), t["A"],
                                     t["B"][:, k].contiguous(), t["C"][:, k].contiguous(), t["D"],
                                     t["z"][:, k].contiguous(), lam=tl[:, k].contiguous(),
                                     x_prev=t["x"][:, k - 1].contiguous(), B_prev=t["B"][:, k - 1].contiguous(),
                                     **kw))
    torch.cuda.synchronize()
    assert_y(y_a, yr[:, :L0], bf16=True, what="first call")
    assert_y(y_b, yr[:, L0:e], bf16=True, what="second call")
    assert_y(torch.stack(ys, 1), yr[:, e:], bf16=True, what="decode")
    assert_state(state, hr, "state after decode")


@pytest.mark.parametrize("given", ["none", "lam", "x_prev", "B_prev", "prev"])
def test_trap_step_optional_inputs(given):
    """Trapezoidal decode steps with the optional inputs given or left out
    (lam: 1/2, x_prev and B_prev: zero), each step against the oracle's
    one-token prefill from the same state.  Three steps of 7 sequences, with
    softplus and dt_bias."""
    print_case(f"trap decode given {given}")
    n_seq, T, d = 7, 3, 136
    inp, lam, xp, Bp, dtb = problem(n_seq, T, d, seed=45, io=synth.IO_BF16, softplus=True)
    use_lam = given == "lam"
    use_x = given in ("x_prev", "prev")
    use_B = given in ("B_prev", "prev")
    o = oracle_inputs(inp)
    state = dev_f32(inp["h0"])
    st64 = inp["h0"].astype(np.float64)
    t = to_device(inp)
    tl = dev_io(lam)
    for k in range(T):
        _, dt, _ = oracle.prologue(o["x"][:, k:k + 1], o["delta"][:, k:k + 1], dt_bias=dtb, softplus=True)
        yr, st64, _, _ = oracle.prefill_trap(o["x"][:, k:k + 1], dt, o["A"], o["B"][:, k:k + 1], o["C"][:, k:k + 1],
                                             o["D"], o["z"][:, k:k + 1], st64,
                                             lam=synth.widen(lam[:, k:k + 1]) if use_lam else None,
                                             x_prev=synth.widen(xp) if use_x else None,
                                             B_prev=synth.widen(Bp) if use_B else None)
        y = js.step_batch_trap(state, t["x"][:, k].contiguous(), t["delta"][:, k].contiguous(), t["A"],
                               t["B"][:, k].contiguous(), t["C"][:, k].contiguous(), t["D"],
                               t["z"][:, k].contiguous(), lam=tl[:, k].contiguous() if use_lam else None,
                               x_prev=dev_io(xp) if use_x else None, B_prev=dev_io(Bp) if use_B else None,
                               dt_bias=dev_f32(dtb), softplus=True)
        torch.cuda.synchronize()
        assert_y(y, yr[:, 0], bf16=True, what=f"y step {k}")
        assert_state(state, st64, f"state step {k}")


@pytest.mark.parametrize("n_seq,d", [(1, 1), (7, 1), (300, 3), (2, 65)])
def test_trap_step_edge_sizes(n_seq, d):
    """Trapezoidal decode steps at degenerate sizes (one channel, one sequence,
    part-filled waves), every optional input given; each step against the
    oracle's one-token prefill from the same state."""
    print_case(f"trap decode edge n_seq={n_seq} d={d}")
    inp, lam, xp, Bp, dtb = problem(n_seq, 2, d, seed=46, io=synth.IO_BF16, softplus=True)
    o = oracle_inputs(inp)
    state = dev_f32(inp["h0"])
    st64 = inp["h0"].astype(np.float64)
    t = to_device(inp)
    tl = dev_io(lam)
    for k in range(2):
        _, dt, _ = oracle.prologue(o["x"][:, k:k + 1], o["delta"][:, k:k + 1], dt_bias=dtb, softplus=True)
        yr, st64, _, _ = oracle.prefill_trap(o["x"][:, k:k + 1], dt, o["A"], o["B"][:, k:k + 1], o["C"][:, k:k + 1],
                                             o["D"], o["z"][:, k:k + 1], st64, lam=synth.widen(lam[:, k:k + 1]),
                                             x_prev=synth.widen(xp), B_prev=synth.widen(Bp))
        # fresh copies: a one-channel slice is contiguous but not 16-byte aligned
        tok = lambda v: v[:, k].clone()
        y = js.step_batch_trap(state, tok(t["x"]), tok(t["delta"]), t["A"], tok(t["B"]), tok(t["C"]), t["D"],
                               tok(t["z"]), lam=tok(tl), x_prev=dev_io(xp), B_prev=dev_io(Bp), dt_bias=dev_f32(dtb),
                               softplus=True)
        torch.cuda.synchronize()
        assert_y(y, yr[:, 0], bf16=True, what=f"y step {k}")
        assert_state(state, st64, f"state step {k}")


def test_trap_step_full_size():
    """The trapezoidal decode step at the decode workload's size, 256
    sequences x 8192 channels, lam and the previous token given: three
    chained steps (each step's previous token is the one before it), every
    output and the state against the oracle's one-token prefill."""
    n_seq, T, d = 256, 3, 8192
    print_case(f"trap decode {n_seq} x {d}")
    inp, lam, xp, Bp, dtb = problem(n_seq, T, d, seed=47, io=synth.IO_BF16, softplus=True)
    o = oracle_inputs(inp)
    state = dev_f32(inp["h0"])
    st64 = inp["h0"].astype(np.float64)
    t = to_device(inp)
    tl = dev_io(lam)
    tok = lambda v, k: v[:, k].clone()
    for k in range(T):
        x_prev = synth.widen(xp) if k == 0 else o["x"][:, k - 1]
        B_prev = synth.widen(Bp) if k == 0 else o["B"][:, k - 1]
        _, dt, _ = oracle.prologue(o["x"][:, k:k + 1], o["delta"][:, k:k + 1], dt_bias=dtb, softplus=True)
        yr, st64, _, _ = oracle.prefill_trap(o["x"][:, k:k + 1], dt, o["A"], o["B"][:, k:k + 1], o["C"][:, k:k + 1],
                                             o["D"], o["z"][:, k:k + 1], st64, lam=synth.widen(lam[:, k:k + 1]),
                                             x_prev=x_prev, B_prev=B_prev)
        gx_prev = dev_io(xp) if k == 0 else tok(t["x"], k - 1)
        gB_prev = dev_io(Bp) if k == 0 else tok(t["B"], k - 1)
        y = js.step_batch_trap(state, tok(t["x"], k), tok(t["delta"], k), t["A"], tok(t["B"], k), tok(t["C"], k),
                               t["D"], tok(t["z"], k), lam=tok(tl, k), x_prev=gx_prev, B_prev=gB_prev,
                               dt_bias=dev_f32(dtb), softplus=True)
        torch.cuda.synchronize()
        assert_y(y, yr[:, 0], bf16=True, what=f"y step {k}")
        assert_state(state, st64, f"state step {k}")


def test_trap_64k_sampled():
    """The 64K-token prefill (batch 1, d_inner 8192, bf16) with lam and the
    token before the first, automatic plan; 24 sampled channels over all tokens."""
    L, d = 65536, 8192
    print_case(f"trap 64K sampled L={L}")
    inp = synth.prefill_inputs(1, L, d, seed=44, io=synth.IO_BF16, h0=True)
    lam, xp, Bp = synth.trap_inputs(1, L, d, seed=44)
    y, hT = gpu_trap(to_device(inp), lam, xp, Bp, None)
    assert torch.isfinite(y.float()).all() and torch.isfinite(hT).all()
    rng = np.random.default_rng(44)
    ch = np.unique(np.concatenate([[0, 63, 64, 4095, 4096, 8191], rng.choice(d, 18, replace=False)]))
    sub = synth.channel_slice(inp, ch)
    yr, hr, _, _ = oracle.prefill_trap(sub["x"], sub["delta"], sub["A"], sub["B"], sub["C"], sub["D"], sub["z"],
                                       sub["h0"], lam=synth.widen(lam[:, :, ch]), x_prev=synth.widen(xp[:, ch]),
                                       B_prev=synth.widen(Bp))
    assert_y(y[:, :, ch], yr, bf16=True)
    assert_state(hT[:, ch], hr, "hT")


def _random_cases(n, seed):
    rng = np.random.default_rng(seed)
    return [dict(batch=int(rng.integers(1, 4)), L=int(rng.integers(1, 1200)),
                 d=int(rng.choice([1, 8, 64, 65, 136, 200])), lam=bool(rng.random() < 0.7),
                 prev=bool(rng.random() < 0.6), softplus=bool(rng.random() < 0.5),
                 io=synth.IO_BF16 if rng.random() < 0.7 else synth.IO_F32,
                 chunks=int(rng.choice([0, 1, 2, 5, 9])), seed=4000 + i) for i in range(n)]


@pytest.mark.parametrize("case", _random_cases(20, 2027),
                         ids=lambda c: "b{batch}L{L}d{d}lam{lam:d}prev{prev:d}sp{softplus:d}io{io}c{chunks}".format(**c))
def test_trap_random(case):
    """Seeded random sizes, lam and the token before the first given or not,
    softplus or not, I/O dtype and chunk count (0: automatic plan); y and hT
    against the oracle."""
    c = case
    print_case(f"trap random {c}")
    inp, lam, xp, Bp, dtb = problem(c["batch"], c["L"], c["d"], seed=c["seed"], io=c["io"], softplus=c["softplus"])
    yr, hr = oracle_trap(inp, lam, xp, Bp, dtb, c["lam"], c["prev"])
    run = lambda: gpu_trap(to_device(inp), lam, xp, Bp, dtb, c["lam"], c["prev"])
    y, hT = with_plan(c["chunks"], run) if c["chunks"] else run()
    assert_y(y, yr, bf16=c["io"] == synth.IO_BF16)
    assert_state(hT, hr, "hT")
