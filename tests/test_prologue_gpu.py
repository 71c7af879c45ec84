"""GPU parity of the fused input prologue (causal depthwise conv + SiLU on x,
softplus(delta + dt_bias)) against the fp64 oracle: ``oracle.prologue``
followed by ``oracle.prefill`` / ``oracle.step``.

Inputs are seeded synthetic data from ``synth`` (token tensors of the scan's
recipe, prologue parameters from ``synth.prologue_params``, raw time steps
from ``synth.raw_time_steps``).  The conv history the library writes back is
a copy of raw x values, so it is compared bit for bit.
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


def problem(batch, L, d_inner, width, seed, io, h0=True, raw_dt=True):
    inp = synth.prefill_inputs(batch, L, d_inner, seed=seed, io=io, h0=h0)
    if raw_dt:
        inp["delta"] = synth.raw_time_steps(batch, L, d_inner, seed=seed, io=io)
    pro = synth.prologue_params(d_inner, max(width, 1), seed=seed, batch=batch)
    return inp, pro


def oracle_fused(inp, pro, width, softplus, conv_state=True, use_h0=True):
    """Reference: prologue, then the scan, all in fp64."""
    o = oracle_inputs(inp)
    w = pro["conv_weight"] if width > 0 else None
    xc, dt, st = oracle.prologue(o["x"], o["delta"], w, pro["conv_bias"] if width > 0 else None,
                                 pro["conv_state"] if (width > 0 and conv_state) else None,
                                 pro["dt_bias"] if softplus else None, softplus)
    y, hT = oracle.prefill(xc, dt, o["A"], o["B"], o["C"], o["D"], o["z"], o["h0"] if use_h0 else None)
    return y, hT, st


def gpu_fused(t, pro, width, softplus, conv_state=True, use_h0=True, in_place=False, **kw):
    """Runs prefill_fused; returns (y, hT, conv_state_out)."""
    batch, L, d_inner = t["x"].shape
    cw = dev_f32(pro["conv_weight"]) if width > 0 else None
    cb = dev_f32(pro["conv_bias"]) if width > 0 else None
    cs_in = dev_f32(pro["conv_state"]) if (width > 0 and conv_state) else None
    if width > 0:
        cs_out = cs_in if (in_place and cs_in is not None) else torch.full(
            (batch, width - 1, d_inner), float("nan"), device="cuda")
    else:
        cs_out = None
    y, hT = js.prefill_fused(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                             t["h0"] if use_h0 else None, conv_weight=cw, conv_bias=cb, conv_state_in=cs_in,
                             conv_state_out=cs_out, dt_bias=dev_f32(pro["dt_bias"]) if softplus else None,
                             softplus=softplus, **kw)
    torch.cuda.synchronize()
    return y, hT, cs_out


def with_plan(K, chunks, fn):
    try:
        js.set_plan_override(K, chunks)
        return fn()
    finally:
        js.set_plan_override(0, 0)


# ------------------------------------------------------------ small, every output
@pytest.mark.parametrize("width", [4, 3, 2, 1])
@pytest.mark.parametrize("softplus", [True, False])
@pytest.mark.parametrize("chunks", [1, 5])
def test_prefill_fused_ragged_bf16(width, softplus, chunks):
    """Two sequences, L 777 (partial last token block), d_inner 200 (partial
    channel group), h0 and a conv history given; single-pass and chunked plans."""
    print_case(f"fused ragged bf16 width={width} softplus={softplus} chunks={chunks}")
    # without softplus the time steps must already be positive: the scan's own recipe
    inp, pro = problem(2, 777, 200, width, seed=11, io=synth.IO_BF16, raw_dt=softplus)
    t = to_device(inp)
    yr, hr, sr = oracle_fused(inp, pro, width, softplus)
    y, hT, so = with_plan(1, chunks, lambda: gpu_fused(t, pro, width, softplus))
    assert_y(y, yr, bf16=True)
    assert_state(hT, hr, "hT")
    assert np.array_equal(host64(so), sr), "conv_state_out"


@pytest.mark.parametrize("chunks", [1, 3])
def test_prefill_fused_f32_no_history(chunks):
    """fp32 I/O, no conv history (zeros) and no h0."""
    print_case(f"fused f32 no history chunks={chunks}")
    inp, pro = problem(1, 333, 64, 4, seed=12, io=synth.IO_F32, h0=False)
    t = to_device(inp)
    yr, hr, sr = oracle_fused(inp, pro, 4, True, conv_state=False, use_h0=False)
    y, hT, so = with_plan(1, chunks, lambda: gpu_fused(t, pro, 4, True, conv_state=False, use_h0=False))
    assert_y(y, yr, bf16=False)
    assert_state(hT, hr, "hT")
    assert np.array_equal(host64(so), sr)


@pytest.mark.parametrize("chunks", [1, 4])
def test_prefill_fused_in_place_conv_state(chunks):
    """conv_state_out is the conv_state_in buffer (the usual carry)."""
    print_case(f"fused in-place conv state chunks={chunks}")
    inp, pro = problem(2, 400, 128, 4, seed=13, io=synth.IO_BF16)
    t = to_device(inp)
    yr, hr, sr = oracle_fused(inp, pro, 4, True)
    y, hT, so = with_plan(1, chunks, lambda: gpu_fused(t, pro, 4, True, in_place=True))
    assert_y(y, yr, bf16=True)
    assert_state(hT, hr, "hT")
    assert np.array_equal(host64(so), sr)


def test_prefill_fused_many_short_chunks():
    """Chunks of 8 tokens (every chunk but the first rescanned from its true
    start by pass 2, the conv history of each chunk read from x)."""
    print_case("fused with 38 chunks of 8 tokens")
    inp, pro = problem(1, 300, 96, 4, seed=14, io=synth.IO_BF16)
    t = to_device(inp)
    yr, hr, sr = oracle_fused(inp, pro, 4, True)
    y, hT, so = with_plan(1, 38, lambda: gpu_fused(t, pro, 4, True))
    assert_y(y, yr, bf16=True)
    assert_state(hT, hr, "hT")
    assert np.array_equal(host64(so), sr)


@pytest.mark.parametrize("L", [1, 2, 3, 9])
def test_prefill_fused_short_sequences(L):
    """Sequences shorter than the conv window: the history written back mixes
    the given history and the new tokens."""
    print_case(f"fused short L={L}")
    inp, pro = problem(2, L, 80, 4, seed=15, io=synth.IO_BF16)
    t = to_device(inp)
    yr, hr, sr = oracle_fused(inp, pro, 4, True)
    y, hT, so = gpu_fused(t, pro, 4, True)
    assert_y(y, yr, bf16=True)
    assert_state(hT, hr, "hT")
    assert np.array_equal(host64(so), sr)
    # in place as well
    y2, hT2, so2 = gpu_fused(t, pro, 4, True, in_place=True)
    assert torch.equal(y2, y) and torch.equal(hT2, hT) and torch.equal(so2, so)


def test_prefill_fused_empty_sequence_copies_history():
    """L = 0: hT = h0 and the conv history passes through unchanged."""
    print_case("fused L=0")
    inp, pro = problem(2, 0, 64, 4, seed=16, io=synth.IO_BF16)
    t = to_device(inp)
    y, hT, so = gpu_fused(t, pro, 4, True)
    assert y.numel() == 0
    assert np.array_equal(host64(hT), inp["h0"].astype(np.float64))
    assert np.array_equal(host64(so), pro["conv_state"].astype(np.float64))


def test_prefill_fused_without_prologue_is_plain_prefill():
    """An empty prologue (no conv, no softplus) is the plain scan, bit for bit."""
    print_case("fused with empty prologue")
    inp = synth.prefill_inputs(1, 500, 128, seed=17, io=synth.IO_BF16, h0=True)
    t = to_device(inp)
    y0, h0 = js.prefill(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"])
    y1, h1 = js.prefill_fused(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"])
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(h0, h1)


@pytest.mark.parametrize("split", [256, 501])
def test_prefill_fused_chained_calls_carry_both_states(split):
    """A sequence cut in two calls, each carrying hT and the conv history into
    the next, gives the single call's result."""
    print_case(f"fused chained split={split}")
    L = 777
    inp, pro = problem(1, L, 136, 4, seed=18, io=synth.IO_BF16)
    yr, hr, sr = oracle_fused(inp, pro, 4, True)
    t = to_device(inp)
    parts = []
    h = t["h0"].clone()
    cs = dev_f32(pro["conv_state"])
    for lo, hi in ((0, split), (split, L)):
        sub = {k: (v[:, lo:hi].contiguous() if k in ("x", "delta", "z", "B", "C") else v) for k, v in t.items()}
        y, _ = js.prefill_fused(sub["x"], sub["delta"], sub["A"], sub["B"], sub["C"], sub["D"], sub["z"], h,
                                hT=h, conv_weight=dev_f32(pro["conv_weight"]), conv_bias=dev_f32(pro["conv_bias"]),
                                conv_state_in=cs, conv_state_out=cs, dt_bias=dev_f32(pro["dt_bias"]),
                                softplus=True)
        parts.append(y)
    torch.cuda.synchronize()
    assert_y(torch.cat(parts, dim=1), yr, bf16=True)
    assert_state(h, hr, "hT")
    assert np.array_equal(host64(cs), sr)


# ------------------------------------------------------------------ decode step
def test_step_fused_matches_oracle_steps():
    """Eight chained fused decode steps for three sequences against the oracle's
    prologue + step, conv history and state carried in place."""
    print_case("fused decode steps")
    n_seq, d, width = 3, 200, 4
    pro = synth.prologue_params(d, width, seed=19, batch=n_seq)
    A, D, _ = synth.params(d, seed=19)
    st64 = synth.decode_state(n_seq, d, seed=19).astype(np.float64)
    cs64 = pro["conv_state"].astype(np.float64)
    state = dev_f32(synth.decode_state(n_seq, d, seed=19))
    cs = dev_f32(pro["conv_state"])
    tA, tD = dev_f32(A), dev_f32(D)
    for k in range(8):
        s = synth.decode_inputs(n_seq, d, seed=19, step=k)
        s["delta"] = synth.raw_time_steps(n_seq, 1, d, seed=100 + k)[:, 0, :]
        xc, dt, cs64 = oracle.prologue(synth.widen(s["x"])[:, None, :], synth.widen(s["delta"])[:, None, :],
                                       pro["conv_weight"], pro["conv_bias"], cs64, pro["dt_bias"], True)
        yr, st64 = oracle.step(st64, xc[:, 0, :], dt[:, 0, :], A.astype(np.float64), synth.widen(s["B"]),
                               synth.widen(s["C"]), D.astype(np.float64), synth.widen(s["z"]))
        y = js.step_batch_fused(state, dev_io(s["x"]), dev_io(s["delta"]), tA, dev_io(s["B"]), dev_io(s["C"]), tD,
                                dev_io(s["z"]), conv_weight=dev_f32(pro["conv_weight"]),
                                conv_bias=dev_f32(pro["conv_bias"]), conv_state=cs,
                                dt_bias=dev_f32(pro["dt_bias"]), softplus=True)
        torch.cuda.synchronize()
        assert_y(y, yr, bf16=True, what=f"y step {k}")
        assert_state(state, st64, f"state step {k}")
        assert np.array_equal(host64(cs), cs64), f"conv state step {k}"


def test_step_fused_full_size():
    """The fused decode step at the decode workload's size, 256 sequences x
    8192 channels (conv(4) + SiLU with its history in place, softplus with
    dt_bias): three chained steps, every output, the state and the history
    against the oracle."""
    print_case("fused decode 256 x 8192")
    n_seq, d = 256, 8192
    pro = synth.prologue_params(d, 4, seed=33, batch=n_seq)
    A, D, _ = synth.params(d, seed=33)
    st64 = synth.decode_state(n_seq, d, seed=33).astype(np.float64)
    cs64 = pro["conv_state"].astype(np.float64)
    state = dev_f32(synth.decode_state(n_seq, d, seed=33))
    cs = dev_f32(pro["conv_state"])
    tA, tD = dev_f32(A), dev_f32(D)
    kw = dict(conv_weight=dev_f32(pro["conv_weight"]), conv_bias=dev_f32(pro["conv_bias"]),
              dt_bias=dev_f32(pro["dt_bias"]), softplus=True)
    for k in range(3):
        s = synth.decode_inputs(n_seq, d, seed=33, step=k)
        s["delta"] = synth.raw_time_steps(n_seq, 1, d, seed=600 + k)[:, 0, :]
        xc, dt, cs64 = oracle.prologue(synth.widen(s["x"])[:, None, :], synth.widen(s["delta"])[:, None, :],
                                       pro["conv_weight"], pro["conv_bias"], cs64, pro["dt_bias"], True)
        yr, st64 = oracle.step(st64, xc[:, 0, :], dt[:, 0, :], A.astype(np.float64), synth.widen(s["B"]),
                               synth.widen(s["C"]), D.astype(np.float64), synth.widen(s["z"]))
        t = {key: dev_io(s[key]) for key in ("x", "delta", "z", "B", "C")}
        y = js.step_batch_fused(state, t["x"], t["delta"], tA, t["B"], t["C"], tD, t["z"], conv_state=cs, **kw)
        torch.cuda.synchronize()
        assert_y(y, yr, bf16=True, what=f"y step {k}")
        assert_state(state, st64, f"state step {k}")
        assert np.array_equal(host64(cs), cs64), f"conv state step {k}"


@pytest.mark.parametrize("n_seq,d", [(1, 1), (1, 8), (7, 1), (300, 3), (2, 65)])
@pytest.mark.parametrize("fused", [False, True])
def test_step_edge_sizes(n_seq, d, fused):
    """Decode steps at degenerate sizes: one channel (each quad of a wave is
    another sequence), one sequence, and channel counts that leave a wave
    part-filled; plain or with the conv(4) + softplus prologue.  Two chained
    steps against the oracle."""
    print_case(f"decode edge n_seq={n_seq} d={d} fused={fused}")
    pro = synth.prologue_params(d, 4, seed=31, batch=n_seq)
    A, D, _ = synth.params(d, seed=31)
    st64 = synth.decode_state(n_seq, d, seed=31).astype(np.float64)
    cs64 = pro["conv_state"].astype(np.float64)
    state = dev_f32(synth.decode_state(n_seq, d, seed=31))
    cs = dev_f32(pro["conv_state"])
    tA, tD = dev_f32(A), dev_f32(D)
    for k in range(2):
        s = synth.decode_inputs(n_seq, d, seed=31, step=k)
        if fused:
            s["delta"] = synth.raw_time_steps(n_seq, 1, d, seed=500 + k)[:, 0, :]
            xc, dt, cs64 = oracle.prologue(synth.widen(s["x"])[:, None, :], synth.widen(s["delta"])[:, None, :],
                                           pro["conv_weight"], pro["conv_bias"], cs64, pro["dt_bias"], True)
            xo, do = xc[:, 0, :], dt[:, 0, :]
        else:
            xo, do = synth.widen(s["x"]), synth.widen(s["delta"])
        yr, st64 = oracle.step(st64, xo, do, A.astype(np.float64), synth.widen(s["B"]), synth.widen(s["C"]),
                               D.astype(np.float64), synth.widen(s["z"]))
        t = {key: dev_io(s[key]) for key in ("x", "delta", "z", "B", "C")}
        if fused:
            y = js.step_batch_fused(state, t["x"], t["delta"], tA, t["B"], t["C"], tD, t["z"],
                                    conv_weight=dev_f32(pro["conv_weight"]), conv_bias=dev_f32(pro["conv_bias"]),
                                    conv_state=cs, dt_bias=dev_f32(pro["dt_bias"]), softplus=True)
        else:
            y = js.step_batch(state, t["x"], t["delta"], tA, t["B"], t["C"], tD, t["z"])
        torch.cuda.synchronize()
        assert_y(y, yr, bf16=True, what=f"y step {k}")
        assert_state(state, st64, f"state step {k}")
        if fused:
            assert np.array_equal(host64(cs), cs64), f"conv state step {k}"


@pytest.mark.parametrize("absent", ["conv_bias", "history", "dt_bias", "all"])
def test_step_fused_optional_inputs_absent(absent):
    """Fused decode steps (width 4, softplus) with optional inputs left out:
    no conv bias (0), no conv history (zeros, nothing written back), no
    dt_bias (0).  Three chained steps of 5 sequences against the oracle."""
    print_case(f"fused decode without {absent}")
    n_seq, d, width = 5, 200, 4
    no = lambda k: absent in (k, "all")
    pro = synth.prologue_params(d, width, seed=23, batch=n_seq)
    A, D, _ = synth.params(d, seed=23)
    st64 = synth.decode_state(n_seq, d, seed=23).astype(np.float64)
    cs64 = None if no("history") else pro["conv_state"].astype(np.float64)
    state = dev_f32(synth.decode_state(n_seq, d, seed=23))
    cs = None if no("history") else dev_f32(pro["conv_state"])
    cb = None if no("conv_bias") else pro["conv_bias"]
    dtb = None if no("dt_bias") else pro["dt_bias"]
    for k in range(3):
        s = synth.decode_inputs(n_seq, d, seed=23, step=k)
        s["delta"] = synth.raw_time_steps(n_seq, 1, d, seed=300 + k)[:, 0, :]
        xc, dt, cs_next = oracle.prologue(synth.widen(s["x"])[:, None, :], synth.widen(s["delta"])[:, None, :],
                                          pro["conv_weight"], cb, cs64, dtb, True)
        if cs64 is not None:
            cs64 = cs_next
        yr, st64 = oracle.step(st64, xc[:, 0, :], dt[:, 0, :], A.astype(np.float64), synth.widen(s["B"]),
                               synth.widen(s["C"]), D.astype(np.float64), synth.widen(s["z"]))
        y = js.step_batch_fused(state, dev_io(s["x"]), dev_io(s["delta"]), dev_f32(A), dev_io(s["B"]),
                                dev_io(s["C"]), dev_f32(D), dev_io(s["z"]), conv_weight=dev_f32(pro["conv_weight"]),
                                conv_bias=dev_f32(cb), conv_state=cs, dt_bias=dev_f32(dtb), softplus=True)
        torch.cuda.synchronize()
        assert_y(y, yr, bf16=True, what=f"y step {k}")
        assert_state(state, st64, f"state step {k}")
        if cs is not None:
            assert np.array_equal(host64(cs), cs64), f"conv state step {k}"


@pytest.mark.parametrize("width", [4, 2, 1])
def test_fused_steps_continue_a_fused_prefill(width):
    """Prefill of 300 tokens then 5 fused steps equals one fused prefill of 305
    tokens (decode continues where the prompt's two states left off)."""
    print_case(f"fused prefill + steps width={width}")
    L0, T, d = 300, 5, 128
    inp, pro = problem(1, L0 + T, d, width, seed=20, io=synth.IO_BF16)
    t = to_device(inp)
    y_all, h_all, cs_all = gpu_fused(t, pro, width, True)
    head = {k: (v[:, :L0].contiguous() if k in ("x", "delta", "z", "B", "C") else v) for k, v in t.items()}
    y_head, state, cs = gpu_fused(head, pro, width, True)
    cw, cb, dtb = dev_f32(pro["conv_weight"]), dev_f32(pro["conv_bias"]), dev_f32(pro["dt_bias"])
    ys = []
    for k in range(L0, L0 + T):
        ys.append(js.step_batch_fused(state, t["x"][:, k].contiguous(), t["delta"][:, k].contiguous(), t["A"],
                                      t["B"][:, k].contiguous(), t["C"][:, k].contiguous(), t["D"],
                                      t["z"][:, k].contiguous(), conv_weight=cw, conv_bias=cb,
                                      conv_state=cs, dt_bias=dtb, softplus=True))
    torch.cuda.synchronize()
    y_steps = torch.stack(ys, dim=1)
    yr, hr, sr = oracle_fused(inp, pro, width, True)
    assert_y(y_steps, yr[:, L0:], bf16=True, what="decoded y")
    assert_y(y_head, yr[:, :L0], bf16=True, what="prompt y")
    assert_state(state, hr, "state after decode")
    assert_state(h_all, hr, "hT of the full prefill")
    if width > 1:
        assert torch.equal(cs, cs_all)
        assert np.array_equal(host64(cs), sr)


# ------------------------------------------------------------ full size, sampled
def test_fused_prefill_64k_sampled():
    """The 64K-token prefill (batch 1, d_inner 8192, bf16) with the full
    prologue, in the automatic plan; 24 channels (three whole channel groups'
    edges and a random spread) compared against the oracle over all 65536
    tokens; every output finite."""
    L, d, width = 65536, 8192, 4
    print_case(f"fused 64K sampled L={L} d={d}")
    inp = synth.prefill_inputs(1, L, d, seed=21, io=synth.IO_BF16, h0=True)
    pro = synth.prologue_params(d, width, seed=21)
    t = to_device(inp)
    y, hT, so = gpu_fused(t, pro, width, True)
    assert torch.isfinite(y.float()).all() and torch.isfinite(hT).all()
    rng = np.random.default_rng(21)
    ch = np.unique(np.concatenate([[0, 63, 64, 4095, 4096, 8191], rng.choice(d, 18, replace=False)]))
    sub = synth.channel_slice(inp, ch)
    xc, dt, st = oracle.prologue(sub["x"], sub["delta"], pro["conv_weight"][ch], pro["conv_bias"][ch],
                                 pro["conv_state"][:, :, ch], pro["dt_bias"][ch], True)
    yr, hr = oracle.prefill(xc, dt, sub["A"], sub["B"], sub["C"], sub["D"], sub["z"], sub["h0"])
    assert_y(y[:, :, ch], yr, bf16=True)
    assert_state(hT[:, ch], hr, "hT")
    assert np.array_equal(host64(so)[:, :, ch], st)


# ------------------------------------------------------------ input RMSNorm
EPS = 1e-5


def rms_case(inp, pro, seed, which=(True, True, True), width=4, softplus=True):
    """Oracle: RMSNorm of delta, B, C, then the prologue, then the scan."""
    w_dt, w_B, w_C = synth.rms_weights(inp["x"].shape[2], seed=seed)
    ws = tuple(w if k else None for w, k in zip((w_dt, w_B, w_C), which))
    o = oracle_inputs(inp)
    # the plain definition in fp64: nothing is rounded between the normalisation and the scan
    dn, Bn, Cn = oracle.rmsnorm_inputs(o["delta"], o["B"], o["C"], *ws, eps=EPS)
    xc, dt, st = oracle.prologue(o["x"], dn, pro["conv_weight"] if width else None,
                                 pro["conv_bias"] if width else None, pro["conv_state"] if width else None,
                                 pro["dt_bias"] if softplus else None, softplus)
    y, hT = oracle.prefill(xc, dt, o["A"], Bn, Cn, o["D"], o["z"], o["h0"])
    return ws, y, hT, st


def gpu_rms(t, pro, ws, width=4, softplus=True):
    batch, L, d = t["x"].shape
    rms = tuple(dev_f32(w) for w in ws) + (EPS,)
    cs_out = torch.empty((batch, width - 1, d), device="cuda") if width else None
    y, hT = js.prefill_fused(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"],
                             conv_weight=dev_f32(pro["conv_weight"]) if width else None,
                             conv_bias=dev_f32(pro["conv_bias"]) if width else None,
                             conv_state_in=dev_f32(pro["conv_state"]) if width else None, conv_state_out=cs_out,
                             dt_bias=dev_f32(pro["dt_bias"]) if softplus else None, softplus=softplus, rms=rms)
    torch.cuda.synchronize()
    return y, hT, cs_out


@pytest.mark.parametrize("chunks", [1, 5])
@pytest.mark.parametrize("io", [synth.IO_BF16, synth.IO_F32])
def test_prefill_rmsnorm_conv_softplus(chunks, io):
    """RMSNorm of delta, B and C, then conv(4) + SiLU and softplus, ragged shape."""
    print_case(f"rmsnorm + conv + softplus chunks={chunks} io={io}")
    inp, pro = problem(2, 777, 200, 4, seed=60, io=io)
    ws, yr, hr, sr = rms_case(inp, pro, seed=60)
    y, hT, so = with_plan(1, chunks, lambda: gpu_rms(to_device(inp), pro, ws))
    assert_y(y, yr, bf16=io == synth.IO_BF16)
    assert_state(hT, hr, "hT")
    assert np.array_equal(host64(so), sr)


@pytest.mark.parametrize("d", [128, 100])
@pytest.mark.parametrize("which", [(False, True, False), (True, False, False), (False, False, True)])
def test_prefill_rmsnorm_one_tensor(which, d):
    """Only one of delta, B, C normalised; no conv, no softplus (delta from the
    scan's own positive recipe).  d_inner 100 is not a whole number of 16-byte
    vectors of bf16, so the time step's normalisation takes its scalar path."""
    print_case(f"rmsnorm {which} d={d}")
    inp, pro = problem(1, 300, d, 4, seed=61, io=synth.IO_BF16, raw_dt=False)
    ws, yr, hr, _ = rms_case(inp, pro, seed=61, which=which, width=0, softplus=False)
    y, hT, _ = gpu_rms(to_device(inp), pro, ws, width=0, softplus=False)
    assert_y(y, yr, bf16=True)
    assert_state(hT, hr, "hT")


@pytest.mark.parametrize("io,d", [(synth.IO_BF16, 2056), (synth.IO_BF16, 8200), (synth.IO_F32, 1028),
                                  (synth.IO_F32, 4100)])
def test_prefill_rmsnorm_row_lengths(io, d):
    """The time step's normalisation over rows that a workgroup holds in
    registers with a partial last group of vectors (2056 bf16, 1028 fp32) and
    over rows too long to hold, which it reads twice (8200 bf16, 4100 fp32)."""
    print_case(f"rmsnorm rows io={io} d={d}")
    inp, pro = problem(1, 40, d, 4, seed=64, io=io, raw_dt=False)
    ws, yr, hr, _ = rms_case(inp, pro, seed=64, which=(True, False, False), width=0, softplus=False)
    y, hT, _ = gpu_rms(to_device(inp), pro, ws, width=0, softplus=False)
    assert_y(y, yr, bf16=io == synth.IO_BF16)
    assert_state(hT, hr, "hT")


@pytest.mark.parametrize("which", [(True, True, True), (False, True, True), (True, False, False)],
                         ids=["dt_B_C", "B_C", "dt"])
def test_step_rmsnorm_matches_oracle(which):
    """Three fused decode steps with RMSNorm, conv history and softplus; the
    weights not in `which` are left out (that tensor is not normalised)."""
    print_case(f"rmsnorm decode {which}")
    n_seq, d, width = 3, 200, 4
    pro = synth.prologue_params(d, width, seed=62, batch=n_seq)
    w_dt, w_B, w_C = (w if k else None for w, k in zip(synth.rms_weights(d, seed=62), which))
    A, D, _ = synth.params(d, seed=62)
    st64 = synth.decode_state(n_seq, d, seed=62).astype(np.float64)
    cs64 = pro["conv_state"].astype(np.float64)
    state = dev_f32(synth.decode_state(n_seq, d, seed=62))
    cs = dev_f32(pro["conv_state"])
    rms = (dev_f32(w_dt), dev_f32(w_B), dev_f32(w_C), EPS)
    for k in range(3):
        s = synth.decode_inputs(n_seq, d, seed=62, step=k)
        s["delta"] = synth.raw_time_steps(n_seq, 1, d, seed=200 + k)[:, 0, :]
        dn, Bn, Cn = oracle.rmsnorm_inputs(synth.widen(s["delta"])[:, None, :], synth.widen(s["B"])[:, None, :],
                                           synth.widen(s["C"])[:, None, :], w_dt, w_B, w_C, eps=EPS)
        xc, dt, cs64 = oracle.prologue(synth.widen(s["x"])[:, None, :], dn, pro["conv_weight"], pro["conv_bias"],
                                       cs64, pro["dt_bias"], True)
        yr, st64 = oracle.step(st64, xc[:, 0], dt[:, 0], A.astype(np.float64), Bn[:, 0], Cn[:, 0],
                               D.astype(np.float64), synth.widen(s["z"]))
        y = js.step_batch_fused(state, dev_io(s["x"]), dev_io(s["delta"]), dev_f32(A), dev_io(s["B"]),
                                dev_io(s["C"]), dev_f32(D), dev_io(s["z"]), conv_weight=dev_f32(pro["conv_weight"]),
                                conv_bias=dev_f32(pro["conv_bias"]), conv_state=cs,
                                dt_bias=dev_f32(pro["dt_bias"]), softplus=True, rms=rms)
        torch.cuda.synchronize()
        assert_y(y, yr, bf16=True, what=f"y step {k}")
        assert_state(state, st64, f"state step {k}")
        assert np.array_equal(host64(cs), cs64)


def test_step_rmsnorm_workspace_equals_scratch():
    """The RMSNorm decode step given a workspace (jscan_step_batch_fused_ws)
    equals the step that allocates its scratch, bit for bit: two steps of 3
    sequences, then one of 2 in the same workspace."""
    print_case("rmsnorm decode workspace")
    d = 200
    A, D, _ = synth.params(d, seed=64)
    tA, tD = dev_f32(A), dev_f32(D)
    pro = synth.prologue_params(d, 4, seed=64, batch=3)
    rms = tuple(dev_f32(w) for w in synth.rms_weights(d, seed=64)) + (EPS,)
    ws = torch.empty(js.step_workspace_size(3, d, rms), dtype=torch.uint8, device="cuda")
    assert ws.numel() >= 3 * 132 and js.step_workspace_size(2, d, rms) <= ws.numel()
    st_a = dev_f32(synth.decode_state(3, d, seed=64))
    st_b = st_a.clone()
    cs_a = dev_f32(pro["conv_state"])
    cs_b = cs_a.clone()
    for k, n_seq in enumerate((3, 3, 2)):
        s = synth.decode_inputs(n_seq, d, seed=64, step=k)
        s["delta"] = synth.raw_time_steps(n_seq, 1, d, seed=400 + k)[:, 0, :]
        t = {key: dev_io(s[key]) for key in ("x", "delta", "z", "B", "C")}
        kw = dict(conv_weight=dev_f32(pro["conv_weight"]), conv_bias=dev_f32(pro["conv_bias"]),
                  dt_bias=dev_f32(pro["dt_bias"]), softplus=True, rms=rms)
        sa, ca, sb, cb = st_a[:n_seq], cs_a[:n_seq], st_b[:n_seq], cs_b[:n_seq]
        ya = js.step_batch_fused(sa, t["x"], t["delta"], tA, t["B"], t["C"], tD, t["z"], conv_state=ca, **kw)
        yb = js.step_batch_fused(sb, t["x"], t["delta"], tA, t["B"], t["C"], tD, t["z"], conv_state=cb,
                                 workspace=ws, **kw)
        torch.cuda.synchronize()
        assert torch.equal(ya, yb), k
        assert torch.equal(sa, sb), k
        assert torch.equal(ca, cb), k


def test_prefill_rmsnorm_jamba_shape():
    """Batch 2 x 4096 x 8192 bf16 with RMSNorm and softplus: every output."""
    print_case("rmsnorm 2x4096x8192")
    inp, pro = problem(2, 4096, 8192, 1, seed=63, io=synth.IO_BF16)
    ws, yr, hr, _ = rms_case(inp, pro, seed=63, width=0)
    y, hT, _ = gpu_rms(to_device(inp), pro, ws, width=0)
    assert_y(y, yr, bf16=True)
    assert_state(hT, hr, "hT")


def _random_cases(n, seed):
    rng = np.random.default_rng(seed)
    return [dict(batch=int(rng.integers(1, 4)), L=int(rng.integers(1, 1200)),
                 d=int(rng.choice([1, 8, 64, 65, 136, 200, 264])), width=int(rng.integers(0, 5)),
                 softplus=bool(rng.random() < 0.7), history=bool(rng.random() < 0.7), h0=bool(rng.random() < 0.6),
                 io=synth.IO_BF16 if rng.random() < 0.7 else synth.IO_F32,
                 chunks=int(rng.choice([0, 1, 2, 5, 9])), seed=3000 + i) for i in range(n)]


@pytest.mark.parametrize("case", _random_cases(24, 2026),
                         ids=lambda c: "b{batch}L{L}d{d}w{width}sp{softplus:d}io{io}c{chunks}".format(**c))
def test_prefill_fused_random(case):
    """Seeded random sizes, conv width 0-4 with or without history, softplus
    or not, h0 or not, I/O dtype and chunk count (0: automatic plan); y and hT
    against the oracle, the written conv history bit for bit."""
    c = case
    print_case(f"fused random {c}")
    inp, pro = problem(c["batch"], c["L"], c["d"], c["width"], seed=c["seed"], io=c["io"], h0=c["h0"],
                       raw_dt=c["softplus"])
    yr, hr, sr = oracle_fused(inp, pro, c["width"], c["softplus"], conv_state=c["history"], use_h0=c["h0"])
    run = lambda: gpu_fused(to_device(inp), pro, c["width"], c["softplus"], conv_state=c["history"], use_h0=c["h0"])
    y, hT, so = with_plan(1, c["chunks"], run) if c["chunks"] else run()
    assert_y(y, yr, bf16=c["io"] == synth.IO_BF16)
    assert_state(hT, hr, "hT")
    if c["width"] > 1:
        assert np.array_equal(host64(so), sr)


def _random_decode_cases(n, seed):
    rng = np.random.default_rng(seed)
    return [dict(n_seq=int(rng.integers(1, 300)), d=int(rng.choice([8, 64, 65, 136, 200, 1000])),
                 width=int(rng.integers(0, 5)), softplus=bool(rng.random() < 0.6),
                 io=synth.IO_BF16 if rng.random() < 0.7 else synth.IO_F32, seed=5000 + i) for i in range(n)]


@pytest.mark.parametrize("case", _random_decode_cases(12, 2028),
                         ids=lambda c: "n{n_seq}d{d}w{width}sp{softplus:d}io{io}".format(**c))
def test_step_random(case):
    """Seeded random sequence counts and widths, conv width 0-4, softplus or
    not, I/O dtype: three chained decode steps (state and conv history in
    place) against the oracle's prologue and step."""
    c = case
    print_case(f"decode random {c}")
    n_seq, d, width, sp, io = c["n_seq"], c["d"], c["width"], c["softplus"], c["io"]
    pro = synth.prologue_params(d, max(width, 1), seed=c["seed"], batch=n_seq)
    A, D, _ = synth.params(d, seed=c["seed"])
    st64 = synth.decode_state(n_seq, d, seed=c["seed"]).astype(np.float64)
    cs64 = pro["conv_state"].astype(np.float64) if width > 0 else None
    state = dev_f32(synth.decode_state(n_seq, d, seed=c["seed"]))
    cs = dev_f32(pro["conv_state"]) if width > 0 else None
    tA, tD = dev_f32(A), dev_f32(D)
    for k in range(3):
        s = synth.decode_inputs(n_seq, d, seed=c["seed"], step=k, io=io)
        if sp:
            s["delta"] = synth.raw_time_steps(n_seq, 1, d, seed=c["seed"] + 7 * k + 1, io=io)[:, 0, :]
        xc, dt, cs64 = oracle.prologue(synth.widen(s["x"])[:, None, :], synth.widen(s["delta"])[:, None, :],
                                       pro["conv_weight"] if width else None, pro["conv_bias"] if width else None,
                                       cs64, pro["dt_bias"] if sp else None, sp)
        yr, st64 = oracle.step(st64, xc[:, 0, :], dt[:, 0, :], A.astype(np.float64), synth.widen(s["B"]),
                               synth.widen(s["C"]), D.astype(np.float64), synth.widen(s["z"]))
        y = js.step_batch_fused(state, dev_io(s["x"]), dev_io(s["delta"]), tA, dev_io(s["B"]), dev_io(s["C"]), tD,
                                dev_io(s["z"]), conv_weight=dev_f32(pro["conv_weight"]) if width else None,
                                conv_bias=dev_f32(pro["conv_bias"]) if width else None, conv_state=cs,
                                dt_bias=dev_f32(pro["dt_bias"]) if sp else None, softplus=sp)
        torch.cuda.synchronize()
        assert_y(y, yr, bf16=io == synth.IO_BF16, what=f"y step {k}")
        assert_state(state, st64, f"state step {k}")
        if width > 1:
            assert np.array_equal(host64(cs), cs64), f"conv state step {k}"
