"""CPU-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call.

No test here launches work: every call below fails validation (or has no work
to do), which the library decides before touching the HIP runtime.
"""
import ctypes
import os
import re

import pytest

import selective_state_space_11_amd as js

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "jscan.h")

OK, NULL, SHAPE, UNSUP, ALIGN, ALIAS, WS, HIP = range(8)
BF16, F32 = js.IO_BF16, js.IO_F32

# Fake device addresses: validation only compares them, never dereferences.
BASE = 0x7F0000000000
MB = 1 << 20


def fake(i, extra=0):
    return ctypes.c_void_p(BASE + i * (1 << 36) + extra)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(js.LIB_PATH):
        from selective_state_space_11_amd import build
        build.build()
    return js.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(jscan_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = header_functions()
    for required in ("jscan_prefill", "jscan_step", "jscan_step_batch", "jscan_status_string"):
        assert required in names
    assert set(names) == set(js.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in js.STATUS_NAMES.items():
        assert lib.jscan_status_string(code).decode() == name
    assert lib.jscan_status_string(99).decode() == "JSCAN_UNKNOWN_STATUS"


def prefill_args(batch=1, L=64, d_inner=128, d_state=16, io=BF16, **over):
    es = 2 if io == BF16 else 4
    args = dict(batch=batch, L=L, d_inner=d_inner, d_state=d_state, io=io,
                x=fake(0), delta=fake(1), A=fake(2), B=fake(3), C=fake(4), D=fake(5), z=fake(6),
                h0=fake(7), y=fake(8), hT=fake(9), workspace=None, ws_bytes=0, stream=None)
    args.update(over)
    return args


def call_prefill(lib, a):
    return lib.jscan_prefill(a["batch"], a["L"], a["d_inner"], a["d_state"], a["io"], a["x"], a["delta"],
                             a["A"], a["B"], a["C"], a["D"], a["z"], a["h0"], a["y"], a["hT"],
                             a["workspace"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("name", ["x", "delta", "A", "B", "C", "D", "z", "y"])
def test_prefill_null_required_pointer(lib, name):
    assert call_prefill(lib, prefill_args(**{name: None})) == NULL
    assert "required" in lib.jscan_last_error().decode()


def test_prefill_shapes_and_support(lib):
    assert call_prefill(lib, prefill_args(batch=-1)) == SHAPE
    assert call_prefill(lib, prefill_args(L=-5)) == SHAPE
    assert call_prefill(lib, prefill_args(d_inner=-1)) == SHAPE
    assert call_prefill(lib, prefill_args(L=1 << 40)) == SHAPE
    assert call_prefill(lib, prefill_args(batch=70000)) == SHAPE
    assert call_prefill(lib, prefill_args(d_state=64)) == UNSUP
    assert call_prefill(lib, prefill_args(io=7)) == UNSUP


def test_prefill_empty_problem_is_a_no_op(lib):
    # batch 0: nothing to scan and no state to copy -> OK without any launch
    assert call_prefill(lib, prefill_args(batch=0)) == OK
    assert call_prefill(lib, prefill_args(d_inner=0)) == OK


@pytest.mark.parametrize("name", ["x", "delta", "A", "B", "C", "D", "z", "h0", "y", "hT"])
def test_prefill_alignment(lib, name):
    a = prefill_args()
    a[name] = ctypes.c_void_p(a[name].value + 2)
    assert call_prefill(lib, a) == ALIGN


def test_prefill_aliasing(lib):
    # y on top of x
    assert call_prefill(lib, prefill_args(y=fake(0))) == ALIAS
    # y inside delta's range: 1 x 64 x 128 bf16 = 16 KiB
    assert call_prefill(lib, prefill_args(y=fake(1, 4096))) == ALIAS
    # hT partially overlapping h0 (state is 1 x 128 x 16 fp32 = 8 KiB)
    assert call_prefill(lib, prefill_args(hT=fake(7, 4096))) == ALIAS
    # hT overlapping y
    assert call_prefill(lib, prefill_args(hT=fake(8, 16))) == ALIAS
    # workspace overlapping an input (a chunked plan, so the workspace is not empty)
    L, d = 65536, 8192
    ws = js.workspace_size(1, L, d)
    assert ws > 0
    assert call_prefill(lib, prefill_args(L=L, d_inner=d, workspace=fake(2), ws_bytes=ws)) == ALIAS
    assert "overlaps" in lib.jscan_last_error().decode()


def call_noalloc(lib, a):
    return lib.jscan_prefill_noalloc(a["batch"], a["L"], a["d_inner"], a["d_state"], a["io"], a["x"],
                                     a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["h0"], a["y"],
                                     a["hT"], a["stream"])


def test_noalloc_validates_like_prefill(lib):
    """jscan_prefill_noalloc rejects what jscan_prefill rejects, before any HIP call."""
    assert call_noalloc(lib, prefill_args(x=None)) == NULL
    assert call_noalloc(lib, prefill_args(L=-1)) == SHAPE
    assert call_noalloc(lib, prefill_args(d_state=8)) == UNSUP
    assert call_noalloc(lib, prefill_args(y=fake(0))) == ALIAS
    assert call_noalloc(lib, prefill_args(batch=0)) == OK


def test_noalloc_rejects_problems_beyond_its_scratch(lib):
    """The scratch holds 64 MiB of chunk records: 136 bytes per (sequence,
    chunk, channel).  Batch 8 x 16K at 1024 chunks needs far more; the
    automatic plan at batch 1 x 64K (32 chunks) fits."""
    try:
        js.set_plan_override(1, 1024)
        assert call_noalloc(lib, prefill_args(batch=8, L=16384, d_inner=8192)) == WS
        msg = lib.jscan_last_error().decode()
        assert "needs" in msg and str(64 << 20) in msg
        js.set_plan_override(1, 60)
        assert 60 * 8192 * 136 <= (64 << 20)
        js.set_plan_override(1, 61)
        assert call_noalloc(lib, prefill_args(batch=1, L=65536, d_inner=8192)) == WS
    finally:
        js.set_plan_override(0, 0)
    assert js.plan(1, 65536, 8192)[1] * 8192 * 136 + 5 * 256 <= (64 << 20)


def rms_region(rows):
    """Bytes of a prefill workspace's RMSNorm region: per token the time step's
    inverse root-mean-square and the normalised B and C rows, fp32, each part
    rounded up to 256 bytes."""
    up = lambda v: (v + 255) // 256 * 256
    return up(rows * 4) + 2 * up(rows * 16 * 4)


def test_prefill_workspace_too_small(lib):
    """jscan_prefill_workspace_size covers every variant: a plain call needs the
    records of its plan, a call with RMSNorm also the RMSNorm region."""
    L, d = 65536, 8192
    ws = js.workspace_size(1, L, d)
    rec = ws - rms_region(L)
    assert rec > 0
    assert call_prefill(lib, prefill_args(L=L, d_inner=d, workspace=fake(10), ws_bytes=rec - 1)) == WS
    base = dict(conv_weight=None, conv_bias=None, conv_state_in=None, conv_state_out=None, dt_bias=None)
    pro = prologue(**base, rms_dt_weight=fake(24))
    a = prefill_args(L=L, d_inner=d, workspace=fake(10), ws_bytes=ws - 1)
    assert call_prefill_fused(lib, a, pro) == WS
    # a one-chunk plan records nothing, but RMSNorm still needs its region
    assert js.plan(64, 100, 8192)[1] == 1
    assert js.workspace_size(64, 100, 8192) == rms_region(6400)


def test_workspace_size_formula(lib):
    # single-pass plans need no workspace; chunked plans hold the sub-chunk
    # records (16 fp32 states and a delta sum per channel) and per-chunk start
    # states
    K, chunks = js.plan(1, 65536, 8192)
    assert K == 1 and chunks > 1
    assert js.workspace_size(1, 65536, 8192) >= 2 * chunks * 8192 * 16 * 4
    # a chunked forward always records; a one-chunk forward records only for the backward's sub-chunks
    assert js.plan(16, 4096, 8192)[1] == 1 or js.workspace_size(16, 4096, 8192) > 0
    assert js.workspace_size(1, 64, 128, 15) == 0
    assert js.workspace_size(-1, 64, 128) == 0
    assert js.workspace_size(0, 0, 0) == 0
    # no channel groups (batch 0 or d_inner 0) with tokens: a single-pass plan
    assert js.workspace_size(0, 65536, 8192) == 0
    assert js.plan(0, 65536, 8192) == (1, 1) and js.plan(1, 65536, 0) == (1, 1)


def test_automatic_plan_fills_mi355x():
    # at least two waves per SIMD and a workgroup per CU for the Jamba shapes
    for batch, L in ((1, 65536), (1, 262144), (2, 4096), (8, 16384), (16, 4096)):
        K, chunks = js.plan(batch, L, 8192)
        assert K == 1
        groups = batch * 8192 // 64
        assert groups * chunks >= 2048
        assert groups * chunks >= 256
    assert js.plan(1, 65536, 8192)[1] > 1            # batch 1 needs chunks


def test_plan_override_round_trip():
    try:
        js.set_plan_override(1, 3)
        assert js.plan(1, 300, 64) == (1, 3)
        js.set_plan_override(1, 1000)                 # chunks are whole 8-token blocks
        assert js.plan(1, 10, 64) == (1, 2)
        assert js.plan(1, 4096, 64) == (1, 512)
        for bad in ((2, 4), (4, 1), (3, 1), (1, 0), (1, 4097)):
            with pytest.raises(js.JscanError):
                js.set_plan_override(*bad)
    finally:
        js.set_plan_override(0, 0)


def step_args(n_seq=2, d_inner=64, d_state=16, io=BF16, **over):
    a = dict(n_seq=n_seq, d_inner=d_inner, d_state=d_state, io=io, state=fake(0), x=fake(1), delta=fake(2),
             A=fake(3), B=fake(4), C=fake(5), D=fake(6), z=fake(7), y=fake(8), stream=None)
    a.update(over)
    return a


def call_step_batch(lib, a):
    return lib.jscan_step_batch(a["n_seq"], a["d_inner"], a["d_state"], a["io"], a["state"], a["x"],
                                a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["y"], a["stream"])


@pytest.mark.parametrize("name", ["state", "x", "delta", "A", "B", "C", "D", "z", "y"])
def test_step_null_and_alignment(lib, name):
    assert call_step_batch(lib, step_args(**{name: None})) == NULL
    a = step_args()
    a[name] = ctypes.c_void_p(a[name].value + 4)
    assert call_step_batch(lib, a) == ALIGN


def test_step_validation(lib):
    assert call_step_batch(lib, step_args(n_seq=-1)) == SHAPE
    assert call_step_batch(lib, step_args(d_state=8)) == UNSUP
    assert call_step_batch(lib, step_args(io=5)) == UNSUP
    assert call_step_batch(lib, step_args(y=fake(1))) == ALIAS        # y on x
    assert call_step_batch(lib, step_args(y=fake(0, 64))) == ALIAS    # y inside the state
    assert call_step_batch(lib, step_args(n_seq=0)) == OK
    assert lib.jscan_step(64, 16, BF16, None, fake(1), fake(2), fake(3), fake(4), fake(5), fake(6),
                          fake(7), fake(8), None) == NULL


def test_binding_fails_loudly_without_library(tmp_path):
    # A missing library is an error, never a silent fallback.
    saved = js._lib
    try:
        js._lib = None
        with pytest.raises(js.JscanUnavailable):
            js.load_library(str(tmp_path / "missing.so"))
    finally:
        js._lib = saved


# ------------------------------------------------------------ fused prologue
def prologue(**over):
    p = dict(conv_weight=fake(11), conv_bias=fake(12), conv_state_in=fake(13), conv_state_out=fake(14),
             dt_bias=fake(15), conv_width=4, dt_softplus=1, rms_dt_weight=None, rms_B_weight=None,
             rms_C_weight=None)
    p.update(over)
    s = js.Prologue()
    for k, v in p.items():
        setattr(s, k, v.value if isinstance(v, ctypes.c_void_p) else v)
    s.rms_eps = 1e-6
    return s


def call_prefill_fused(lib, a, pro):
    return lib.jscan_prefill_fused(a["batch"], a["L"], a["d_inner"], a["d_state"], a["io"], a["x"], a["delta"],
                                   a["A"], a["B"], a["C"], a["D"], a["z"], a["h0"], a["y"], a["hT"],
                                   ctypes.byref(pro) if pro is not None else None, a["workspace"], a["ws_bytes"],
                                   a["stream"])


def test_prefill_fused_validation(lib):
    a = prefill_args()
    for w in (0, 5, -1):
        assert call_prefill_fused(lib, a, prologue(conv_width=w)) == UNSUP
    # conv bias or history without weights
    assert call_prefill_fused(lib, a, prologue(conv_weight=None)) == NULL
    # misaligned prologue arrays
    for name in ("conv_weight", "conv_bias", "conv_state_in", "conv_state_out", "dt_bias"):
        bad = ctypes.c_void_p(getattr(prologue(), name) + 4)
        assert call_prefill_fused(lib, a, prologue(**{name: bad})) == ALIGN
    # conv_state_out on top of an input, or of y
    assert call_prefill_fused(lib, a, prologue(conv_state_out=fake(0))) == ALIAS
    assert call_prefill_fused(lib, a, prologue(conv_state_out=fake(8, 256))) == ALIAS
    # conv_state_out partly over conv_state_in (history is 1 x 3 x 128 fp32 = 1536 B)
    assert call_prefill_fused(lib, a, prologue(conv_state_out=fake(13, 512))) == ALIAS
    # y over the conv weights
    assert call_prefill_fused(lib, prefill_args(y=fake(11)), prologue()) == ALIAS
    # the nothing-to-do case still validates the prologue
    assert call_prefill_fused(lib, prefill_args(batch=0), prologue(conv_width=9)) == UNSUP


def test_prefill_fused_in_place_history_is_allowed(lib):
    # conv_state_out == conv_state_in passes the alias check; the call then
    # stops at the (deliberately short) workspace, before any launch.
    L, d = 65536, 8192
    ws = js.workspace_size(1, L, d) - rms_region(L)     # the records (no RMSNorm here)
    a = prefill_args(L=L, d_inner=d, workspace=fake(10), ws_bytes=ws - 1)
    assert call_prefill_fused(lib, a, prologue(conv_state_out=fake(13))) == WS
    assert call_prefill_fused(lib, a, prologue()) == WS
    assert call_prefill_fused(lib, a, None) == WS


def test_step_fused_validation(lib):
    a = step_args()

    def call(pro):
        return lib.jscan_step_batch_fused(a["n_seq"], a["d_inner"], a["d_state"], a["io"], a["state"], a["x"],
                                          a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["y"],
                                          ctypes.byref(pro), a["stream"])
    assert call(prologue(conv_width=7)) == UNSUP
    assert call(prologue(conv_weight=None)) == NULL
    assert call(prologue(dt_bias=ctypes.c_void_p(fake(15).value + 8))) == ALIGN
    # history over the state (2 x 64 x 16 fp32 = 8 KiB)
    assert call(prologue(conv_state_out=fake(0, 1024), conv_state_in=fake(13))) == ALIAS
    # y over the conv weights
    assert lib.jscan_step_batch_fused(2, 64, 16, BF16, fake(0), fake(1), fake(2), fake(3), fake(4), fake(5),
                                      fake(6), fake(7), fake(11), ctypes.byref(prologue()), None) == ALIAS
    assert lib.jscan_step_batch_fused(0, 64, 16, BF16, None, None, None, None, None, None, None, None, None,
                                      ctypes.byref(prologue(conv_width=9)), None) == UNSUP


def test_step_fused_workspace_validation(lib):
    """jscan_step_batch_fused_ws: the RMSNorm rows need jscan_step_workspace_size()
    bytes; the workspace is checked like any other output buffer; without
    RMSNorm it needs none."""
    a = step_args()
    rms = prologue(rms_B_weight=fake(24), rms_C_weight=fake(25))
    need = lib.jscan_step_workspace_size(a["n_seq"], a["d_inner"], 16, BF16, ctypes.byref(rms))
    assert need >= a["n_seq"] * 132
    assert lib.jscan_step_workspace_size(a["n_seq"], a["d_inner"], 16, BF16, ctypes.byref(prologue())) == 0
    assert lib.jscan_step_workspace_size(a["n_seq"], a["d_inner"], 16, BF16, None) == 0
    assert lib.jscan_step_workspace_size(0, a["d_inner"], 16, BF16, ctypes.byref(rms)) == 0

    def call(pro, ws, ws_bytes):
        return lib.jscan_step_batch_fused_ws(a["n_seq"], a["d_inner"], a["d_state"], a["io"], a["state"], a["x"],
                                             a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["y"],
                                             ctypes.byref(pro), ws, ws_bytes, a["stream"])
    assert call(rms, fake(30), need - 1) == WS
    assert call(rms, ctypes.c_void_p(fake(30).value + 8), need) == ALIGN
    assert call(rms, fake(0, 256), need) == ALIAS                  # workspace inside the state
    assert call(rms, fake(1), need) == ALIAS                       # over x
    assert call(prologue(conv_width=7), fake(30), need) == UNSUP
    # no RMSNorm: the workspace is not needed, so a short one is accepted (nothing to
    # launch here would fail only on the GPU, so only the rejected calls are made)
    assert call(prologue(conv_weight=None), fake(30), 0) == NULL


# ------------------------------------------------------------------ backward
def bwd_args(batch=1, L=64, d_inner=128, d_state=16, io=BF16, **over):
    a = dict(batch=batch, L=L, d_inner=d_inner, d_state=d_state, io=io, x=fake(0), delta=fake(1), A=fake(2),
             B=fake(3), C=fake(4), D=fake(5), z=fake(6), h0=fake(7), dy=fake(8), dhT=fake(9), dx=fake(16),
             ddelta=fake(17), dz=fake(18), dA=fake(19), dB=fake(20), dC=fake(21), dD=fake(22), dh0=fake(23),
             workspace=None, ws_bytes=0, stream=None)
    a.update(over)
    return a


def call_bwd(lib, a):
    keys = ("batch", "L", "d_inner", "d_state", "io", "x", "delta", "A", "B", "C", "D", "z", "h0", "dy", "dhT",
            "dx", "ddelta", "dz", "dA", "dB", "dC", "dD", "dh0", "workspace", "ws_bytes", "stream")
    return lib.jscan_backward(*(a[k] for k in keys))


@pytest.mark.parametrize("name", ["x", "delta", "B", "C", "z", "dy", "dx", "ddelta", "dz", "dB", "dC", "A", "D",
                                  "dA", "dD"])
def test_backward_null_required_pointer(lib, name):
    assert call_bwd(lib, bwd_args(**{name: None})) == NULL


@pytest.mark.parametrize("name", ["x", "dy", "dhT", "dx", "dA", "dB", "dh0"])
def test_backward_alignment(lib, name):
    a = bwd_args()
    a[name] = ctypes.c_void_p(a[name].value + 4)
    assert call_bwd(lib, a) == ALIGN


def test_backward_validation(lib):
    assert call_bwd(lib, bwd_args(L=-1)) == SHAPE
    assert call_bwd(lib, bwd_args(d_state=8)) == UNSUP
    assert call_bwd(lib, bwd_args(io=3)) == UNSUP
    assert call_bwd(lib, bwd_args(dx=fake(0))) == ALIAS                 # dx on x
    assert call_bwd(lib, bwd_args(dh0=fake(9))) == ALIAS                # dh0 on dhT (no in-place)
    assert call_bwd(lib, bwd_args(dB=fake(16, 64))) == ALIAS            # dB inside dx
    assert call_bwd(lib, bwd_args(dA=fake(5))) == ALIAS                 # dA on D
    ws = js.backward_workspace_size(1, 64, 128)
    assert ws > 0
    assert call_bwd(lib, bwd_args(workspace=fake(30), ws_bytes=ws - 1)) == WS
    assert call_bwd(lib, bwd_args(workspace=fake(8), ws_bytes=ws)) == ALIAS   # workspace over dy


def call_bwd_saved(lib, a):
    keys = ("batch", "L", "d_inner", "d_state", "io", "x", "delta", "A", "B", "C", "D", "z", "h0", "dy", "dhT",
            "dx", "ddelta", "dz", "dA", "dB", "dC", "dD", "dh0", "pws", "pws_bytes", "workspace", "ws_bytes",
            "stream")
    return lib.jscan_backward_saved(*(a[k] for k in keys))


def test_backward_saved_validation(lib):
    """jscan_backward_saved checks the prefill workspace like any other buffer
    (required when the plan runs in chunks) and needs a smaller workspace."""
    try:
        js.set_plan_override(1, 4)
        pws = js.workspace_size(1, 64, 128)
        full = js.backward_workspace_size(1, 64, 128)
        assert pws > 0 and full > pws
        sv = lambda **kw: call_bwd_saved(lib, bwd_args(**{"pws": fake(31), "pws_bytes": pws, **kw}))
        assert sv(pws=None) == NULL                           # chunked plan: the prefill's workspace is required
        assert sv(pws_bytes=pws - 1) == WS
        assert sv(pws=fake(31, 4)) == ALIGN
        assert sv(pws=fake(16)) == ALIAS                      # prefill workspace under dx
        assert sv(workspace=fake(31, 64)) == ALIAS            # workspace over the prefill workspace
        assert sv(workspace=fake(30), ws_bytes=full - pws - 1) == WS
        assert sv(x=None) == NULL
        assert sv(L=-1) == SHAPE
        assert sv(d_state=8) == UNSUP
    finally:
        js.set_plan_override(0, 0)


def test_backward_workspace_size():
    # recomputed states (~8 B per channel-token) and the dB/dC partials dominate
    L, d = 65536, 8192
    assert js.backward_workspace_size(1, L, d) >= L * d * 8
    assert js.backward_workspace_size(0, L, d) == 0
    assert js.backward_workspace_size(1, L, d, 15) == 0


# ------------------------------------------------------------- trapezoidal
def test_prefill_trap_validation(lib):
    a = prefill_args()
    keys = ("batch", "L", "d_inner", "d_state", "io", "x", "delta", "A", "B", "C", "D", "z", "h0", "y", "hT")

    def call(trap, pro=None, **over):
        b = dict(a, **over)
        return lib.jscan_prefill_trap(*(b[k] for k in keys), ctypes.byref(trap) if trap is not None else None,
                                      ctypes.byref(pro) if pro is not None else None, b["workspace"],
                                      b["ws_bytes"], b["stream"])
    t = js.Trap()
    t.lam, t.x_prev, t.B_prev = fake(11).value, fake(12).value, fake(13).value
    assert call(t, prologue()) == UNSUP                          # no convolution with the trapezoidal form
    bad = js.Trap()
    bad.lam = fake(11).value + 2
    assert call(bad) == ALIGN
    alias = js.Trap()
    alias.lam = fake(8).value                                    # lam on top of y
    assert call(alias) == ALIAS
    assert call(t, batch=0) == OK                                # nothing to do
    # the decode step: lam [n_seq][d_inner] over the state is an alias
    s = step_args()
    st = js.Trap()
    st.lam = fake(0, 128).value
    assert lib.jscan_step_batch_trap(s["n_seq"], s["d_inner"], s["d_state"], s["io"], s["state"], s["x"],
                                     s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"], s["y"],
                                     ctypes.byref(st), None, None) == ALIAS


def test_prologue_rmsnorm_validation(lib):
    a = prefill_args()
    base = dict(conv_weight=None, conv_bias=None, conv_state_in=None, conv_state_out=None, dt_bias=None)
    p = prologue(**base, rms_dt_weight=fake(24), rms_B_weight=fake(25), rms_C_weight=fake(26))
    p.rms_eps = -1.0
    assert call_prefill_fused(lib, a, p) == UNSUP                 # eps must be >= 0
    p.rms_eps = float("nan")
    assert call_prefill_fused(lib, a, p) == UNSUP
    p.rms_eps = 1e-6
    p.rms_B_weight = fake(25).value + 4
    assert call_prefill_fused(lib, a, p) == ALIGN
    p.rms_B_weight = fake(8).value                                # weight on top of y
    assert call_prefill_fused(lib, a, p) == ALIAS
    # with the trapezoidal form: unsupported
    q = prologue(**base, rms_dt_weight=fake(24))
    t = js.Trap()
    keys = ("batch", "L", "d_inner", "d_state", "io", "x", "delta", "A", "B", "C", "D", "z", "h0", "y", "hT")
    assert lib.jscan_prefill_trap(*(a[k] for k in keys), ctypes.byref(t), ctypes.byref(q), None, 0, None) == UNSUP


def test_prefill_stats_arguments(lib):
    """jscan_prefill_stats checks its arguments before it touches the workspace:
    a single-chunk plan reads nothing, and a workspace smaller than the plan's
    records is refused."""
    ST = {v: k for k, v in js.STATUS_NAMES.items()}
    out = (ctypes.c_double * 3)()
    fake = ctypes.c_void_p(0x1000)       # never dereferenced on these paths
    assert lib.jscan_prefill_stats(None, 0, 1, 65536, 8192, out, None) == ST["JSCAN_ERR_NULL"]
    assert lib.jscan_prefill_stats(fake, 1 << 30, 1, 65536, 8192, None, None) == ST["JSCAN_ERR_NULL"]
    assert lib.jscan_prefill_stats(fake, 1 << 30, -1, 65536, 8192, out, None) == ST["JSCAN_ERR_SHAPE"]
    assert lib.jscan_prefill_stats(fake, 1 << 30, 1, 0, 8192, out, None) == ST["JSCAN_ERR_SHAPE"]
    assert js.plan(1, 64, 128)[1] == 1
    assert lib.jscan_prefill_stats(fake, 0, 1, 64, 128, out, None) == js.JSCAN_OK
    assert tuple(out) == (0.0, 0.0, 1.0)
    assert js.plan(1, 65536, 8192)[1] > 1
    need = js.workspace_size(1, 65536, 8192) - rms_region(65536)
    assert lib.jscan_prefill_stats(fake, need - 1, 1, 65536, 8192, out, None) == ST["JSCAN_ERR_WORKSPACE"]


def test_step_size_limit(lib):
    """The decode step's one-dimensional grid (four lanes per sequence-channel)
    holds at most 2^32 work-items: n_seq * d_inner up to 2^30 - 64 passes the
    size check (and then fails on the NULL pointers, before any GPU work), one
    more is JSCAN_ERR_SHAPE, for the plain, fused and trapezoidal steps."""
    ST = {v: k for k, v in js.STATUS_NAMES.items()}
    limit = (1 << 30) - 64
    args = [None] * 9 + [None]

    def plain(n, d):
        return lib.jscan_step_batch(n, d, 16, js.IO_BF16, *args)

    def fused(n, d):
        return lib.jscan_step_batch_fused(n, d, 16, js.IO_BF16, *([None] * 9), None, None)

    def trap(n, d):
        return lib.jscan_step_batch_trap(n, d, 16, js.IO_BF16, *([None] * 9), None, None, None)

    for call in (plain, fused, trap):
        assert call(1, limit) == ST["JSCAN_ERR_NULL"]
        assert call(1, limit + 1) == ST["JSCAN_ERR_SHAPE"]
        assert call(limit // 8192 + 1, 8192) == ST["JSCAN_ERR_SHAPE"]
        assert call(-1, 8192) == ST["JSCAN_ERR_SHAPE"]
        assert call(1 << 40, 1 << 40) == ST["JSCAN_ERR_SHAPE"]      # the product overflows
    # jscan_step is the one-sequence case of the same check
    assert lib.jscan_step(limit + 1, 16, js.IO_BF16, *([None] * 9), None) == ST["JSCAN_ERR_SHAPE"]


def test_ubench_library_exports_its_header():
    """libjscan_ubench.so (the VALU measurement library bench.py loads) exports
    every function include/jscan_ubench.h declares, with C linkage."""
    path = os.path.join(os.path.dirname(js.LIB_PATH), "libjscan_ubench.so")
    if not os.path.exists(path):
        from selective_state_space_11_amd import build
        build.build()
    text = open(os.path.join(os.path.dirname(HEADER), "jscan_ubench.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(jscan_[a-z_]+)\s*\(", text)))
    assert names == ["jscan_ubench_valu"]
    ub = ctypes.CDLL(path)
    for name in names:
        assert hasattr(ub, name), name
    # argument checks return before any GPU work
    d = ctypes.c_double()
    fn = ub.jscan_ubench_valu
    fn.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int] + [ctypes.POINTER(ctypes.c_double)] * 5
    ptrs = [ctypes.byref(d)] * 5
    assert fn(9, 4, 1, *ptrs) == 1          # unknown kind
    assert fn(0, 6, 1, *ptrs) == 1          # waves not a multiple of 4
    assert fn(0, 4, 0, *ptrs) == 1          # no iterations
