"""HIP-graph capture of libjscan calls (torch.cuda.CUDAGraph): decode steps
(plain, fused, fused with RMSNorm, trapezoidal), a chunked prefill, the fused
prefill with RMSNorm, the trapezoidal prefill and the backward, given caller
workspaces, launch only kernels on the caller's stream, so they can be
captured once and replayed.

Each graph is replayed several times from the same starting state, with eager
library work and synchronisations between the replays, and every replay must
equal the eager calls bit for bit (the same kernels on the same inputs).
Inputs follow the seeded recipes of ``synth``.
"""
import numpy as np
import pytest
import torch

import synth
import selective_state_space_11_amd as js
from gpu_util import dev_f32, dev_io, to_device

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only machines, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

REPLAYS = 3


def print_case(msg):
    print(f"[case] {msg}", flush=True)


def capture(fn):
    """fn() once on a side stream (warm-up), then captured into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def decode_tokens(n_seq, d, T, seed):
    toks = [synth.decode_inputs(n_seq, d, seed=seed, step=k) for k in range(T)]
    return [{k: dev_io(v[k]) for k in ("x", "delta", "z", "B", "C")} for v in toks]


@pytest.mark.parametrize("variant", ["plain", "fused", "rmsnorm", "trapezoidal"])
def test_decode_steps_replayed(variant):
    """Eight decode steps of 4 sequences x 256 channels: plain; with the
    conv(4) + SiLU and softplus prologue and its conv history in place; the
    same with RMSNorm of delta, B and C, given a step workspace; and the
    exponential-trapezoidal step (lam, and the previous token's x and B row)."""
    print_case(f"graph decode {variant}")
    fused = variant in ("fused", "rmsnorm")
    n_seq, d, T = 4, 256, 8
    A, D, _ = synth.params(d, seed=90)
    A, D = dev_f32(A), dev_f32(D)
    toks = decode_tokens(n_seq, d, T, seed=90)
    pro = synth.prologue_params(d, 4, seed=90, batch=n_seq)
    st0 = dev_f32(synth.decode_state(n_seq, d, seed=90))
    cs0 = dev_f32(pro["conv_state"])
    kw = dict(conv_weight=dev_f32(pro["conv_weight"]), conv_bias=dev_f32(pro["conv_bias"]),
              dt_bias=dev_f32(pro["dt_bias"]), softplus=True)
    if variant == "rmsnorm":
        kw["rms"] = tuple(dev_f32(w) for w in synth.rms_weights(d, seed=90)) + (1e-5,)
        kw["workspace"] = torch.empty(js.step_workspace_size(n_seq, d, kw["rms"]), dtype=torch.uint8,
                                      device="cuda")
        assert kw["workspace"].numel() > 0

    lam = [dev_io(synth.trap_inputs(n_seq, 1, d, seed=90 + k)[0][:, 0, :]) for k in range(T)]

    def steps(st, cs, ys):
        for k, t in enumerate(toks):
            if fused:
                js.step_batch_fused(st, t["x"], t["delta"], A, t["B"], t["C"], D, t["z"], conv_state=cs, y=ys[k],
                                    **kw)
            elif variant == "trapezoidal":
                prev = toks[k - 1] if k else toks[T - 1]
                js.step_batch_trap(st, t["x"], t["delta"], A, t["B"], t["C"], D, t["z"], lam=lam[k], x_prev=prev["x"],
                                   B_prev=prev["B"], y=ys[k])
            else:
                js.step_batch(st, t["x"], t["delta"], A, t["B"], t["C"], D, t["z"], y=ys[k])

    st_ref, cs_ref = st0.clone(), cs0.clone()
    ys_ref = [torch.empty_like(toks[0]["x"]) for _ in range(T)]
    steps(st_ref, cs_ref, ys_ref)
    torch.cuda.synchronize()

    st, cs = st0.clone(), cs0.clone()
    ys = [torch.empty_like(toks[0]["x"]) for _ in range(T)]
    g = capture(lambda: steps(st, cs, ys))
    other = st0.clone()
    for rep in range(REPLAYS):
        st.copy_(st0)
        cs.copy_(cs0)
        for y in ys:
            y.zero_()
        js.step_batch(other, toks[rep]["x"], toks[rep]["delta"], A, toks[rep]["B"], toks[rep]["C"], D,
                      toks[rep]["z"])           # eager library work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in range(T):
            assert torch.equal(ys[k], ys_ref[k]), (rep, k)
        assert torch.equal(st, st_ref), rep
        if fused:
            assert torch.equal(cs, cs_ref), rep


def test_chunked_prefill_replayed():
    """A prefill of 2 x 1000 tokens x 256 channels in a forced 4-chunk plan with
    a caller workspace (chunk-local pass, combine and rescan in the graph)."""
    print_case("graph prefill chunks=4")
    b, L, d = 2, 1000, 256
    inp = synth.prefill_inputs(b, L, d, seed=91, io=synth.IO_BF16, h0=True)
    t = to_device(inp)
    try:
        js.set_plan_override(1, 4)
        assert js.plan(b, L, d)[1] == 4
        ws = torch.empty(js.workspace_size(b, L, d), dtype=torch.uint8, device="cuda")
        y_ref, h_ref = js.prefill(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"],
                                  workspace=ws)
        torch.cuda.synchronize()
        y, hT = torch.empty_like(y_ref), torch.empty_like(h_ref)
        g = capture(lambda: js.prefill(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"], y=y,
                                       hT=hT, workspace=ws))
        for rep in range(REPLAYS):
            y.zero_()
            hT.zero_()
            ws.zero_()
            js.prefill(t["x"][:1], t["delta"][:1], t["A"], t["B"][:1], t["C"][:1], t["D"], t["z"][:1])
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, y_ref), rep
            assert torch.equal(hT, h_ref), rep
    finally:
        js.set_plan_override(0, 0)


def test_backward_and_trapezoidal_prefill_replayed():
    """The backward (chunked plan, caller workspace and outputs) and the
    trapezoidal prefill (lam given, caller workspace) captured and replayed."""
    print_case("graph backward and trapezoidal prefill")
    b, L, d = 2, 600, 136
    inp = synth.prefill_inputs(b, L, d, seed=92, io=synth.IO_BF16, h0=True)
    dy, dhT = synth.output_grads(b, L, d, seed=92)
    lam, xp, Bp = synth.trap_inputs(b, L, d, seed=92)
    t = to_device(inp)
    tdy, tdh, tl = dev_io(dy), dev_f32(dhT), dev_io(lam)
    args = (t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"])
    try:
        js.set_plan_override(1, 3)
        bws = torch.empty(js.backward_workspace_size(b, L, d), dtype=torch.uint8, device="cuda")
        pws = torch.empty(js.workspace_size(b, L, d), dtype=torch.uint8, device="cuda")
        g_ref = js.backward(*args, tdy, t["h0"], tdh, workspace=bws)
        y_ref, h_ref = js.prefill_trap(*args, t["h0"], lam=tl, x_prev=dev_io(xp), B_prev=dev_io(Bp), workspace=pws)
        torch.cuda.synchronize()
        g = {k: torch.empty_like(v) for k, v in g_ref.items()}
        y, hT = torch.empty_like(y_ref), torch.empty_like(h_ref)
        txp, tBp = dev_io(xp), dev_io(Bp)

        def work():
            js.backward(*args, tdy, t["h0"], tdh, workspace=bws, out=g)
            js.prefill_trap(*args, t["h0"], lam=tl, x_prev=txp, B_prev=tBp, y=y, hT=hT, workspace=pws)

        graph = capture(work)
        for rep in range(REPLAYS):
            for v in list(g.values()) + [y, hT]:
                v.zero_()
            bws.zero_()
            pws.zero_()
            js.prefill(t["x"][:1], t["delta"][:1], t["A"], t["B"][:1], t["C"][:1], t["D"], t["z"][:1])
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for k in g_ref:
                assert torch.equal(g[k], g_ref[k]), (rep, k)
            assert torch.equal(y, y_ref) and torch.equal(hT, h_ref), rep
    finally:
        js.set_plan_override(0, 0)


def test_fused_rmsnorm_prefill_replayed():
    """The prefill with the whole prologue (conv width 4 + SiLU, softplus, and
    RMSNorm of delta, B and C) given a caller workspace, in a forced 4-chunk
    plan: the RMSNorm pre-pass writes its per-token region inside the
    workspace, so the call allocates nothing and replays bit for bit."""
    print_case("graph fused prefill with RMSNorm chunks=4")
    b, L, d = 2, 1000, 256
    inp = synth.prefill_inputs(b, L, d, seed=93, io=synth.IO_BF16, h0=True)
    t = to_device(inp)
    pro = synth.prologue_params(d, 4, seed=93, batch=b)
    cw, cb, cs, dtb = (torch.from_numpy(pro[k]).cuda() for k in ("conv_weight", "conv_bias", "conv_state",
                                                                 "dt_bias"))
    rms = tuple(torch.from_numpy(w).cuda() for w in synth.rms_weights(d, seed=93)) + (1e-5,)
    try:
        js.set_plan_override(1, 4)
        ws = torch.empty(js.workspace_size(b, L, d), dtype=torch.uint8, device="cuda")
        cso_ref = torch.empty_like(cs)

        def call(y=None, hT=None, cso=cso_ref):
            return js.prefill_fused(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"], y=y,
                                    hT=hT, workspace=ws, conv_weight=cw, conv_bias=cb, conv_state_in=cs,
                                    conv_state_out=cso, dt_bias=dtb, softplus=True, rms=rms)
        y_ref, h_ref = call()
        torch.cuda.synchronize()
        y, hT, cso = torch.empty_like(y_ref), torch.empty_like(h_ref), torch.empty_like(cs)
        g = capture(lambda: call(y, hT, cso))
        for rep in range(REPLAYS):
            y.zero_()
            hT.zero_()
            cso.zero_()
            ws.zero_()
            js.prefill(t["x"][:1], t["delta"][:1], t["A"], t["B"][:1], t["C"][:1], t["D"], t["z"][:1])
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, y_ref), rep
            assert torch.equal(hT, h_ref), rep
            assert torch.equal(cso, cso_ref), rep
    finally:
        js.set_plan_override(0, 0)
