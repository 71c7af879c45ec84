"""jscan_prefill_noalloc through the C ABI against jscan_prefill.

The allocation-free prefill keeps its chunk records in the library's per-GPU
scratch array instead of a workspace.  It runs the same kernels on the same
forward plan as jscan_prefill, so y and hT must match it bit for bit; the
small case is also held to the fp64 oracle.  Two calls in a row, the second
smaller, so the second reuses the array with the first call's contents left
in it.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import selective_state_space_11_amd as js
from gpu_util import assert_state, assert_y, oracle_inputs, to_device

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only machines, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = "cuda"


def print_case(msg):
    print(f"[case] {msg}", flush=True)


def random_problem(batch, L, d_inner, seed):
    """Jamba-distributed inputs drawn on the GPU (x, z ~ N(0,1); delta =
    softplus(N(0,1) - 2); B, C ~ N(0,1)/4; A = -exp(U(0, log 16)); D ~ N(0,1);
    h0 ~ N(0,1)), bf16 I/O."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    bf = torch.bfloat16
    n = lambda *s: torch.randn(*s, generator=g, device=DEV)
    return dict(x=n(batch, L, d_inner).to(bf),
                delta=torch.nn.functional.softplus(n(batch, L, d_inner) - 2).to(bf),
                z=n(batch, L, d_inner).to(bf), B=(n(batch, L, 16) / 4).to(bf), C=(n(batch, L, 16) / 4).to(bf),
                A=-torch.exp(torch.rand(d_inner, 16, generator=g, device=DEV) * float(np.log(16.0))),
                D=n(d_inner), h0=n(batch, d_inner, 16))


def both(t):
    args = (t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"])
    y1, h1 = js.prefill(*args)
    y2 = torch.empty_like(t["x"])
    h2 = torch.empty_like(t["h0"])
    js.prefill_noalloc(*args, y=y2, hT=h2)
    torch.cuda.synchronize()
    return (y1, h1), (y2, h2)


def test_noalloc_matches_prefill_on_two_calls():
    # first call: the benchmark's 64K-token context in its automatic (chunked) plan
    print_case("noalloc 1 x 65536 x 8192")
    assert js.plan(1, 65536, 8192)[1] > 1
    t = random_problem(1, 65536, 8192, seed=71)
    (y1, h1), (y2, h2) = both(t)
    assert torch.equal(y1, y2)
    assert torch.equal(h1, h2)
    del t, y1, y2
    # second call, smaller (ragged sizes, two sequences, a forced 9-chunk plan), also against the oracle
    print_case("noalloc 2 x 777 x 200, 9 chunks")
    inp = synth.prefill_inputs(2, 777, 200, seed=72, io=synth.IO_BF16, h0=True)
    t = to_device(inp)
    try:
        js.set_plan_override(1, 9)
        (y1, h1), (y2, h2) = both(t)
    finally:
        js.set_plan_override(0, 0)
    assert torch.equal(y1, y2)
    assert torch.equal(h1, h2)
    o = oracle_inputs(inp)
    yr, hr = oracle.prefill(o["x"], o["delta"], o["A"], o["B"], o["C"], o["D"], o["z"], o["h0"])
    assert_y(y2, yr, bf16=True)
    assert_state(h2, hr, "hT")


def test_noalloc_single_chunk_and_empty():
    """A one-chunk plan uses no scratch at all; an empty sequence copies h0."""
    print_case("noalloc single chunk / empty")
    t = random_problem(16, 300, 8192, seed=73)
    assert js.plan(16, 300, 8192)[1] == 1
    (y1, h1), (y2, h2) = both(t)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    e = torch.empty(2, 0, 64, dtype=torch.bfloat16, device=DEV)
    eb = torch.empty(2, 0, 16, dtype=torch.bfloat16, device=DEV)
    h0 = torch.randn(2, 64, 16, device=DEV)
    hT = torch.empty_like(h0)
    js.prefill_noalloc(e, e.clone(), torch.randn(64, 16, device=DEV), eb, eb.clone(), torch.randn(64, device=DEV),
                       e.clone(), h0, y=torch.empty_like(e), hT=hT)
    torch.cuda.synchronize()
    assert torch.equal(hT, h0)
