#!/usr/bin/env python3
"""Benchmark: the selective-scan prefill at the Jamba shape with a 64K context.

One step = one jscan_prefill call over batch 1, L = 65536 tokens, d_inner 8192,
d_state 16, bf16 I/O (fp32 state and arithmetic), inputs resident in HBM.
Reports channel-tokens/s (batch * L * d_inner per second), the fraction of the
MI355X HBM roofline those algorithmic bytes reach, the roofline of the main
scan kernel (timed on its own with HIP events recorded by the library on the
launch stream), a decode-step measurement (256 sequences), the same prefill
with the fused input prologue (causal conv of width 4 + SiLU, softplus time
step), the exponential-trapezoidal recurrence, the backward (gradient) scan
of the same prefill, and the fp64 CPU oracle timed on a bounded sample of the
same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
VALU_PEAK_TFLOPS = 157.3       # MI355X fp32 vector, FMA = 2 flops
D_STATE = 16

# Algorithmic VALU issue slots per channel-token of the scan (one slot = one
# fp32 FMA lane-op; a transcendental v_exp_f32 / v_rcp_f32 costs 4 slots, as
# measured on gfx950): per state, delta*A' (1) + exp2 (4) + (delta*x)*B (1) +
# state FMA (1) + C*h FMA (1) = 8, times 16 states = 128; per channel-token,
# delta*x (1), the D skip FMA (1), SiLU(z) = z * rcp(1 + exp2(-z log2 e))
# (mul 1 + exp 4 + add 1 + rcp 4 + mul 1) and the gate multiply (1) = 14.
SLOTS_PER_CHTOK = 16 * 8 + 14


def alg_bytes_prefill(batch, L, d_inner, io_bytes=2, h0=False, hT=True):
    tok = batch * L * d_inner * io_bytes * 4           # x, delta, z in; y out
    rows = batch * L * D_STATE * io_bytes * 2          # B, C
    params = d_inner * D_STATE * 4 + d_inner * 4       # A, D
    state = batch * d_inner * D_STATE * 4 * ((1 if h0 else 0) + (1 if hT else 0))
    return tok + rows + params + state


def alg_bytes_step(n_seq, d_inner, io_bytes=2):
    return (2 * n_seq * d_inner * D_STATE * 4 + n_seq * d_inner * io_bytes * 4
            + n_seq * D_STATE * io_bytes * 2 + d_inner * D_STATE * 4 + d_inner * 4)


def source_digest():
    """Digest of the sources the forward kernels are compiled from."""
    h = hashlib.sha256()
    for f in ("jscan.hip", "common.h"):
        h.update(open(os.path.join(ROOT, "selective_state_space_11_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel_tag):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        data = json.load(open(p))
    except (OSError, ValueError):
        return None
    ent = data.get(kernel_tag)
    if not ent or ent.get("source_sha") != source_digest():
        return None
    return ent.get("hbm_bytes_per_launch")


def _db_rows(db, sql):
    import sqlite3
    con = sqlite3.connect(db)
    try:
        return list(con.execute(sql))
    finally:
        con.close()


def _short(name):
    base = name.replace("(anonymous namespace)::", "").replace("jscan_detail::", "")
    if base.startswith("void "):
        base = base[5:]
    return base.split("(")[0].strip()


def summarize_trace(db, out_md, command):
    """Per-kernel duration table from a rocprofv3 --kernel-trace database."""
    rows = _db_rows(db, "select name, duration from kernels order by start")
    stats = {}
    for name, dur in rows:
        stats.setdefault(_short(name), []).append(dur / 1000.0)
    lines = [f"# Kernel trace: {os.path.basename(os.path.dirname(out_md)) and os.path.basename(out_md)[:-3]}", "",
             "Command (on the MI355X box, from the repository root):", "", "```", command, "```", "",
             "| kernel | calls | average (us) | median (us) | min (us) | max (us) | total (us) |",
             "|---|---|---|---|---|---|---|"]
    for k, v in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        med = sorted(v)[len(v) // 2]
        lines.append(f"| {k} | {len(v)} | {sum(v) / len(v):.1f} | {med:.1f} | {min(v):.1f} | {max(v):.1f} | "
                     f"{sum(v):.1f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")
    return stats


def summarize_traffic(pmc_dir, out_md, out_json, command):
    """HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for a plain 1 GiB -> 1 GiB copy."""
    def per_kernel(sub, counter):
        rows = _db_rows(os.path.join(pmc_dir, sub, "run_results.db"),
                        f"select name, dispatch_id, counter_value from pmc_events where counter_name='{counter}'")
        per = {}
        for name, disp, val in rows:
            per.setdefault(_short(name), {}).setdefault(disp, 0.0)
            per[_short(name)][disp] += val
        return {k: sorted(v.values())[len(v) // 2] * 1024.0 for k, v in per.items()}   # median, bytes
    fetch, write = per_kernel("fetch", "FETCH_SIZE"), per_kernel("write", "WRITE_SIZE")
    cf, cw = per_kernel("copy_fetch", "FETCH_SIZE"), per_kernel("copy_write", "WRITE_SIZE")
    copy = "__amd_rocclr_copyBuffer"
    f_scale, w_scale = (1 << 30) / cf[copy], (1 << 30) / cw[copy]
    lines = ["# HBM traffic per dispatch (rocprofv3 counters, 64K-token prefill, batch 1, d_inner 8192)", "",
             "Commands (on the MI355X box, from the repository root):", "", "```", command, "```", "",
             f"Calibration: a 1 GiB -> 1 GiB device copy reads FETCH_SIZE = {cf[copy] / 1024:.0f} KiB and "
             f"WRITE_SIZE = {cw[copy] / 1024:.0f} KiB, so FETCH_SIZE is scaled by {f_scale:.3f} and "
             f"WRITE_SIZE by {w_scale:.3f}.", "",
             "| kernel | read (MB) | written (MB) | total (MB) |", "|---|---|---|---|"]
    res = {}
    for k in sorted(fetch, key=lambda k: -fetch[k]):
        if k.startswith("__amd") or k.startswith("at::"):
            continue
        r, w = fetch[k] * f_scale, write.get(k, 0.0) * w_scale
        res[k] = r + w
        lines.append(f"| {k} | {r / 1e6:.1f} | {w / 1e6:.1f} | {(r + w) / 1e6:.1f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")
    # the plain main scan: bf16, one wave per 64 channels, every optional stage off
    plain = [k for k in res if re.fullmatch(r"k_scan<unsigned short, 1(, false)*>", k)]
    data = {"k_scan_64k": {"source_sha": source_digest(),
                           "hbm_bytes_per_launch": res[plain[0]] if plain else None,
                           "fetch_scale": f_scale, "write_scale": w_scale}}
    json.dump(data, open(out_json, "w"), indent=1)
    return res


def summarize_counters(pmc_dir, out_md, command, trace_db=None):
    """Per-kernel medians of every SQ_/GRBM_ counter found in the rocprofv3
    --pmc runs under pmc_dir (one sub-folder per run), with the VALU issue
    figures derived from them.

    A VALU wave instruction covers 64 lanes.  A transcendental (exp2, log2,
    rcp) takes the issue time of four plain fp32 instructions, so the fp32
    slot count is SQ_INSTS_VALU + 3 * SQ_INSTS_VALU_TRANS_F32.  The chip's
    plain fp32 rate is 157.3e12 / 2 lane-instructions per second."""
    import glob
    per = {}
    for db in sorted(glob.glob(os.path.join(pmc_dir, "*", "run_results.db"))):
        rows = _db_rows(db, "select name, dispatch_id, counter_name, counter_value from pmc_events")
        acc = {}
        for name, disp, cname, val in rows:
            key = (_short(name), cname)
            acc.setdefault(key, {}).setdefault(disp, 0.0)
            acc[key][disp] += val
        for (k, c), v in acc.items():
            vals = sorted(v.values())
            per.setdefault(k, {})[c] = vals[len(vals) // 2]
    durs = {}
    if trace_db:
        for name, dur in _db_rows(trace_db, "select name, duration from kernels"):
            durs.setdefault(_short(name), []).append(dur / 1e9)
    counters = sorted({c for v in per.values() for c in v})
    lines = ["# SQ counters per dispatch (rocprofv3 --pmc, median over dispatches)", "",
             "Commands (on the MI355X box, from the repository root):", "", "```", command, "```", "",
             "`fp32 slots` = SQ_INSTS_VALU + 3 x SQ_INSTS_VALU_TRANS_F32 (a transcendental issues in the time "
             "of four plain instructions), in wave instructions of 64 lanes. `VALU issue` = fp32 slots x 64 / "
             "(median kernel-trace duration x 78.65e12 lane-instructions/s), the fraction of the chip's plain "
             "fp32 issue rate the kernel kept busy (trace durations include the profiler's own overhead).", "",
             "| kernel | " + " | ".join(counters) + " | fp32 slots | VALU issue |",
             "|---|" + "---|" * (len(counters) + 2)]
    order = sorted(per, key=lambda k: -per[k].get("SQ_INSTS_VALU", 0.0))
    for k in order:
        if k.startswith("__amd") or k.startswith("at::"):
            continue
        v = per[k]
        slots = v.get("SQ_INSTS_VALU", 0.0) + 3 * v.get("SQ_INSTS_VALU_TRANS_F32", 0.0)
        busy = ""
        if k in durs and slots and "SQ_INSTS_VALU_TRANS_F32" in v:
            d = sorted(durs[k])[len(durs[k]) // 2]
            busy = f"{slots * 64 / (d * 78.65e12):.3f}"
        cells = [f"{v[c]:.4g}" if c in v else "" for c in counters]
        lines.append(f"| {k} | " + " | ".join(cells) + f" | {slots:.4g} | {busy} |")
    open(out_md, "w").write("\n".join(lines) + "\n")
    return per


UBENCH_KINDS = {0: "fp32 FMA", 1: "exp2 (v_exp_f32)", 2: "1 exp2 + 4 independent FMA",
                3: "scan token step (16 x: mul, exp2, mul, FMA, FMA)"}


def valu_ceiling(waves_per_simd=(1, 2, 4, 8)):
    """Measured VALU rates of this GPU (libjscan_ubench.so), per CU per shader
    clock.  Returns a dict; the plain-FMA rate is the chip's fp32 issue peak,
    the scan-step rate the ceiling of the scan's instruction mix."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "selective_state_space_11_amd", "libjscan_ubench.so"))
    d = ctypes.c_double
    lib.jscan_ubench_valu.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int] + [ctypes.POINTER(d)] * 6
    lib.jscan_ubench_valu.restype = ctypes.c_int
    n_cu = 256
    iters = {0: 20000, 1: 5000, 2: 20000, 3: 5000}
    rows = []
    for kind in (0, 1, 2, 3):
        for wps in (waves_per_simd if kind == 0 else (8,)):
            waves = n_cu * 4 * wps
            it = max(1, iters[kind] * 8 // wps)
            out = [d() for _ in range(6)]
            rc = lib.jscan_ubench_valu(kind, waves, it, *[ctypes.byref(o) for o in out])
            if rc != 0:
                raise RuntimeError(f"jscan_ubench_valu(kind {kind}) failed with {rc}")
            sec, lane, trans, clk, wall = (o.value for o in out[:5])
            rate = lane / sec
            rows.append({"kind": UBENCH_KINDS[kind], "waves_per_simd": wps, "seconds": sec,
                         "lane_instr_per_s": rate, "trans_lane_instr_per_s": trans / sec,
                         "clock_mhz": round(clk, 1),
                         "lane_instr_per_cu_per_clock": rate / (n_cu * clk * 1e6) if clk else None})
    fma = max(r["lane_instr_per_s"] for r in rows if r["kind"] == UBENCH_KINDS[0])
    exp = next(r for r in rows if r["kind"] == UBENCH_KINDS[1])["lane_instr_per_s"]
    mix = next(r for r in rows if r["kind"] == UBENCH_KINDS[2])
    scan = next(r for r in rows if r["kind"] == UBENCH_KINDS[3])
    # a transcendental's cost in plain-FMA issue slots, and whether it overlaps FMAs:
    # group = 1 exp + 4 FMA; serial cost = 4 + exp_slots, parallel = max(4, exp_slots)
    exp_slots = fma / exp
    group_slots = 5 * fma / mix["lane_instr_per_s"]
    scan_instr = 5 * 16 + 3                           # per token: 16 x (mul, exp, mul, fma, fma) + 3
    scan_slots_model = scan_instr - 16 + 16 * exp_slots
    scan_slot_rate = scan["lane_instr_per_s"] / scan_instr * scan_slots_model / fma
    return {"rows": rows, "fma_lane_instr_per_s": fma, "exp_slots": exp_slots,
            "exp_plus_4fma_group_slots": group_slots, "scan_step_slots_per_chtok": scan_slots_model,
            "scan_step_frac_of_fma_peak": scan_slot_rate,
            "scan_step_chtok_per_s": scan["lane_instr_per_s"] / scan_instr}


def run_valu_ceiling(out_md, command):
    r = valu_ceiling()
    print(json.dumps(r), flush=True)
    if not out_md:
        return
    lines = ["# VALU throughput of the MI355X (gfx950) for the scan's instruction mixes", "",
             "Command (on the MI355X box, from the repository root):", "", "```", command, "```", "",
             "Kernels: `selective_state_space_11_amd/csrc/ubench.hip` (built by `__graft_entry__.build()`), plain "
             "fp32 only (packed fp32 off). `rate` is VALU lane-instructions per second over one timed launch; "
             "`per CU per clock` divides by 256 CUs and the shader clock the kernel itself read (s_memtime "
             "over s_memrealtime).", "",
             "| kernel | waves per SIMD | time (ms) | rate (lane-instr/s) | clock (MHz) | per CU per clock |",
             "|---|---|---|---|---|---|"]
    for x in r["rows"]:
        pc = x["lane_instr_per_cu_per_clock"]
        lines.append(f"| {x['kind']} | {x['waves_per_simd']} | {x['seconds'] * 1e3:.2f} | "
                     f"{x['lane_instr_per_s']:.4g} | {x['clock_mhz']:.0f} | {pc:.1f} |")
    lines += ["", f"- one v_exp_f32 costs {r['exp_slots']:.2f} plain-FMA issue slots;",
              f"- a group of 1 exp2 + 4 independent FMAs costs {r['exp_plus_4fma_group_slots']:.2f} slots "
              f"(4 + {r['exp_slots']:.2f} = {4 + r['exp_slots']:.2f} if they do not overlap, "
              f"{max(4, r['exp_slots']):.2f} if they do);",
              f"- the scan's token step (16 states) costs {r['scan_step_slots_per_chtok']:.1f} slots and runs at "
              f"{r['scan_step_frac_of_fma_peak']:.3f} of the plain-FMA rate: "
              f"{r['scan_step_chtok_per_s']:.4g} channel-token steps per second, the VALU ceiling of a single "
              f"pass of the scan over its inputs."]
    open(out_md, "w").write("\n".join(lines) + "\n")


def run_all_configs(log):
    """Time every workload once (GPU) beside the oracle on a sample.

    Prints one JSON line per workload.  Inputs come from synth (numpy, seeded);
    the seven hybrid-block layers use seeds 40..46.
    """
    import numpy as np
    import torch

    import oracle
    import synth
    import selective_state_space_11_amd as js

    dev = torch.device("cuda:0")

    def dio(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).to(dev)

    def timed(fn, reps):
        # untimed calls for at least 100 ms first: after the inputs are made on
        # the host the GPU has idled, and its clocks take a while to come up
        t_end = time.time() + 0.1
        while True:
            fn(); torch.cuda.synchronize()
            if time.time() >= t_end:
                break
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record(); torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def cpu_rate(inp, n_ch):
        d_inner = inp["x"].shape[2]
        chans = np.linspace(0, d_inner - 1, n_ch).astype(int)
        sub = synth.channel_slice(inp, chans)
        t0 = time.time()
        oracle.prefill(sub["x"], sub["delta"], sub["A"], sub["B"], sub["C"], sub["D"], sub["z"], sub["h0"])
        return inp["x"].shape[0] * inp["x"].shape[1] * n_ch / (time.time() - t0)

    def cpu_bwd_rate(inp, dy, dhT, n_ch):
        d_inner = inp["x"].shape[2]
        chans = np.linspace(0, d_inner - 1, n_ch).astype(int)
        sub = synth.channel_slice(inp, chans)
        dys = synth.widen(dy[:, :, chans])
        dhs = dhT[:, chans].astype(np.float64)
        t0 = time.time()
        oracle.backward(sub["x"], sub["delta"], sub["A"], sub["B"], sub["C"], sub["D"], sub["z"], dys, sub["h0"],
                        dhs)
        return inp["x"].shape[0] * inp["x"].shape[1] * n_ch / (time.time() - t0)

    def emit(name, chtok, ms, abytes, cpu, extra=None):
        rec = {"workload": name, "gpu_ms": round(ms, 4), "channel_tokens_per_s": chtok / (ms * 1e-3),
               "alg_GBps": round(abytes / (ms * 1e-3) / 1e9, 1),
               "hbm_frac": round(abytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "cpu_oracle_channel_tokens_per_s": cpu, "cpu_threads": oracle.num_threads()}
        rec.update(extra or {})
        print(json.dumps(rec), flush=True)

    prefill_cases = [("jamba prefill batch 2 x 4096", 2, 4096, 1), ("64K context batch 1", 1, 65536, 2),
                     ("256K context batch 1 (single call)", 1, 262144, 2)]
    for name, batch, L, seed in prefill_cases:
        inp = synth.prefill_inputs(batch, L, 8192, seed=seed)
        x, dl, z, B, C = (dio(inp[k]) for k in ("x", "delta", "z", "B", "C"))
        A, D = dio(inp["A"]), dio(inp["D"])
        y = torch.empty_like(x)
        hT = torch.empty(batch, 8192, 16, device=dev)
        ws = torch.empty(max(1, js.workspace_size(batch, L, 8192)), dtype=torch.uint8, device=dev)
        ms = timed(lambda: js.prefill(x, dl, A, B, C, D, z, None, y=y, hT=hT, workspace=ws), 10)
        emit(name, batch * L * 8192, ms, alg_bytes_prefill(batch, L, 8192), cpu_rate(inp, 256),
             {"plan": js.plan(batch, L, 8192)})
        if L <= 65536:
            dy_np, dhT_np = synth.output_grads(batch, L, 8192, seed=seed)
            dy, dhT = dio(dy_np), dio(dhT_np)
            bws = torch.empty(js.backward_workspace_size(batch, L, 8192), dtype=torch.uint8, device=dev)
            g = js.backward(x, dl, A, B, C, D, z, dy, None, dhT, workspace=bws)
            bms = timed(lambda: js.backward(x, dl, A, B, C, D, z, dy, None, dhT, workspace=bws, out=g), 5)
            emit("backward of " + name, batch * L * 8192, bms, alg_bytes_prefill(batch, L, 8192) * 2,
                 cpu_bwd_rate(inp, dy_np, dhT_np, 64), {"over_forward": round(bms / ms, 3)})
            del dy_np
            del g, bws, dy
        if L == 262144:
            state = torch.zeros(1, 8192, 16, device=dev)
            ws2 = torch.empty(max(1, js.workspace_size(1, 4096, 8192)), dtype=torch.uint8, device=dev)

            def chained():
                state.zero_()
                for i in range(64):
                    sl = slice(i * 4096, (i + 1) * 4096)
                    js.prefill(x[:, sl], dl[:, sl], A, B[:, sl], C[:, sl], D, z[:, sl], state, y=y[:, sl],
                               hT=state, workspace=ws2)
            ms = timed(chained, 3)
            emit("256K context as 64 chained calls of 4096 tokens", L * 8192, ms,
                 alg_bytes_prefill(1, L, 8192) + 64 * 2 * 8192 * 64, None, {"plan": js.plan(1, 4096, 8192)})
        del x, dl, z, y, inp
        torch.cuda.empty_cache()

    # decode: 256 sequences, 1024 steps with per-step seeded inputs
    n_seq = 256
    st_np = synth.decode_state(n_seq, 8192, seed=3)
    st = dio(st_np)
    A_np, D_np, _ = synth.params(8192, seed=3)
    A, D = dio(A_np), dio(D_np)
    # the oracle's decode rate on 256 of the channels over the first 16 steps
    chans = np.linspace(0, 8191, 256).astype(int)
    toks = []
    for k in range(16):
        di = synth.decode_inputs(n_seq, 8192, seed=3, step=k)
        toks.append([synth.widen(di[n][..., chans]) if n in ("x", "delta", "z") else synth.widen(di[n])
                     for n in ("x", "delta", "z", "B", "C")])
    s64 = st_np[:, chans].astype(np.float64)
    A64, D64 = A_np[chans].astype(np.float64), D_np[chans].astype(np.float64)
    t0 = time.time()
    for (ox, od, oz, oB, oC) in toks:
        _, s64 = oracle.step(s64, ox, od, A64, oB, oC, D64, oz)
    cpu_dec = n_seq * len(chans) * len(toks) / (time.time() - t0)
    del toks, st_np
    steps = []
    for k in range(1024):
        di = synth.decode_inputs(n_seq, 8192, seed=3, step=k)
        steps.append(tuple(dio(di[n]) for n in ("x", "delta", "z", "B", "C")))
    yd = torch.empty(n_seq, 8192, dtype=torch.bfloat16, device=dev)

    def decode_run():
        for (dx, dd, dz, dB, dC) in steps:
            js.step_batch(st, dx, dd, A, dB, dC, D, dz, y=yd)
    ms = timed(decode_run, 2)
    emit("decode 256 sequences x 1024 steps", n_seq * 8192 * 1024, ms, 1024 * alg_bytes_step(n_seq, 8192), cpu_dec,
         {"us_per_step": round(ms * 1e3 / 1024, 2)})
    del steps

    # hybrid block: seven independent Mamba layers, batch 8 x 16384
    layers = []
    for l in range(7):
        inp = synth.prefill_inputs(8, 16384, 8192, seed=40 + l)
        layers.append(tuple(dio(inp[k]) for k in ("x", "delta", "z", "B", "C", "A", "D")))
        if l == 0:
            cpu = cpu_rate(inp, 64)
        del inp
    y = torch.empty_like(layers[0][0])
    hT = torch.empty(8, 8192, 16, device=dev)
    ws = torch.empty(max(1, js.workspace_size(8, 16384, 8192)), dtype=torch.uint8, device=dev)

    def block():
        for (x, dl, z, B, C, A, D) in layers:
            js.prefill(x, dl, A, B, C, D, z, None, y=y, hT=hT, workspace=ws)
    ms = timed(block, 3)
    emit("hybrid block: 7 layers of batch 8 x 16384", 7 * 8 * 16384 * 8192, ms,
         7 * alg_bytes_prefill(8, 16384, 8192), cpu, {"plan": js.plan(8, 16384, 8192)})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--L", type=int, default=65536)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--backward-steps", type=int, default=5, help="timed backward calls (0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB (read) to 1 GiB (write), --steps times, "
                         "to calibrate HBM byte counters")
    ap.add_argument("--all-configs", action="store_true",
                    help="time every workload (batch 2 x 4K, 64K, 256K single and chained, decode x1024, "
                         "7-layer hybrid block) with the oracle on a sample; one JSON line each")
    ap.add_argument("--valu-ceiling", action="store_true",
                    help="only measure the VALU rates of this GPU for the scan's instruction mixes "
                         "(libjscan_ubench.so); --out writes a summary")
    ap.add_argument("--summarize-trace", metavar="DB", help="write a kernel-trace summary (no GPU work)")
    ap.add_argument("--summarize-traffic", metavar="PMC_DIR", help="write the HBM traffic summary (no GPU work)")
    ap.add_argument("--summarize-counters", metavar="PMC_DIR",
                    help="write the SQ counter summary of the --pmc runs under PMC_DIR (no GPU work)")
    ap.add_argument("--trace-db", help="kernel-trace database giving the durations for --summarize-counters")
    ap.add_argument("--out", help="output file of a summary")
    ap.add_argument("--command", default="", help="the profiling command, recorded in a summary")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.command)
        return
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic, args.out, os.path.join(ROOT, "profiles", "traffic.json"),
                          args.command)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.out, args.command, args.trace_db)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: libjscan has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import selective_state_space_11_amd as js

    if not os.path.exists(js.LIB_PATH):
        from __graft_entry__ import build
        build()
    js.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)

    if args.all_configs:
        run_all_configs(log)
        return

    if args.valu_ceiling:
        run_valu_ceiling(args.out, args.command)
        return

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)      # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read_per_copy": src.numel() * 4,
                                               "bytes_written_per_copy": dst.numel() * 4,
                                               "copies": args.steps}}))
        return

    batch, L, d_inner = 1, args.L, 8192
    t_gen = time.time()
    inp = synth.prefill_inputs(batch, L, d_inner, seed=2, io=synth.IO_BF16)
    log(f"[bench] generated inputs in {time.time() - t_gen:.1f}s")

    def dio(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).to(dev)

    x, delta, z, B, C = (dio(inp[k]) for k in ("x", "delta", "z", "B", "C"))
    A = torch.from_numpy(inp["A"]).to(dev)
    D = torch.from_numpy(inp["D"]).to(dev)
    y = torch.empty_like(x)
    hT = torch.empty(batch, d_inner, D_STATE, dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, js.workspace_size(batch, L, d_inner)), dtype=torch.uint8, device=dev)
    K, chunks = js.plan(batch, L, d_inner)

    def step():
        js.prefill(x, delta, A, B, C, D, z, None, y=y, hT=hT, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done (plan: {K} waves per 64 channels, {chunks} chunks)")

    # whole-step timing
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # main scan kernel alone: events recorded by the library around its launch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        js.time_next_prefill(a, b)
        step()
    torch.cuda.synchronize()
    scan_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    log(f"[bench] step {ms_per_step:.4f} ms, main scan kernel {scan_ms:.4f} ms")

    # the device copy rate on this GPU (1 GiB read and 1 GiB written per copy),
    # the practical ceiling the HBM fractions are also quoted against
    csrc = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        cdst.copy_(csrc)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * csrc.numel() * 4 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del csrc, cdst
    log(f"[bench] device copy {copy_gbs:.0f} GB/s")

    chtok = batch * L * d_inner
    value = chtok / (ms_per_step * 1e-3)
    abytes = alg_bytes_prefill(batch, L, d_inner)
    hbm_gbs = abytes / (ms_per_step * 1e-3) / 1e9
    kern_tflops = chtok * SLOTS_PER_CHTOK * 2 / (scan_ms * 1e-3) / 1e12
    traffic = load_traffic("k_scan_64k")

    # decode: 256 sequences x 8192 channels, one token each, state in place
    n_seq = 256
    st = torch.from_numpy(synth.decode_state(n_seq, d_inner, seed=3)).to(dev)
    di = synth.decode_inputs(n_seq, d_inner, seed=3, step=0)
    dx, dd, dz, dB, dC = (dio(di[k]) for k in ("x", "delta", "z", "B", "C"))
    Ad, Dd, _ = synth.params(d_inner, seed=3)
    Ad, Dd = torch.from_numpy(Ad).to(dev), torch.from_numpy(Dd).to(dev)
    yd = torch.empty_like(dx)
    for _ in range(10):
        js.step_batch(st, dx, dd, Ad, dB, dC, Dd, dz, y=yd)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.decode_steps):
        js.step_batch(st, dx, dd, Ad, dB, dC, Dd, dz, y=yd)
    e1.record()
    torch.cuda.synchronize()
    us_step = e0.elapsed_time(e1) * 1e3 / args.decode_steps
    dec_bytes = alg_bytes_step(n_seq, d_inner)
    decode = {"workload": "decode step, 256 sequences x d_inner 8192, state in place",
              "us_per_step": round(us_step, 3),
              "channel_tokens_per_s": n_seq * d_inner / (us_step * 1e-6),
              "alg_GBps": round(dec_bytes / (us_step * 1e-6) / 1e9, 1),
              "hbm_frac": round(dec_bytes / (us_step * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
              "frac_of_measured_copy": round(dec_bytes / (us_step * 1e-6) / 1e9 / copy_gbs, 4),
              "note": "the 128 MiB state can stay resident in the 256 MB last-level cache"}
    log(f"[bench] decode {us_step:.2f} us/step")

    # one sequence per step (8192 channels, a launch-bound kernel): 64 eager
    # calls against the same 64 steps captured once in a HIP graph and replayed
    st1 = st[:1].clone()
    t1 = [v[:1].contiguous() for v in (dx, dd, dz, dB, dC)]
    y1 = torch.empty_like(t1[0])

    def steps64():
        for _ in range(64):
            js.step_batch(st1, t1[0], t1[1], Ad, t1[3], t1[4], Dd, t1[2], y=y1)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        steps64()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps64()
    for _ in range(3):
        steps64()
        graph.replay()
    torch.cuda.synchronize()
    e0.record()
    steps64()
    e1.record()
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / 64
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / 64
    decode["single_sequence"] = {"workload": "decode step of one sequence x d_inner 8192",
                                 "eager_us_per_step": round(eager_us, 3), "hip_graph_us_per_step": round(graph_us, 3)}
    del graph
    log(f"[bench] decode of one sequence {eager_us:.2f} us/step eager, {graph_us:.2f} us/step from a HIP graph")

    # the same prefill with the fused input prologue (conv width 4 + SiLU, softplus(delta + dt_bias))
    pro = synth.prologue_params(d_inner, 4, seed=2)
    cw, cb, cs, dtb = (torch.from_numpy(pro[k]).to(dev) for k in ("conv_weight", "conv_bias", "conv_state",
                                                                  "dt_bias"))
    cso = torch.empty_like(cs)

    def fused_step():
        js.prefill_fused(x, delta, A, B, C, D, z, None, y=y, hT=hT, workspace=ws, conv_weight=cw, conv_bias=cb,
                         conv_state_in=cs, conv_state_out=cso, dt_bias=dtb, softplus=True)
    for _ in range(2):
        fused_step()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        fused_step()
    e1.record()
    torch.cuda.synchronize()
    fused_ms = e0.elapsed_time(e1) / args.steps
    w_dt, w_B, w_C = (torch.from_numpy(w).to(dev) for w in synth.rms_weights(d_inner, seed=2))

    def rms_step():
        js.prefill_fused(x, delta, A, B, C, D, z, None, y=y, hT=hT, workspace=ws, conv_weight=cw, conv_bias=cb,
                         conv_state_in=cs, conv_state_out=cso, dt_bias=dtb, softplus=True,
                         rms=(w_dt, w_B, w_C, 1e-5))
    for _ in range(2):
        rms_step()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        rms_step()
    e1.record()
    torch.cuda.synchronize()
    rms_ms = e0.elapsed_time(e1) / args.steps
    fused = {"workload": "the same prefill with the input prologue fused (causal depthwise conv width 4 + SiLU "
                         "on x, softplus(delta + dt_bias))",
             "ms_per_step": round(fused_ms, 4), "channel_tokens_per_s": chtok / (fused_ms * 1e-3),
             "with_rmsnorm_ms_per_step": round(rms_ms, 4)}
    log(f"[bench] fused prologue prefill {fused_ms:.4f} ms, with RMSNorm of delta, B, C {rms_ms:.4f} ms")

    # the exponential-trapezoidal recurrence on the same inputs (lam ~ U(0,1), token before the first)
    lam_np, xp_np, Bp_np = synth.trap_inputs(batch, L, d_inner, seed=2)
    lam_t, xp_t, Bp_t = dio(lam_np), dio(xp_np), dio(Bp_np)
    del lam_np

    def trap_step():
        js.prefill_trap(x, delta, A, B, C, D, z, None, lam=lam_t, x_prev=xp_t, B_prev=Bp_t, y=y, hT=hT,
                        workspace=ws)
    for _ in range(2):
        trap_step()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        trap_step()
    e1.record()
    torch.cuda.synchronize()
    trap_ms = e0.elapsed_time(e1) / args.steps
    trap = {"workload": "the same prefill with the exponential-trapezoidal recurrence (lam per channel-token)",
            "ms_per_step": round(trap_ms, 4), "channel_tokens_per_s": chtok / (trap_ms * 1e-3)}
    log(f"[bench] trapezoidal prefill {trap_ms:.4f} ms")
    del lam_t

    # backward of the same prefill, output gradients dy ~ N(0,1), dhT ~ N(0,1)
    backward = None
    if args.backward_steps > 0:
        dy_np, dhT_np = synth.output_grads(batch, L, d_inner, seed=2)
        dy = dio(dy_np)
        del dy_np
        dhT = torch.from_numpy(dhT_np).to(dev)
        bws = torch.empty(js.backward_workspace_size(batch, L, d_inner), dtype=torch.uint8, device=dev)
        grads = js.backward(x, delta, A, B, C, D, z, dy, None, dhT, workspace=bws)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.backward_steps):
            js.backward(x, delta, A, B, C, D, z, dy, None, dhT, workspace=bws, out=grads)
        e1.record()
        torch.cuda.synchronize()
        bwd_ms = e0.elapsed_time(e1) / args.backward_steps
        # the same gradients from the chunk starting states the prefill left in
        # its workspace (jscan_backward_saved)
        step()
        js.backward(x, delta, A, B, C, D, z, dy, None, dhT, workspace=bws, prefill_workspace=ws, out=grads)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.backward_steps):
            js.backward(x, delta, A, B, C, D, z, dy, None, dhT, workspace=bws, prefill_workspace=ws, out=grads)
        e1.record()
        torch.cuda.synchronize()
        saved_ms = e0.elapsed_time(e1) / args.backward_steps
        backward = {"workload": "gradients of the same prefill (dx, ddelta, dz, dA, dB, dC, dD, dh0)",
                    "ms_per_step": round(bwd_ms, 4), "channel_tokens_per_s": chtok / (bwd_ms * 1e-3),
                    "over_forward": round(bwd_ms / ms_per_step, 3),
                    "with_saved_chunk_states_ms_per_step": round(saved_ms, 4),
                    "workspace_GiB": round(bws.numel() / 2 ** 30, 2)}
        log(f"[bench] backward {bwd_ms:.4f} ms, from the prefill's saved chunk states {saved_ms:.4f} ms")
        del grads, bws, dy

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        n_ch = 4096
        chans = np.arange(0, d_inner, d_inner // n_ch)[:n_ch]
        sub = synth.channel_slice(inp, chans)
        t0 = time.time()
        oracle.prefill(sub["x"], sub["delta"], sub["A"], sub["B"], sub["C"], sub["D"], sub["z"], None)
        dt = time.time() - t0
        cpu = {"value": n_ch * L / dt, "unit": "channel-tokens/s", "cores": oracle.num_threads(),
               "kind": "oracle",
               "sample": f"{n_ch} of the {d_inner} channels (every {d_inner // n_ch}th) over all {L} tokens "
                         f"of the same inputs; fp64 C oracle, {dt:.2f} s wall on {oracle.num_threads()} threads"}
        log(f"[bench] cpu oracle {cpu['value']:.3e} ch-tok/s on {cpu['cores']} threads")

    out = {
        "metric": "channel-tokens/s and % HBM roofline, d_inner=8192 N=16 @ 64K ctx",
        "value": value,
        "unit": "channel-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"selective-scan prefill, batch {batch}, L {L}, d_inner {d_inner}, "
                               f"d_state 16, bf16 I/O, fp32 state",
                   "batch": batch, "seq_len": L, "d_inner": d_inner, "d_state": D_STATE,
                   "plan": {"waves_per_64_channels": K, "chunks": chunks}},
        "hbm_roofline": {"achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(hbm_gbs / HBM_PEAK_GBS, 4), "alg_bytes_per_step": abytes,
                         "measured_copy_GBps": round(copy_gbs, 1),
                         "frac_of_measured_copy": round(hbm_gbs / copy_gbs, 4)},
        "roofline": {"bound": "alu", "kernel": "k_scan (main scan)",
                     "achieved": round(kern_tflops, 2), "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kern_tflops / VALU_PEAK_TFLOPS, 4),
                     "traffic": traffic, "kernel_ms": round(scan_ms, 4),
                     "work": f"{SLOTS_PER_CHTOK} fp32 VALU slots (x2 flop) per channel-token, "
                             f"{chtok} channel-tokens per launch"},
        "decode": decode,
        "prefill_fused_prologue": fused,
        "prefill_trapezoidal": trap,
        "backward": backward,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
