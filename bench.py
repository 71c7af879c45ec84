#!/usr/bin/env python3
"""Benchmark: the selective-scan prefill at the Jamba shape with a 64K context.

One step = one jscan_prefill call over batch 1, L = 65536 tokens, d_inner 8192,
d_state 16, bf16 I/O, fp32 state and arithmetic, inputs resident in HBM.
`value` is channel-tokens/s (batch * L * d_inner per second of the whole call).

The `roofline` object is the HBM roofline: the call's algorithmic bytes (x,
delta, z read and y written, 2 B each, the B and C rows, A, D and the final
state; re-reads by the chunked plan do not count) divided by the average
duration of the dominant kernel (pass 1 of the chunked scan, timed with HIP
events the library records on its launch stream during the timed steps),
against the MI355X's 8 TB/s.  Beside it: the same bytes over the whole call,
and over the device-copy rate measured on this GPU.  `valu` holds the ceiling
the chip's vector ALU puts on the same work, measured by libjscan_ubench's
scan-step kernel during the run.  `traffic` (HBM bytes per launch from
rocprofv3's FETCH_SIZE / WRITE_SIZE counters) is read from
profiles/traffic.json when those counters were taken on the current kernel
sources, else null.

Further legs (each printed inside the same JSON line): the decode step of 256
sequences at HBM (seven 128 MiB state pools stepped in turn with fresh
inputs; also with the fused prologue and with the trapezoidal recurrence)
and with its state resident in the last-level cache, the prefill with
the fused input prologue, with RMSNorm, with the exponential-trapezoidal
recurrence, the backward scan, and the fp64 CPU oracle on a bounded sample.

    python bench.py [--gpus 1] [--steps 20] [--warmup 20]
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
D_STATE = 16
N_CU = 256

# The kernels a plain bf16 prefill launches (names as rocprofv3 prints them,
# without the namespace): pass 1 (the dominant kernel), the carry combine and
# pass 2; and the decode step.
PASS1 = "k_scan<unsigned short, false, false, false, false, 1>"
PASS2 = "k_scan<unsigned short, false, false, false, false, 2>"
COMBINE = "k_combine<unsigned short>"
STEP = "k_step<unsigned short, false, false, false, false>"
PREFILL_GRID = (8192, 32, 1)        # pass 1's grid at 1 x 65536 x 8192 (work-items)
PASS2_GRID = (8192, 31, 1)          # pass 2's (the chunks after the first)
COMBINE_GRID = (131072, 1, 1)       # the combine's (d_inner x 16 lanes)
STEP_GRID = (256 * 8192 * 4, 1, 1)  # the 256-sequence decode step


def alg_bytes_prefill(batch, L, d_inner, io_bytes=2, h0=False, hT=True):
    tok = batch * L * d_inner * io_bytes * 4           # x, delta, z in; y out
    rows = batch * L * D_STATE * io_bytes * 2          # B, C
    params = d_inner * D_STATE * 4 + d_inner * 4       # A, D
    state = batch * d_inner * D_STATE * 4 * ((1 if h0 else 0) + (1 if hT else 0))
    return tok + rows + params + state


def alg_bytes_step(n_seq, d_inner, io_bytes=2):
    return (2 * n_seq * d_inner * D_STATE * 4 + n_seq * d_inner * io_bytes * 4
            + n_seq * D_STATE * io_bytes * 2 + d_inner * D_STATE * 4 + d_inner * 4)


def alg_bytes_step_fused(n_seq, d_inner, width=4, io_bytes=2):
    """The decode step with the prologue: the conv history (width - 1 fp32 per
    sequence-channel) read and written, the conv weights and bias, dt_bias."""
    return (alg_bytes_step(n_seq, d_inner, io_bytes) + 2 * n_seq * d_inner * (width - 1) * 4
            + d_inner * (width + 2) * 4)


def alg_bytes_step_trap(n_seq, d_inner, io_bytes=2):
    """The trapezoidal decode step: lam and the previous token's x and B as well."""
    return alg_bytes_step(n_seq, d_inner, io_bytes) + 2 * n_seq * d_inner * io_bytes + n_seq * D_STATE * io_bytes


def _code_only(text):
    """Source text without comments and with whitespace collapsed (a comment
    does not change a kernel)."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif text[i] in "\"'":                     # string and character literals pass through
            q, j = text[i], i + 1
            while j < n and text[j] != q:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return " ".join("".join(out).split())


def source_digest():
    """Digest of the code (comments aside) the forward kernels and their plan
    are compiled from."""
    h = hashlib.sha256()
    for f in ("jscan.hip", "common.h", "host.h"):
        text = open(os.path.join(ROOT, "selective_state_space_11_amd", "csrc", f), encoding="utf-8").read()
        h.update(_code_only(text).encode())
    return h.hexdigest()[:16]


def load_traffic(tag):
    """Counter-derived HBM bytes for `tag` from profiles/traffic.json, if they
    were taken on the current kernel sources; else None."""
    try:
        data = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    except (OSError, ValueError):
        return None
    ent = data.get(tag)
    if not ent or ent.get("source_sha") != source_digest():
        return None
    return ent


def cpu_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return model, avail


# ----------------------------------------------------------- profile summaries
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


def _grid(gx, gy, gz):
    return f"{gx}x{gy}x{gz}"


def summarize_trace(db, out_md, command):
    """Per-kernel duration table (kernel and grid in work-items) from a
    rocprofv3 --kernel-trace database."""
    rows = _db_rows(db, "select name, grid_x, grid_y, grid_z, duration from kernels order by start")
    stats = {}
    for name, gx, gy, gz, dur in rows:
        stats.setdefault((_short(name), _grid(gx, gy, gz)), []).append(dur / 1000.0)
    lines = [f"# Kernel trace: {os.path.basename(out_md)[:-3]}", "",
             "Command (on the MI355X box, from the repository root):", "", "```", command, "```", "",
             "| kernel | grid (work-items) | calls | average (us) | median (us) | min (us) | max (us) | total (us) |",
             "|---|---|---|---|---|---|---|---|"]
    for (k, g), v in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        med = sorted(v)[len(v) // 2]
        lines.append(f"| {k} | {g} | {len(v)} | {sum(v) / len(v):.1f} | {med:.1f} | {min(v):.1f} | "
                     f"{max(v):.1f} | {sum(v):.1f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")
    return stats


def _counter_medians(db, counter):
    """{(kernel, grid): median bytes per dispatch} of a rocprofv3 --pmc run of
    one counter reported in KiB (summed over its instances per dispatch)."""
    rows = _db_rows(db, "select k.name, k.grid_x, k.grid_y, k.grid_z, p.dispatch_id, p.counter_value "
                        "from pmc_events p join kernels k on k.dispatch_id = p.dispatch_id "
                        f"where p.counter_name = '{counter}'")
    per = {}
    for name, gx, gy, gz, disp, val in rows:
        d = per.setdefault((_short(name), _grid(gx, gy, gz)), {})
        d[disp] = d.get(disp, 0.0) + val
    return {k: sorted(v.values())[len(v) // 2] * 1024.0 for k, v in per.items()}


def summarize_traffic(pmc_dir, out_md, out_json, command):
    """HBM bytes per dispatch from FETCH_SIZE and WRITE_SIZE (two --pmc runs of
    the bench, in sub-folders fetch/ and write/), each scaled by what the
    counter reads for the bench's own 1 GiB -> 1 GiB device copy."""
    fetch = _counter_medians(os.path.join(pmc_dir, "fetch", "run_results.db"), "FETCH_SIZE")
    write = _counter_medians(os.path.join(pmc_dir, "write", "run_results.db"), "WRITE_SIZE")
    copies_f = {k: v for k, v in fetch.items() if k[0] == "__amd_rocclr_copyBuffer"}
    copies_w = {k: v for k, v in write.items() if k[0] == "__amd_rocclr_copyBuffer"}
    ck = max(copies_f, key=copies_f.get)             # the largest copy: the 1 GiB one
    f_scale, w_scale = (1 << 30) / copies_f[ck], (1 << 30) / copies_w[ck]
    lines = ["# HBM traffic per dispatch (rocprofv3 counters over the default bench run)", "",
             "Commands (on the MI355X box, from the repository root):", "", "```", command, "```", "",
             f"Calibration: the bench's 1 GiB -> 1 GiB device copy (grid {ck[1]}) reads FETCH_SIZE = "
             f"{copies_f[ck] / 1024:.0f} KiB and WRITE_SIZE = {copies_w[ck] / 1024:.0f} KiB, so FETCH_SIZE is "
             f"scaled by {f_scale:.3f} and WRITE_SIZE by {w_scale:.3f}. Medians over the dispatches of each "
             "kernel and grid.", "",
             "| kernel | grid (work-items) | read (MB) | written (MB) | total (MB) |", "|---|---|---|---|---|"]
    res = {}
    for k in sorted(fetch, key=lambda k: -fetch[k]):
        if k[0].startswith("__amd") or k[0].startswith("at::") or k[0].startswith("void at::"):
            continue
        r, w = fetch[k] * f_scale, write.get(k, 0.0) * w_scale
        res[k] = (r, w)
        lines.append(f"| {k[0]} | {k[1]} | {r / 1e6:.1f} | {w / 1e6:.1f} | {(r + w) / 1e6:.1f} |")

    def find(name, grid=None):
        cands = [k for k in res if k[0] == name and (grid is None or k[1] == _grid(*grid))]
        return sum(res[cands[0]]) if cands else None

    p1 = find(PASS1, PREFILL_GRID)
    p2 = find(PASS2, PASS2_GRID)
    cmb = find(COMBINE, COMBINE_GRID)
    step = find(STEP, STEP_GRID)
    a_pre, a_step = alg_bytes_prefill(1, 65536, 8192), alg_bytes_step(256, 8192)
    data = {"source_sha": source_digest(), "fetch_scale": f_scale, "write_scale": w_scale,
            "prefill_64k": {"source_sha": source_digest(), "kernel": PASS1, "hbm_bytes_per_launch": p1,
                            "whole_call_bytes": (p1 + p2 + cmb) if None not in (p1, p2, cmb) else None,
                            "alg_bytes": a_pre},
            "decode_256": {"source_sha": source_digest(), "kernel": STEP, "hbm_bytes_per_launch": step,
                           "alg_bytes": a_step}}
    lines += ["", "Per call of the plain 64K prefill (batch 1 x 65536 x 8192, bf16): algorithmic "
              f"{a_pre / 1e6:.1f} MB."]
    if p1 is not None:
        lines.append(f"- pass 1 ({PASS1}): {p1 / 1e6:.1f} MB, {p1 / a_pre:.3f} x algorithmic;")
    if data["prefill_64k"]["whole_call_bytes"]:
        wc = data["prefill_64k"]["whole_call_bytes"]
        lines.append(f"- whole call (pass 1 + combine + pass 2): {wc / 1e6:.1f} MB, {wc / a_pre:.3f} x algorithmic.")
    if step is not None:
        lines.append(f"\nDecode step of 256 sequences ({STEP}, grid {_grid(*STEP_GRID)}): {step / 1e6:.1f} MB per "
                     f"step against {a_step / 1e6:.1f} MB algorithmic ({step / a_step:.3f} x).")
    open(out_md, "w").write("\n".join(lines) + "\n")
    json.dump(data, open(out_json, "w"), indent=1)
    return res


def _valu_rates():
    """Measured plain-FMA lane-instruction rate and exp2 cost (in FMA slots)
    from profiles/valu_ceiling.json, or None."""
    try:
        v = json.load(open(os.path.join(ROOT, "profiles", "valu_ceiling.json")))
        return v["fma_lane_instr_per_s"], v["exp_slots"]
    except (OSError, ValueError, KeyError):
        return None


def summarize_counters(pmc_dir, out_md, command, trace_db=None):
    """Per-kernel medians of every SQ_/GRBM_ counter found in the rocprofv3
    --pmc runs under pmc_dir (one sub-folder per run), with the VALU issue
    figures derived from them.

    A VALU wave instruction covers 64 lanes.  A transcendental (exp2, log2,
    rcp) takes the issue time of `exp_slots` plain fp32 instructions, both as
    measured on this GPU (profiles/valu_ceiling.json), so the fp32 slot count
    is SQ_INSTS_VALU + (exp_slots - 1) * SQ_INSTS_VALU_TRANS_F32."""
    import glob
    rates = _valu_rates()
    per = {}
    for db in sorted(glob.glob(os.path.join(pmc_dir, "*", "run_results.db"))):
        rows = _db_rows(db, "select k.name, k.grid_x, k.grid_y, k.grid_z, p.dispatch_id, p.counter_name, "
                            "p.counter_value from pmc_events p join kernels k on k.dispatch_id = p.dispatch_id")
        acc = {}
        for name, gx, gy, gz, disp, cname, val in rows:
            key = ((_short(name), _grid(gx, gy, gz)), cname)
            acc.setdefault(key, {}).setdefault(disp, 0.0)
            acc[key][disp] += val
        for (k, c), v in acc.items():
            vals = sorted(v.values())
            per.setdefault(k, {})[c] = vals[len(vals) // 2]
    durs = {}
    if trace_db:
        for name, gx, gy, gz, dur in _db_rows(trace_db, "select name, grid_x, grid_y, grid_z, duration from kernels"):
            durs.setdefault((_short(name), _grid(gx, gy, gz)), []).append(dur / 1e9)
    counters = sorted({c for v in per.values() for c in v})
    note = ("`fp32 slots` = SQ_INSTS_VALU + (e - 1) x SQ_INSTS_VALU_TRANS_F32 in wave instructions of 64 lanes, "
            "e the measured cost of one transcendental in plain-FMA issue slots. `VALU issue` = fp32 slots x 64 / "
            "(median kernel-trace duration x the measured plain-FMA rate): the fraction of the chip's plain fp32 "
            "issue rate the kernel kept busy (trace durations include the profiler's own overhead).")
    if rates:
        note += f" Here e = {rates[1]:.2f} and the rate is {rates[0]:.4g} lane-instructions/s."
    lines = ["# SQ counters per dispatch (rocprofv3 --pmc, median over dispatches)", "",
             "Commands (on the MI355X box, from the repository root):", "", "```", command, "```", "", note, "",
             "| kernel | grid | " + " | ".join(counters) + " | fp32 slots | VALU issue |",
             "|---|---|" + "---|" * (len(counters) + 2)]
    order = sorted(per, key=lambda k: -per[k].get("SQ_INSTS_VALU", 0.0))
    for k in order:
        if k[0].startswith("__amd") or "at::" in k[0]:
            continue
        v = per[k]
        e = rates[1] if rates else 2.0
        slots = v.get("SQ_INSTS_VALU", 0.0) + (e - 1) * v.get("SQ_INSTS_VALU_TRANS_F32", 0.0)
        busy = ""
        if rates and k in durs and slots and "SQ_INSTS_VALU_TRANS_F32" in v:
            d = sorted(durs[k])[len(durs[k]) // 2]
            busy = f"{slots * 64 / (d * rates[0]):.3f}"
        cells = [f"{v[c]:.4g}" if c in v else "" for c in counters]
        lines.append(f"| {k[0]} | {k[1]} | " + " | ".join(cells) + f" | {slots:.4g} | {busy} |")
    open(out_md, "w").write("\n".join(lines) + "\n")
    return per


# ------------------------------------------------------------- VALU ceiling
UBENCH_KINDS = {0: "fp32 FMA", 1: "exp2 (v_exp_f32)", 2: "1 exp2 + 4 independent FMA",
                3: "scan token step (16 x: mul, exp2, mul, FMA, FMA)"}
SCAN_STEP_INSTR = 5 * 16 + 3        # VALU instructions of one ubench scan token step


def _ubench():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "selective_state_space_11_amd", "libjscan_ubench.so"))
    d = ctypes.c_double
    lib.jscan_ubench_valu.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int] + [ctypes.POINTER(d)] * 5
    lib.jscan_ubench_valu.restype = ctypes.c_int

    def run(kind, waves, iters):
        out = [d() for _ in range(5)]
        rc = lib.jscan_ubench_valu(kind, waves, iters, *[ctypes.byref(o) for o in out])
        if rc != 0:
            raise RuntimeError(f"jscan_ubench_valu(kind {kind}) failed with {rc}")
        return tuple(o.value for o in out)      # seconds, lane instr, trans lane instr, clock MHz, wall MHz
    return run


def scan_step_ceiling():
    """Channel-token steps per second of the ubench scan-step kernel (8 waves
    per SIMD): the VALU ceiling of one pass of the scan's arithmetic."""
    run = _ubench()
    sec, lane, _, clk, _ = run(3, N_CU * 4 * 8, 2000)
    return lane / sec / SCAN_STEP_INSTR, clk


def valu_ceiling(waves_per_simd=(1, 2, 4, 8)):
    """Measured VALU rates of this GPU (libjscan_ubench.so), per CU per shader
    clock.  Returns a dict; the plain-FMA rate is the chip's fp32 issue peak,
    the scan-step rate the ceiling of the scan's instruction mix."""
    run = _ubench()
    iters = {0: 20000, 1: 5000, 2: 20000, 3: 5000}
    rows = []
    for kind in (0, 1, 2, 3):
        for wps in (waves_per_simd if kind == 0 else (8,)):
            waves = N_CU * 4 * wps
            it = max(1, iters[kind] * 8 // wps)
            sec, lane, trans, clk, wall = run(kind, waves, it)
            rate = lane / sec
            rows.append({"kind": UBENCH_KINDS[kind], "waves_per_simd": wps, "seconds": sec,
                         "lane_instr_per_s": rate, "trans_lane_instr_per_s": trans / sec,
                         "clock_mhz": round(clk, 1),
                         "lane_instr_per_cu_per_clock": rate / (N_CU * clk * 1e6) if clk else None})
    fma = max(r["lane_instr_per_s"] for r in rows if r["kind"] == UBENCH_KINDS[0])
    exp = next(r for r in rows if r["kind"] == UBENCH_KINDS[1])["lane_instr_per_s"]
    mix = next(r for r in rows if r["kind"] == UBENCH_KINDS[2])
    scan = next(r for r in rows if r["kind"] == UBENCH_KINDS[3])
    # a transcendental's cost in plain-FMA issue slots, and whether it overlaps FMAs:
    # group = 1 exp + 4 FMA; serial cost = 4 + exp_slots, parallel = max(4, exp_slots)
    exp_slots = fma / exp
    group_slots = 5 * fma / mix["lane_instr_per_s"]
    scan_slots_model = SCAN_STEP_INSTR - 16 + 16 * exp_slots
    scan_slot_rate = scan["lane_instr_per_s"] / SCAN_STEP_INSTR * scan_slots_model / fma
    clk = max(r["clock_mhz"] for r in rows)
    return {"rows": rows, "fma_lane_instr_per_s": fma, "exp_slots": exp_slots,
            "fma_lanes_per_cu_per_clock": fma / (N_CU * clk * 1e6),
            "fp32_tflops_plain": 2 * fma / 1e12,
            "exp_plus_4fma_group_slots": group_slots, "scan_step_slots_per_chtok": scan_slots_model,
            "scan_step_frac_of_fma_peak": scan_slot_rate,
            "scan_step_chtok_per_s": scan["lane_instr_per_s"] / SCAN_STEP_INSTR}


def run_valu_ceiling(out_md, command):
    r = valu_ceiling()
    print(json.dumps(r), flush=True)
    if not out_md:
        return
    json.dump({k: v for k, v in r.items() if k != "rows"}, open(out_md[:-3] + ".json", "w"), indent=1)
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
    lines += ["", f"- plain fp32 FMA: {r['fma_lanes_per_cu_per_clock']:.1f} lanes per CU per clock, "
              f"{r['fp32_tflops_plain']:.1f} TFLOP/s (FMA = 2 flop). The vendor's 157.3 TFLOP/s counts 128 lanes per "
              "CU per clock, the packed (v_pk_*) fp32 forms this library is built without;",
              f"- one v_exp_f32 costs {r['exp_slots']:.2f} plain-FMA issue slots;",
              f"- a group of 1 exp2 + 4 independent FMAs costs {r['exp_plus_4fma_group_slots']:.2f} slots "
              f"(4 + {r['exp_slots']:.2f} = {4 + r['exp_slots']:.2f} if they do not overlap, "
              f"{max(4, r['exp_slots']):.2f} if they do);",
              f"- the scan's token step (16 states) costs {r['scan_step_slots_per_chtok']:.1f} slots and runs at "
              f"{r['scan_step_frac_of_fma_peak']:.3f} of the plain-FMA rate: "
              f"{r['scan_step_chtok_per_s']:.4g} channel-token steps per second, the VALU ceiling of a single "
              f"pass of the scan over its inputs ({alg_bytes_prefill(1, 65536, 8192) / (65536 * 8192) * r['scan_step_chtok_per_s'] / 1e9:.0f} GB/s of "
              "algorithmic prefill bytes, "
              f"{alg_bytes_prefill(1, 65536, 8192) / (65536 * 8192) * r['scan_step_chtok_per_s'] / 1e9 / HBM_PEAK_GBS:.3f} "
              "of the HBM roofline)."]
    open(out_md, "w").write("\n".join(lines) + "\n")


# ------------------------------------------------------------ timing helpers
def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _timed(torch, fn, reps, warm_s=0.1):
    """Average ms of `reps` back-to-back calls after at least warm_s seconds
    of untimed calls (the GPU's clocks come up after an idle host phase)."""
    t_end = time.time() + warm_s
    while True:
        fn()
        torch.cuda.synchronize()
        if time.time() >= t_end:
            break
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


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
    model, avail = cpu_info()

    def dio(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).to(dev)

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
               "cpu_oracle_channel_tokens_per_s": cpu, "cpu_threads": oracle.num_threads(),
               "cpu_model": model, "cpu_available_cores": avail}
        rec.update(extra or {})
        print(json.dumps(rec), flush=True)

    timed = lambda fn, reps: _timed(torch, fn, reps)
    prefill_cases = [("jamba prefill batch 2 x 4096", 2, 4096, 1), ("64K context batch 1", 1, 65536, 2),
                     ("256K context batch 1 (single call)", 1, 262144, 2)]
    for name, batch, L, seed in prefill_cases:
        log(f"[all-configs] generating {name}")
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

    # decode: 256 sequences, 1024 steps with per-step seeded inputs (32
    # input sets in turn over seven 128 MiB state pools, as in the default
    # run), and the oracle's decode rate on 256 channels of every sequence
    # over the first 16 steps
    n_seq = 256
    st_np = synth.decode_state(n_seq, 8192, seed=3)
    A_np, D_np, _ = synth.params(8192, seed=3)
    chans = np.linspace(0, 8191, 256).astype(int)
    s64 = st_np[:, chans].astype(np.float64)
    A64, D64 = A_np[chans].astype(np.float64), D_np[chans].astype(np.float64)
    toks = []
    for k in range(16):
        di = synth.decode_inputs(n_seq, 8192, seed=3, step=k)
        toks.append([synth.widen(di[n][..., chans]) if n in ("x", "delta", "z") else synth.widen(di[n])
                     for n in ("x", "delta", "z", "B", "C")])
    t0 = time.time()
    for (ox, od, oz, oB, oC) in toks:
        _, s64 = oracle.step(s64, ox, od, A64, oB, oC, D64, oz)
    cpu_dec = n_seq * len(chans) * len(toks) / (time.time() - t0)
    del toks, st_np
    csrc = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    cdst = torch.empty_like(csrc)
    copy_gbs = 2 * csrc.numel() * 4 / (_timed(torch, lambda: cdst.copy_(csrc), 10) * 1e-3) / 1e9
    del csrc, cdst
    dec = bench_decode(torch, js, synth, dio, dev, copy_gbs, log)
    emit("decode 256 sequences x 1024 steps (fresh inputs, seven 128 MiB state pools)", n_seq * 8192 * 1024,
         dec["us_per_step"] * 1024e-3, 1024 * alg_bytes_step(n_seq, 8192), cpu_dec,
         {"us_per_step": dec["us_per_step"], "fused_prologue_us_per_step": dec["fused_prologue"]["us_per_step"],
          "trapezoidal_us_per_step": dec["trapezoidal"]["us_per_step"],
          "cache_resident_128_seq_us_per_step": dec["cache_resident"]["us_per_step"]})

    # hybrid block: seven independent Mamba layers, batch 8 x 16384
    layers = []
    for l in range(7):
        log(f"[all-configs] generating hybrid-block layer {l}")
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


# -------------------------------------------------------------------- legs
def bench_decode(torch, js, synth, dio, dev, copy_gbs, log, n_pools=7, n_sets=32, steps=1024):
    """The decode step of 256 sequences x d_inner 8192 (state updated in
    place).  At HBM: seven 128 MiB state pools (the seven Mamba layers of a
    block, 896 MiB) stepped in turn, step k with fresh inputs (set k % 32 of
    32 seeded sets, 12 MiB each): neither fits the 256 MB last-level cache.
    Also one pool with one input set replayed (cache-resident), and one
    sequence per step eagerly and from a HIP graph."""
    n_seq, d_inner = 256, 8192
    t0 = time.time()
    pools = [dio(synth.decode_state(n_seq, d_inner, seed=3 + l)) for l in range(n_pools)]
    sets = []
    for k in range(n_sets):
        di = synth.decode_inputs(n_seq, d_inner, seed=3, step=k)
        sets.append(tuple(dio(di[n]) for n in ("x", "delta", "z", "B", "C")))
    Ad, Dd, _ = synth.params(d_inner, seed=3)
    Ad, Dd = torch.from_numpy(Ad).to(dev), torch.from_numpy(Dd).to(dev)
    yd = torch.empty(n_seq, d_inner, dtype=torch.bfloat16, device=dev)
    log(f"[bench] decode inputs in {time.time() - t0:.1f}s")

    def hbm_run():
        for k in range(steps):
            dx, dd, dz, dB, dC = sets[k % n_sets]
            js.step_batch(pools[k % n_pools], dx, dd, Ad, dB, dC, Dd, dz, y=yd)
    ms = _timed(torch, hbm_run, 1, warm_s=0.0)         # one untimed pass of all steps first
    us_step = ms * 1e3 / steps
    abytes = alg_bytes_step(n_seq, d_inner)
    gbs = abytes / (us_step * 1e-6) / 1e9
    traffic = load_traffic("decode_256")
    decode = {"workload": f"decode step, {n_seq} sequences x d_inner {d_inner}, state in place; {n_pools} state "
                          f"pools of 128 MiB stepped in turn, fresh inputs every step ({n_sets} seeded sets), "
                          f"{steps} steps",
              "us_per_step": round(us_step, 3), "channel_tokens_per_s": n_seq * d_inner / (us_step * 1e-6),
              "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(gbs / HBM_PEAK_GBS, 4), "alg_bytes_per_step": abytes,
                           "frac_of_measured_copy": round(gbs / copy_gbs, 4),
                           "traffic": traffic["hbm_bytes_per_launch"] if traffic else None}}
    log(f"[bench] decode at HBM {us_step:.2f} us/step ({gbs:.0f} GB/s)")

    # The fused step (conv width 4 + SiLU with each layer's own conv history,
    # softplus(delta + dt_bias)) and the trapezoidal step (lam per
    # sequence-channel, the previous step's x and B), at HBM like the above.
    pro = synth.prologue_params(d_inner, 4, seed=3, batch=n_seq)
    cw, cb, dtb = (torch.from_numpy(pro[k]).to(dev) for k in ("conv_weight", "conv_bias", "dt_bias"))
    hists = [torch.from_numpy(pro["conv_state"]).to(dev).clone() for _ in range(n_pools)]

    def fused_run():
        for k in range(steps):
            dx, dd, dz, dB, dC = sets[k % n_sets]
            js.step_batch_fused(pools[k % n_pools], dx, dd, Ad, dB, dC, Dd, dz, conv_weight=cw, conv_bias=cb,
                                conv_state=hists[k % n_pools], dt_bias=dtb, softplus=True, y=yd)
    us_fused = _timed(torch, fused_run, 1, warm_s=0.0) * 1e3 / steps
    lam = dio(synth.trap_inputs(n_seq, 1, d_inner, seed=3)[0][:, 0, :])

    def trap_run():
        for k in range(steps):
            dx, dd, dz, dB, dC = sets[k % n_sets]
            px, _, _, pB, _ = sets[(k - 1) % n_sets]
            js.step_batch_trap(pools[k % n_pools], dx, dd, Ad, dB, dC, Dd, dz, lam=lam, x_prev=px, B_prev=pB, y=yd)
    us_trap = _timed(torch, trap_run, 1, warm_s=0.0) * 1e3 / steps
    fb, tb = alg_bytes_step_fused(n_seq, d_inner), alg_bytes_step_trap(n_seq, d_inner)
    decode["fused_prologue"] = {"workload": "the same steps with conv width 4 + SiLU (each pool with its own conv "
                                            "history, updated in place) and softplus(delta + dt_bias)",
                                "us_per_step": round(us_fused, 3),
                                "alg_GBps": round(fb / (us_fused * 1e-6) / 1e9, 1),
                                "frac_of_hbm_peak": round(fb / (us_fused * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    decode["trapezoidal"] = {"workload": "the same steps with the exponential-trapezoidal recurrence",
                             "us_per_step": round(us_trap, 3),
                             "alg_GBps": round(tb / (us_trap * 1e-6) / 1e9, 1),
                             "frac_of_hbm_peak": round(tb / (us_trap * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del hists, lam
    log(f"[bench] decode at HBM: fused prologue {us_fused:.2f} us/step, trapezoidal {us_trap:.2f} us/step")

    # cache-resident: 128 of the sequences (a 64 MiB state) with one input set
    # replayed, so that state and inputs stay in the 256 MB last-level cache
    # (a grid of its own in a kernel trace)
    h = n_seq // 2
    st = pools[0][:h].clone()
    dx, dd, dz, dB, dC = (v[:h].contiguous() for v in sets[0])
    yh = yd[:h].clone()
    ms = _timed(torch, lambda: js.step_batch(st, dx, dd, Ad, dB, dC, Dd, dz, y=yh), 200)
    gbs_llc = alg_bytes_step(h, d_inner) / (ms * 1e-3) / 1e9
    decode["cache_resident"] = {"workload": f"the step of {h} sequences (a 64 MiB state) with one input set "
                                            "replayed: state and inputs stay in the 256 MB last-level cache",
                                "us_per_step": round(ms * 1e3, 3), "alg_GBps": round(gbs_llc, 1),
                                "frac_of_hbm_peak": round(gbs_llc / HBM_PEAK_GBS, 4)}
    log(f"[bench] decode cache-resident {ms * 1e3:.2f} us/step")

    # one sequence per step (8192 channels, launch-bound): 64 eager calls
    # against the same 64 steps captured once in a HIP graph and replayed
    st1 = pools[0][:1].clone()
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
    eager_us = _timed(torch, steps64, 3) * 1e3 / 64
    graph_us = _timed(torch, graph.replay, 3) * 1e3 / 64
    decode["single_sequence"] = {"workload": "decode step of one sequence x d_inner 8192",
                                 "eager_us_per_step": round(eager_us, 3), "hip_graph_us_per_step": round(graph_us, 3)}
    del graph, pools, sets
    log(f"[bench] decode of one sequence {eager_us:.2f} us/step eager, {graph_us:.2f} us/step from a HIP graph")
    return decode


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--L", type=int, default=65536)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--leg-steps", type=int, default=10, help="timed calls of each further prefill leg")
    ap.add_argument("--backward-steps", type=int, default=5, help="timed backward calls (0: skip)")
    ap.add_argument("--all-configs", action="store_true",
                    help="time every workload (batch 2 x 4K, 64K, 256K single and chained, decode of 256 "
                         "sequences, 7-layer hybrid block) with the oracle on a sample; one JSON line each")
    ap.add_argument("--valu-ceiling", action="store_true",
                    help="only measure the VALU rates of this GPU for the scan's instruction mixes "
                         "(libjscan_ubench.so); --out writes a summary (and a .json beside it)")
    ap.add_argument("--summarize-trace", metavar="DB", help="write a kernel-trace summary (no GPU work)")
    ap.add_argument("--summarize-traffic", metavar="PMC_DIR",
                    help="write the HBM traffic summary, and traffic.json beside it (no GPU work)")
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
        summarize_traffic(args.summarize_traffic, args.out,
                          os.path.join(os.path.dirname(os.path.abspath(args.out)), "traffic.json"), args.command)
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
        raise SystemExit("libjscan.so is not built: run __graft_entry__.build() first")
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
    _, chunks = js.plan(batch, L, d_inner)

    def step():
        js.prefill(x, delta, A, B, C, D, z, None, y=y, hT=hT, workspace=ws)

    # Untimed: 0.25 s of calls while the clocks come up after the host-side
    # input generation and the fresh buffers are first touched, then the W
    # warmup steps.
    t_end = time.time() + 0.25
    while time.time() < t_end:
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({chunks} chunks)")

    # The timed steps.  Before each, the library is asked to record a pair of
    # events around that call's pass-1 kernel on its launch stream.
    evs = [_events(torch) for _ in range(args.steps)]
    for a, b in evs:                     # torch creates the event handles at their first record
        a.record(), b.record()
    e0, e1 = _events(torch)
    torch.cuda.synchronize()
    e0.record()
    for a, b in evs:
        js.time_next_prefill(a, b)
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    kern = [a.elapsed_time(b) for a, b in evs]
    kernel_ms = sum(kern) / len(kern)
    stats = js.prefill_stats(ws, batch, L, d_inner)
    log(f"[bench] step {ms_per_step:.4f} ms, pass 1 {kernel_ms:.4f} ms; chunks after the first: "
        f"{stats[0]:.3f} scanned state-only by pass 1, {stats[1]:.3f} rescanned by pass 2")

    # the device copy rate on this GPU (1 GiB read and 1 GiB written per copy)
    csrc = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    cdst = torch.empty_like(csrc)
    copy_ms = _timed(torch, lambda: cdst.copy_(csrc), 10)
    copy_gbs = 2 * csrc.numel() * 4 / (copy_ms * 1e-3) / 1e9
    del csrc, cdst
    log(f"[bench] device copy {copy_gbs:.0f} GB/s")

    chtok = batch * L * d_inner
    value = chtok / (ms_per_step * 1e-3)
    abytes = alg_bytes_prefill(batch, L, d_inner)
    kern_gbs = abytes / (kernel_ms * 1e-3) / 1e9
    call_gbs = abytes / (ms_per_step * 1e-3) / 1e9
    traffic = load_traffic("prefill_64k") if L == 65536 else None
    step_rate, clk = scan_step_ceiling()
    floor_ms = chtok / step_rate * 1e3
    log(f"[bench] VALU ceiling of one scan pass {step_rate:.4g} ch-tok/s ({floor_ms:.4f} ms at this size)")

    # The no-decay worst case: A = 0, pass 2 rescans every chunk after the
    # first.  Run as batch 2 x L/2 (the same channel-tokens and chunk length)
    # so that its kernels have a grid of their own in a kernel trace.
    A0 = torch.zeros_like(A)
    wb, wL = (2 * batch, L // 2) if L % 2 == 0 else (batch, L)
    xw, dw, zw, Bw, Cw = (t.view(wb, wL, -1) for t in (x, delta, z, B, C))
    yw, hw = y.view(wb, wL, -1), torch.empty(wb, d_inner, D_STATE, device=dev)
    wws = torch.empty(max(1, js.workspace_size(wb, wL, d_inner)), dtype=torch.uint8, device=dev)
    worst_ms = _timed(torch, lambda: js.prefill(xw, dw, A0, Bw, Cw, D, zw, None, y=yw, hT=hw, workspace=wws),
                      args.leg_steps)
    worst_stats = js.prefill_stats(wws, wb, wL, d_inner)
    worst_chunks = js.plan(wb, wL, d_inner)[1]
    del A0, wws, hw
    log(f"[bench] no-decay worst case (A = 0) {worst_ms:.4f} ms")

    decode = bench_decode(torch, js, synth, dio, dev, copy_gbs, log)

    # the same prefill with the fused input prologue (conv width 4 + SiLU, softplus(delta + dt_bias))
    pro = synth.prologue_params(d_inner, 4, seed=2)
    cw, cb, cs, dtb = (torch.from_numpy(pro[k]).to(dev) for k in ("conv_weight", "conv_bias", "conv_state",
                                                                  "dt_bias"))
    cso = torch.empty_like(cs)
    w_dt, w_B, w_C = (torch.from_numpy(w).to(dev) for w in synth.rms_weights(d_inner, seed=2))

    def fused(rms=None):
        js.prefill_fused(x, delta, A, B, C, D, z, None, y=y, hT=hT, workspace=ws, conv_weight=cw, conv_bias=cb,
                         conv_state_in=cs, conv_state_out=cso, dt_bias=dtb, softplus=True, rms=rms)
    fused_ms = _timed(torch, fused, args.leg_steps)
    fused_stats = js.prefill_stats(ws, batch, L, d_inner)
    rms_ms = _timed(torch, lambda: fused((w_dt, w_B, w_C, 1e-5)), args.leg_steps)
    prologue = {"workload": "the same prefill with the input prologue fused: causal depthwise conv width 4 + SiLU "
                            "on x, softplus(delta + dt_bias) with dt_bias = softplus^-1 of U(log 1e-3, log 1e-1)",
                "ms_per_step": round(fused_ms, 4), "channel_tokens_per_s": chtok / (fused_ms * 1e-3),
                "pass1_state_only_frac": round(fused_stats[0], 4), "pass2_rescanned_frac": round(fused_stats[1], 4),
                "with_rmsnorm": {"workload": "and RMSNorm of delta (over d_inner), B and C (over d_state), "
                                             "weights U(0.5, 1.5), eps 1e-5",
                                 "ms_per_step": round(rms_ms, 4), "over_fused": round(rms_ms - fused_ms, 4)}}
    log(f"[bench] fused prologue {fused_ms:.4f} ms, with RMSNorm {rms_ms:.4f} ms")

    # the exponential-trapezoidal recurrence on the same inputs (lam ~ U(0,1), token before the first)
    lam_np, xp_np, Bp_np = synth.trap_inputs(batch, L, d_inner, seed=2)
    lam_t, xp_t, Bp_t = dio(lam_np), dio(xp_np), dio(Bp_np)
    del lam_np
    trap_ms = _timed(torch, lambda: js.prefill_trap(x, delta, A, B, C, D, z, None, lam=lam_t, x_prev=xp_t,
                                                    B_prev=Bp_t, y=y, hT=hT, workspace=ws), args.leg_steps)
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
        bwd_ms = _timed(torch, lambda: js.backward(x, delta, A, B, C, D, z, dy, None, dhT, workspace=bws,
                                                   out=grads), args.backward_steps)
        # the same gradients from the chunk starting states the prefill left in
        # its workspace (jscan_backward_saved)
        step()
        saved_ms = _timed(torch, lambda: js.backward(x, delta, A, B, C, D, z, dy, None, dhT, workspace=bws,
                                                     prefill_workspace=ws, out=grads), args.backward_steps,
                          warm_s=0.0)
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
        model, avail = cpu_info()
        n_ch = 4096
        chans = np.arange(0, d_inner, d_inner // n_ch)[:n_ch]
        sub = synth.channel_slice(inp, chans)
        t0 = time.time()
        oracle.prefill(sub["x"], sub["delta"], sub["A"], sub["B"], sub["C"], sub["D"], sub["z"], None)
        dt = time.time() - t0
        threads = oracle.num_threads()
        cpu = {"value": n_ch * L / dt, "unit": "channel-tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{n_ch} of the {d_inner} channels (every {d_inner // n_ch}th) over all {L} tokens of the "
                         f"same inputs; the fp64 C oracle, {dt:.2f} s wall, one channel per OpenMP thread at a time",
               "threads": threads, "cpu_model": model, "available_cores": avail}
        log(f"[bench] cpu oracle {cpu['value']:.3e} ch-tok/s on {threads} threads ({model}, {avail} cores available)")

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
        "io_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"selective-scan prefill, batch {batch}, L {L}, d_inner {d_inner}, d_state 16, "
                               f"bf16 x/delta/z/B/C/y, fp32 A/D/state and arithmetic",
                   "batch": batch, "seq_len": L, "d_inner": d_inner, "d_state": D_STATE, "chunks": chunks},
        "roofline": {"bound": "hbm", "kernel": f"{PASS1} (pass 1 of the chunked scan)",
                     "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic["hbm_bytes_per_launch"] if traffic else None,
                     "kernel_ms": round(kernel_ms, 4), "alg_bytes_per_launch": abytes,
                     "whole_call": {"achieved": round(call_gbs, 1), "frac": round(call_gbs / HBM_PEAK_GBS, 4),
                                    "traffic": traffic["whole_call_bytes"] if traffic else None},
                     "measured_copy_GBps": round(copy_gbs, 1),
                     "frac_of_measured_copy": round(call_gbs / copy_gbs, 4)},
        "valu": {"bound": "alu", "ceiling": "libjscan_ubench scan-step kernel measured in this run: 16 x (mul, "
                                            "exp2, mul, FMA, FMA) + 3 plain fp32 instructions per channel-token",
                 "scan_step_chtok_per_s": step_rate, "shader_clock_mhz": round(clk, 1),
                 "single_pass_floor_ms": round(floor_ms, 4),
                 "frac_kernel": round(floor_ms / kernel_ms, 4), "frac_whole_call": round(floor_ms / ms_per_step, 4),
                 "hbm_frac_at_ceiling": round(abytes / (floor_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "chunked_plan": {"chunks": chunks, "pass1_state_only_frac": round(stats[0], 4),
                         "pass2_rescanned_frac": round(stats[1], 4),
                         "no_decay_worst_case": {"workload": f"A = 0 (nothing decays: pass 2 rescans every chunk "
                                                             f"after the first) on the same tokens as batch {wb} x "
                                                             f"{wL}, {worst_chunks} chunks of the same length",
                                                 "ms_per_step": round(worst_ms, 4),
                                                 "pass2_rescanned_frac": round(worst_stats[1], 4)}},
        "decode": decode,
        "prefill_fused_prologue": prologue,
        "prefill_trapezoidal": trap,
        "backward": backward,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
