#!/usr/bin/env python3
"""Benchmark: importance-weighted IQ encode throughput on one MI355X.

One step = the whole hot path on the dense 5632x2048 workload: collect the
imatrix from 4,096 bf16 tokens (1,024-row chunks) into a 2048-wide statistic,
turn it into importance, encode the 5632x2048 bf16 weight in the IQ2_XS layout
(512-entry seeded grid), decode it back to bf16.  Inputs are resident in HBM
before the timed region.  `value` = encoded elements per second of the whole
step (M elem/s).  Before the warm-up steps the chip is brought to the clock it
holds under this work: 0.25 s of a full-chip FMA stream, the ceiling
measurement, then 0.1 s of untimed steps (reported as `before_warmup`).

Also reported: the dominant kernel's roofline (the encoder's search kernel,
timed alone with HIP events around its own launches in every EVENT_STRIDE-th
timed step: an event pair costs the stream some 15-20 us, ~2.5% of a step, so
not every step carries one) in FLOP against the fp32
vector peak and against the VALU instruction rate measured on the same chip
(twice the fastest of three instruction streams, in FLOP), per-layout
encode throughput on the same weight, the fixed-choice IQ2_S variant, the IQ1
layouts on 17408x5120, the fused-MoE workload, and the CPU oracle's throughput
on a bounded sample of the same step.

Work model (FLOP, an FMA two, a MUL, ADD or MIN one), what the exhaustive
search needs and no more:
  per (row, 8-value group, grid entry): the -2P chain (8 FMA, 16) and the 16
    candidates of that entry (one FMA and one MIN each, 48); IQ1 adds the two
    shift terms (2 FMA, 4); an IQ2_XXS / IQ2_XS group with an odd count of
    negative values adds the parity term (8 MUL, 7 MIN, 1 FMA: 17), an even
    one needs none;
  per (expert, 8-column group, grid entry): the weighted norm (IQ2: 8 MUL and
    8 FMA, 24; IQ1: per shift 8 ADD, 8 MUL, 8 FMA, 64), which does not depend
    on the row.
The per-group setup (a few ops per value), the unit scoring (a few ops per
choice per group) and the index recovery of the argmin are not counted.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "encode M elem/s per IQ format on 5632×2048 (+ % of compute roofline)"
GRID_N = {"IQ2_XXS": 256, "IQ2_XS": 512, "IQ2_S": 1024, "IQ1_S": 2048, "IQ1_M": 2048}
# FLOP per (row, group, entry) for every group, and extra for odd-parity groups
ENTRY_FLOP = {"IQ2_XXS": (64, 17), "IQ2_XS": (64, 17), "IQ2_S": (64, 0), "IQ1_S": (68, 0), "IQ1_M": (68, 0)}
# FLOP per (expert, column group, entry): the weighted norms
NORM_FLOP = {"IQ2_XXS": 24, "IQ2_XS": 24, "IQ2_S": 24, "IQ1_S": 64, "IQ1_M": 64}
# MI355X fp32 vector peak (AMD's published dense figure): 157.3 TFLOP/s
PEAK_TFLOPS = 157.3
EVENT_STRIDE = 4  # timed steps whose search kernel carries a HIP-event pair: 0, 4, 8, ...
GRID_SEED = {"IQ2_XXS": 201, "IQ2_XS": 202, "IQ2_S": 203, "IQ1_S": 204, "IQ1_M": 204}
# The pages' own encode throughput on a 5632x2048 weight (CUDA kernels on NVIDIA
# GPUs, not this hardware; IQ2_XS not reported), for context next to ours
PAGES_M_ELEM_S = {"IQ2_XXS": 1047.9, "IQ2_S": 725.7, "IQ1_S": 306.0, "IQ1_M": 318.0}


def search_flop(fmt: str, rows: int, cols: int, experts: int, odd_groups: int) -> int:
    """FLOP the exhaustive search of one encode needs (module docstring)."""
    n = GRID_N[fmt]
    base, parity = ENTRY_FLOP[fmt]
    groups = rows * cols // 8
    return n * (groups * base + odd_groups * parity) + n * experts * (cols // 8) * NORM_FLOP[fmt]


def odd_parity_groups(w) -> int:
    """8-value groups of w with an odd count of negative values (-0 counts as
    positive), which are the groups the parity layouts charge a flip."""
    import torch
    neg = (w.view(w.shape[0], -1, 8) < 0).sum(dim=-1)
    return int((neg % 2).sum().item())


def source_hash() -> str:
    """Hash of the sources the search kernel is built from (the kernel the
    roofline line reports); stored traffic figures are used only while it matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "ggml_iq_codebook_imatrix_amd", "csrc")
    for name in ("iq_common.hpp", "iq_internal.hpp", "iq_encode.hip"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def cpu_model() -> str | None:
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _peak_lib():
    import ctypes
    path = os.path.join(ROOT, "ggml_iq_codebook_imatrix_amd", "libvalu_peak.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run the package build first")
    L = ctypes.CDLL(path)
    d = ctypes.POINTER(ctypes.c_double)
    L.valu_peak.argtypes = [ctypes.c_int, ctypes.c_int, d, d, d]
    L.valu_peak.restype = ctypes.c_int
    L.shader_clock.argtypes = [ctypes.c_int, d]
    L.shader_clock.restype = ctypes.c_int
    return L


def measured_valu_peak(iters: int = 2000) -> dict:
    """What this GPU sustains for the sweep's instruction forms (independent
    chains, 8 waves per SIMD, built like the encoder): VGPR-only fp32 FMA, the
    3-input min, and the candidate mix of two FMAs per 3-input min; in
    algorithmic ops (FMA 1, 3-input min 2) and in instructions, with the shader
    clock measured during the run.  By the work model every instruction the
    search issues carries at most 2 FLOP (an FMA or a 3-input min), so its FLOP
    rate is at most twice its instruction rate; the ceiling is twice the highest
    instruction rate of the three streams.  That is the mix: an FMA pairs with a
    3-input min as well as with another FMA, so it retires more instructions
    than the FMA stream (about 1.7x against 1.6x one wave instruction per SIMD
    per 4 clocks; the 3-input min alone stays at 1.0x).  It is a measured
    reference, not a proof: a stream with a better pairing would pass it.
    From libvalu_peak.so (ggml_iq_codebook_imatrix_amd/peak)."""
    import ctypes
    L = _peak_lib()
    d = ctypes.c_double
    out = {}
    clocks = []
    for mode, name in ((0, "fma"), (1, "min3"), (2, "mix")):
        ops, ins, clk = d(), d(), d()
        if L.valu_peak(mode, iters, ctypes.byref(ops), ctypes.byref(ins), ctypes.byref(clk)) != 0:
            raise RuntimeError(f"valu_peak mode {mode} failed")
        out[f"{name}_TOP_s"] = round(ops.value / 1e12, 2)
        out[f"{name}_Tinstr_s"] = round(ins.value / 1e12, 2)
        clocks.append(clk.value)
    out["fma_TFLOP_s"] = round(out["fma_TOP_s"] * 2, 2)
    out["ceiling_TFLOP_s"] = round(2 * max(out["fma_Tinstr_s"], out["min3_Tinstr_s"], out["mix_Tinstr_s"]), 2)
    out["clock_GHz"] = round(min(clocks) / 1e9, 3) if min(clocks) > 0 else None
    return out


def settle_clocks(seconds: float) -> dict:
    """Hold every CU under the ceiling's VGPR-only FMA stream for `seconds`
    before anything is measured; returns how long, how many runs, and the
    shader clock of the last one.  A fresh or idle MI355X meets a burst of work
    ~13% below its sustained clock and needs ~10-20 ms of full load to reach it
    (the microbenchmark back to back: 1.79 GHz in its first runs, 2.04-2.07 GHz
    from ~20 ms on), so a warm-up of a few steps would otherwise time the ramp
    rather than the kernels."""
    import ctypes
    L = _peak_lib()
    d = ctypes.c_double
    clk = d()
    t0 = time.perf_counter()
    runs = 0
    while runs == 0 or time.perf_counter() - t0 < seconds:
        ops, ins = d(), d()
        if L.valu_peak(0, 8000, ctypes.byref(ops), ctypes.byref(ins), ctypes.byref(clk)) != 0:
            raise RuntimeError("valu_peak failed")
        runs += 1
    return {"seconds": round(time.perf_counter() - t0, 3), "runs": runs, "clock_GHz": round(clk.value / 1e9, 3)}


def best_ceiling(a: dict, b: dict) -> dict:
    """Of two ceiling measurements, the higher one (a run can catch the clocks
    lower than the other)."""
    return a if a["ceiling_TFLOP_s"] >= b["ceiling_TFLOP_s"] else b


def shader_clock_ghz(us: int = 200) -> float | None:
    import ctypes
    c = ctypes.c_double()
    return round(c.value / 1e9, 3) if _peak_lib().shader_clock(us, ctypes.byref(c)) == 0 else None


def frac(achieved: float, peak: float, what: str) -> float:
    """achieved / the published peak; above 1 the work model counts work the
    kernel does not do, so the figure is refused rather than printed."""
    f = achieved / peak
    if f > 1.0:
        raise RuntimeError(f"{what}: {achieved:.2f} of a {peak:.2f} peak -- the work model is wrong")
    return round(f, 4)


def frac_measured(achieved: float, ceiling: float):
    """achieved / a measured ceiling, or None when the ceiling came out below
    the kernel's own rate (a clock change between the two runs): a fraction
    above 1 is not printed."""
    f = achieved / ceiling
    return round(f, 4) if f <= 1.0 else None


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--settle-s", type=float, default=0.25,
                    help="seconds of full-chip VALU load before the ceiling and the steps (0: none)")
    ap.add_argument("--step-settle-s", type=float, default=0.1,
                    help="seconds of untimed steps after the ceiling run, before the warm-up steps (0: none)")
    ap.add_argument("--reps", type=int, default=10, help="repetitions per extra encode measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the per-layout / MoE / 17408x5120 tables")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run 3 plain device copies of this many MiB (calibrates HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the encoder shards by rows or experts "
              "with no exchange, so a multi-GPU figure is not measured here.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from ggml_iq_codebook_imatrix_amd import api, inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_mb:
        n = args.copy_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n}))
        return 0
    log = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)

    def to_dev_bf16(a32):
        bits = inputs.f32_to_bf16_bits(a32)
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    # ---------------- inputs (resident before timing) ----------------------
    w32, x32, grid32, spec = inputs.workload("iq2_xs_5632x2048")
    rows, cols = w32.shape
    T = x32.shape[0]
    fmt = spec["fmt"]
    w = to_dev_bf16(w32)
    x = to_dev_bf16(x32)
    grid = torch.from_numpy(grid32).to(dev)
    # the statistics accumulate, so each step clears them: one buffer holds
    # sums [1, cols] f32 and counts [1] i64, cleared by one fill
    acc = torch.zeros(cols * 4 + 8, dtype=torch.uint8, device=dev)
    sums = acc[:cols * 4].view(torch.float32).view(1, cols)
    counts = acc[cols * 4:].view(torch.int64)
    imp = torch.empty((1, cols), dtype=torch.float32, device=dev)
    packed = torch.empty((rows, cols // 256, api.format_info(fmt)["block_bytes"]), dtype=torch.uint8, device=dev)
    w_hat = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
    status = api.new_status(dev)
    ws_c = torch.empty(api.collect_workspace_size(T, cols), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(api.quantize_workspace_size(fmt, rows, cols), dtype=torch.uint8, device=dev)
    odd = odd_parity_groups(w)
    log("inputs ready", fmt, rows, cols, "tokens", T, "odd-parity groups", odd)

    ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    timed_steps = list(range(0, args.steps, EVENT_STRIDE))  # the steps whose search kernel carries events

    def step(i=None):
        acc.zero_()
        api.imatrix_collect(x, chunk_rows=1024, sums=sums, counts=counts, status=status, workspace=ws_c)
        api.imatrix_importance(sums, counts, out=imp, status=status)
        api.quantize(fmt, w, grid, imp, out=packed, status=status, workspace=ws_q,
                     events=None if i is None or i % EVENT_STRIDE else (ev_s[i], ev_e[i]))
        api.dequantize(fmt, packed, grid, out=w_hat)

    # the clocks are brought up first, then the measured ceilings run (again
    # after the timed steps; the higher of the two is the ceiling), then the
    # untimed warm-up steps
    settle = settle_clocks(args.settle_s) if args.settle_s > 0 else None
    log("clocks settled", settle)
    meas0 = measured_valu_peak()
    log("measured VALU ceiling (before)", meas0)
    # the ceiling's FMA streams draw more power than the step, and the clock
    # they leave behind is below the one the step settles at (the search
    # kernel measured ~3% slower in the first steps after them), so the step
    # itself runs untimed for a moment before the warm-up steps
    step_settle = None
    if args.step_settle_s > 0:
        n_settle, ts = 0, time.perf_counter()
        while n_settle == 0 or time.perf_counter() - ts < args.step_settle_s:
            for _ in range(8):
                step()
            torch.cuda.synchronize()
            n_settle += 8
        step_settle = {"seconds": round(time.perf_counter() - ts, 3), "steps": n_settle}
        log("settled on the step", step_settle)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if api.read_status(status):
        raise RuntimeError(f"device status {api.read_status(status):#x}")
    log("warmup done")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    clock_after = shader_clock_ghz()
    meas1 = measured_valu_peak()
    meas = best_ceiling(meas0, meas1)
    log("measured VALU ceiling (after)", meas1)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    search_ms = float(np.mean([ev_s[i].elapsed_time(ev_e[i]) for i in timed_steps]))
    value = rows * cols / (ms_per_step * 1e-3) / 1e6
    log(f"step {ms_per_step:.4f} ms, search kernel {search_ms:.4f} ms, clock after {clock_after} GHz")

    flop = search_flop(fmt, rows, cols, 1, odd)
    achieved = flop / (search_ms * 1e-3) / 1e12
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "search_iq2_xs_5632x2048_traffic.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            tr = json.load(f)
        if tr.get("source_hash") == source_hash():
            traffic = tr.get("bytes_per_launch")
    roofline = {"bound": "alu", "achieved": round(achieved, 3), "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": frac(achieved, PEAK_TFLOPS, "search kernel vs fp32 peak"), "traffic": traffic,
                "kernel": "search_kernel<IQ2_XS>", "flop_per_launch": flop,
                "flop_per_elem": round(flop / (rows * cols), 1), "odd_parity_groups": odd,
                "ms_per_launch": round(search_ms, 4), "launches_timed": len(timed_steps),
                "measured_ceiling_TFLOP_s": meas["ceiling_TFLOP_s"],
                "frac_of_measured_ceiling": frac_measured(achieved, meas["ceiling_TFLOP_s"]),
                "clock_GHz_ceiling_run": meas["clock_GHz"], "clock_GHz_after_timed_steps": clock_after,
                "clock_settle": settle}
    roofline["measured"] = meas

    # ---------------- extras: every layout on the same weight --------------
    # each measurement below follows host-side set-up that leaves the chip
    # idle, so the clocks are brought up again before it (0.05 s: the ramp
    # takes ~10-20 ms), else a burst of a few ms would time the ramp
    def resettle():
        if args.settle_s > 0:
            settle_clocks(min(args.settle_s, 0.05))

    extras = {}
    if not args.no_extras:
        def time_encode(f, wd, g, impd, rpe=None, choices=None, reps=args.reps, odd_groups=None):
            ws = torch.empty(api.quantize_workspace_size(f, wd.shape[0], wd.shape[1], rpe, impd is not None),
                             dtype=torch.uint8, device=dev)
            out = api.quantize(f, wd, g, impd, rows_per_expert=rpe, choices=choices, workspace=ws)
            torch.cuda.synchronize()
            resettle()
            es = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
            ee = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
            ks = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
            ke = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
            for r in range(reps):
                es[r].record()
                api.quantize(f, wd, g, impd, rows_per_expert=rpe, choices=choices, out=out, workspace=ws,
                             events=(ks[r], ke[r]))
                ee[r].record()
            torch.cuda.synchronize()
            whole = float(np.median([es[r].elapsed_time(ee[r]) for r in range(reps)]))
            kern = float(np.median([ks[r].elapsed_time(ke[r]) for r in range(reps)]))
            n = wd.shape[0] * wd.shape[1]
            res = {"encode_ms": round(whole, 4), "search_ms": round(kern, 4),
                   "encode_M_elem_s": round(n / whole / 1e3, 1)}
            if choices is None:
                E = 1 if rpe is None else wd.shape[0] // rpe
                if odd_groups is None:
                    odd_groups = odd_parity_groups(wd)
                a = search_flop(f, wd.shape[0], wd.shape[1], E, odd_groups) / (kern * 1e-3) / 1e12
                res["search_TFLOP_s"] = round(a, 2)
                res["roofline_frac"] = frac(a, PEAK_TFLOPS, f"{f} search vs fp32 peak")
                res["frac_of_measured_ceiling"] = frac_measured(a, meas["ceiling_TFLOP_s"])
            return res

        per = {}
        for f in api.FORMATS:
            g = torch.from_numpy(inputs.grid_for(f, GRID_SEED[f])).to(dev)
            per[f] = time_encode(f, w, g, imp, odd_groups=odd)
            if f in PAGES_M_ELEM_S:
                per[f]["pages_cuda_M_elem_s"] = PAGES_M_ELEM_S[f]
            log(f, per[f])
        g = torch.from_numpy(inputs.grid_for("IQ2_S", 203)).to(dev)
        ch = torch.full((rows, cols // 256, 16), 7, dtype=torch.uint8, device=dev)
        per["IQ2_S_fixed_choice_7"] = time_encode("IQ2_S", w, g, imp, choices=ch)
        extras["per_format_5632x2048"] = per
        del ch

        # every-choice encode: one payload per choice from a single sweep
        ev = {}
        for f in api.FORMATS:
            g = torch.from_numpy(inputs.grid_for(f, GRID_SEED[f])).to(dev)
            out = api.quantize_every_choice(f, w, g, imp)
            torch.cuda.synchronize()
            resettle()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.reps):
                api.quantize_every_choice(f, w, g, imp, out=out)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.reps
            nc = api.format_info(f)["num_choices"]
            ev[f] = {"every_choice_ms": round(ms, 4), "choices": nc,
                     "vs_one_encode": round(ms / per[f]["encode_ms"], 2)}
            del out
        extras["every_choice_5632x2048"] = ev
        log("every choice", ev)

        # local-Hessian path: Hessian blocks from the same 4,096 tokens, then
        # the choice search (every-choice encode + unit picks + two passes)
        # writing the payload under its picks; for comparison, the choice
        # search alone and a separate encode under the picked choices
        def timed(fn, reps):
            fn()
            torch.cuda.synchronize()
            resettle()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        hess = torch.zeros((1, cols // 256, 256, 256), dtype=torch.float32, device=dev)

        def hess_fn():
            hess.zero_()
            api.hessian_collect(x, hess=hess)

        lh = {"hessian_collect_ms": round(timed(hess_fn, args.reps), 4)}
        hess_flops = 2.0 * T * cols * 256
        lh["hessian_TFLOP_s"] = round(hess_flops / (lh["hessian_collect_ms"] * 1e-3) / 1e12, 2)
        for f in api.FORMATS:
            g = torch.from_numpy(inputs.grid_for(f, GRID_SEED[f])).to(dev)
            chs, pay = api.choice_search(f, w, g, hess, imp, payload=True)
            cs_ms = timed(lambda: api.choice_search(f, w, g, hess, imp, out=chs), max(2, args.reps // 3))
            csp_ms = timed(lambda: api.choice_search(f, w, g, hess, imp, out=chs, payload=pay), max(2, args.reps // 3))
            enc = time_encode(f, w, g, imp, choices=chs)
            lh[f] = {"choice_search_ms": round(cs_ms, 4), "with_payload_ms": round(csp_ms, 4),
                     "separate_fixed_encode_ms": enc["encode_ms"],
                     "path_ms": round(lh["hessian_collect_ms"] + csp_ms, 4)}
            del chs, pay
        extras["local_hessian_5632x2048"] = lh
        log("local hessian", lh)
        del hess

        # IQ1 layouts on 17408x5120 (importance from 4,096 tokens)
        wl, xl, gl, sl = inputs.workload("iq1_s_17408x5120")
        wld, xld = to_dev_bf16(wl), to_dev_bf16(xl)
        del wl, xl
        s2, c2 = api.imatrix_collect(xld, chunk_rows=1024)
        impl = api.imatrix_importance(s2, c2)
        gl = torch.from_numpy(gl).to(dev)
        extras["iq1_17408x5120"] = {f: time_encode(f, wld, gl, impl, reps=max(3, args.reps // 2))
                                    for f in ("IQ1_S", "IQ1_M")}
        log("iq1 17408x5120", extras["iq1_17408x5120"])
        del wld, xld

        # fused MoE: 128 experts of 768x2048, top-8 routing with idle experts
        wm, xm, ids, gm, sm = inputs.moe_workload()
        wmd, xmd = to_dev_bf16(wm), to_dev_bf16(xm)
        idsd = torch.from_numpy(ids).to(dev)
        gmd = torch.from_numpy(gm).to(dev)
        E, rpe = sm["experts"], sm["rows_per_expert"]
        del wm, xm
        s3, c3 = api.imatrix_collect(xmd, idsd, E, chunk_rows=1024)
        torch.cuda.synchronize()
        resettle()
        ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ce0.record()
        for _ in range(args.reps):
            s3.zero_(); c3.zero_()
            api.imatrix_collect(xmd, idsd, E, chunk_rows=1024, sums=s3, counts=c3)
            impm = api.imatrix_importance(s3, c3)
        ce1.record()
        torch.cuda.synchronize()
        moe = time_encode("IQ2_XXS", wmd, gmd, impm, rpe=rpe, reps=max(3, args.reps // 2))
        moe["collect_importance_ms"] = round(ce0.elapsed_time(ce1) / args.reps, 4)
        moe["idle_experts"] = int((c3 == 0).sum().item())
        extras["moe_128x768x2048_iq2_xxs"] = moe
        log("moe", moe)
        # local-Hessian path per routed expert: each expert's Hessian blocks from
        # its own tokens, the choice search over all 128 experts in one launch
        hm = torch.zeros((E, cols // 256, 256, 256), dtype=torch.float32, device=dev)

        def hm_fn():
            hm.zero_()
            api.hessian_collect(xmd, idsd, E, hess=hm)

        mlh = {"hessian_collect_ms": round(timed(hm_fn, 3), 4)}
        chm, paym = api.choice_search("IQ2_XXS", wmd, gmd, hm, impm, rows_per_expert=rpe, payload=True)
        mlh["with_payload_ms"] = round(timed(lambda: api.choice_search("IQ2_XXS", wmd, gmd, hm, impm,
                                                                      rows_per_expert=rpe, out=chm, payload=paym),
                                             2), 4)
        mlh["path_ms"] = round(mlh["hessian_collect_ms"] + mlh["with_payload_ms"], 4)
        extras["moe_local_hessian_iq2_xxs"] = mlh
        log("moe local hessian", mlh)
        del hm, chm, paym, wmd, xmd

    # ---------------- CPU baseline: the oracle on a bounded sample ----------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
        t = time.perf_counter()
        oracle.quantize(fmt, w32[:32], grid32, np.ones((1, cols), np.float32), threads=threads)
        per_row = (time.perf_counter() - t) / 32
        n = int(min(rows, max(64, 12.0 / max(per_row, 1e-9))))
        t = time.perf_counter()
        s_o, c_o, _ = oracle.collect(x32)
        imp_o, _ = oracle.importance(s_o.astype(np.float32), c_o)
        p_o, _ = oracle.quantize(fmt, w32[:n], grid32, imp_o, threads=threads)
        oracle.dequantize(fmt, p_o, n, cols, grid32)
        dt = time.perf_counter() - t
        # the encode on one host thread, on the first 64 rows (same importance)
        t1 = time.perf_counter()
        oracle.quantize(fmt, w32[:64], grid32, imp_o, threads=1)
        dt1 = time.perf_counter() - t1
        cpu = {"value": round(n * cols / dt / 1e6, 4), "unit": "M elem/s", "cores": threads, "kind": "oracle",
               "sample": f"whole step (collect 4096x2048, importance, IQ2_XS encode + decode) on the first {n} of "
                         f"{rows} rows; {dt:.1f} s",
               "encode_one_thread": {"value": round(64 * cols / dt1 / 1e6, 4), "unit": "M elem/s",
                                     "sample": f"IQ2_XS encode of the first 64 rows on 1 thread; {dt1:.2f} s"},
               "host_cpus": os.cpu_count(), "host_cpu_model": cpu_model()}
        log("cpu baseline", cpu)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "M elem/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded; bf16 weights and tokens)",
        "config": {"workload": "dense IQ2_XS: collect 4096x2048 bf16 tokens in 1024-row chunks, importance, "
                               "encode + decode a 5632x2048 bf16 weight (512-entry seeded grid)",
                   "rows": rows, "cols": cols, "tokens": T, "format": fmt},
        # untimed work before the warm-up steps: the ceiling's FMA stream, then the step itself
        "before_warmup": {"fma_stream": settle, "steps": step_settle},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extras": extras,
        "source_hash": source_hash(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
