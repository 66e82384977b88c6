#!/usr/bin/env python3
"""Benchmark: importance-weighted IQ encode throughput on one MI355X.

One step = the whole hot path on the dense 5632x2048 workload: collect the
imatrix from 4,096 bf16 tokens (1,024-row chunks) into a 2048-wide statistic,
turn it into importance, encode the 5632x2048 bf16 weight in the IQ2_XS layout
(512-entry seeded grid), decode it back to bf16.  Inputs are resident in HBM
before the timed region.  `value` = encoded elements per second of the whole
step (M elem/s).

Also reported: the dominant kernel's roofline (the encoder's search kernel,
timed alone with HIP events around its own launches), per-layout encode
throughput on the same weight, the fixed-choice IQ2_S variant, the IQ1 layouts
on 17408x5120, the fused-MoE workload, and the CPU oracle's throughput on a
bounded sample of the same step.
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
# Algorithmic work of the exhaustive search per weight element (FMA, MUL and MIN
# count one op each): per (group, entry) the grid terms (IQ2_S 16, parity
# layouts and IQ1 32) plus 2 ops for each of the 16 (choice or shift, scale)
# candidates, times entries / 8 elements per group.
OPS_PER_ELEM = {"IQ2_XXS": 2048, "IQ2_XS": 4096, "IQ2_S": 6144, "IQ1_S": 16384, "IQ1_M": 16384}
# VALU peak: 256 CUs x 64 lanes x 2 ops per lane per clock (a 3-input min or a
# packed FMA retires two) x 2.4 GHz
PEAK_TOPS = 256 * 64 * 2 * 2.4e9 / 1e12
GRID_SEED = {"IQ2_XXS": 201, "IQ2_XS": 202, "IQ2_S": 203, "IQ1_S": 204, "IQ1_M": 204}


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


def measured_valu_peak(iters: int = 2000) -> dict:
    """What this GPU sustains for the sweep's instruction forms (independent
    chains, 8 waves per SIMD, built like the encoder): VGPR-only fp32 FMA, the
    3-input min, and the candidate mix of two FMAs per 3-input min; in
    algorithmic ops (FMA 1, 3-input min 2), with the shader clock measured
    during the run.  From libvalu_peak.so (ggml_iq_codebook_imatrix_amd/peak)."""
    import ctypes
    path = os.path.join(ROOT, "ggml_iq_codebook_imatrix_amd", "libvalu_peak.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run the package build first")
    L = ctypes.CDLL(path)
    d = ctypes.c_double
    L.valu_peak.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(d), ctypes.POINTER(d), ctypes.POINTER(d)]
    L.valu_peak.restype = ctypes.c_int
    out = {}
    clocks = []
    for mode, name in ((0, "fma"), (1, "min3"), (2, "mix")):
        ops, ins, clk = d(), d(), d()
        if L.valu_peak(mode, iters, ctypes.byref(ops), ctypes.byref(ins), ctypes.byref(clk)) != 0:
            raise RuntimeError(f"valu_peak mode {mode} failed")
        out[f"{name}_TOP_s"] = round(ops.value / 1e12, 2)
        out[f"{name}_Tinstr_s"] = round(ins.value / 1e12, 2)
        clocks.append(clk.value)
    out["clock_GHz"] = round(min(clocks) / 1e9, 3) if min(clocks) > 0 else None
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=40)
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
    sums = torch.zeros((1, cols), dtype=torch.float32, device=dev)
    counts = torch.zeros((1,), dtype=torch.int64, device=dev)
    imp = torch.empty((1, cols), dtype=torch.float32, device=dev)
    packed = torch.empty((rows, cols // 256, api.format_info(fmt)["block_bytes"]), dtype=torch.uint8, device=dev)
    w_hat = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
    status = api.new_status(dev)
    log("inputs ready", fmt, rows, cols, "tokens", T)

    ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]

    def step(i=None):
        sums.zero_()
        counts.zero_()
        api.imatrix_collect(x, chunk_rows=1024, sums=sums, counts=counts, status=status)
        api.imatrix_importance(sums, counts, out=imp, status=status)
        if i is not None:
            api.time_next_search(ev_s[i], ev_e[i])
        api.quantize(fmt, w, grid, imp, out=packed, status=status)
        api.dequantize(fmt, packed, grid, out=w_hat)

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
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    search_ms = float(np.mean([ev_s[i].elapsed_time(ev_e[i]) for i in range(args.steps)]))
    value = rows * cols / (ms_per_step * 1e-3) / 1e6
    log(f"step {ms_per_step:.4f} ms, search kernel {search_ms:.4f} ms")

    ops = OPS_PER_ELEM[fmt] * rows * cols
    achieved = ops / (search_ms * 1e-3) / 1e12
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "search_iq2_xs_5632x2048_traffic.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            tr = json.load(f)
        if tr.get("source_hash") == source_hash():
            traffic = tr.get("bytes_per_launch")
    roofline = {"bound": "alu", "achieved": round(achieved, 3), "peak": round(PEAK_TOPS, 2), "unit": "TOP/s",
                "frac": round(achieved / PEAK_TOPS, 4), "traffic": traffic,
                "kernel": "search_kernel<IQ2_XS>", "ops_per_launch": ops, "ms_per_launch": round(search_ms, 4)}
    meas = measured_valu_peak()
    meas["frac_of_mix"] = round(achieved / meas["mix_TOP_s"], 4)
    roofline["measured"] = meas
    log("measured VALU ceiling", meas)

    # ---------------- extras: every layout on the same weight --------------
    extras = {}
    if not args.no_extras:
        def time_encode(f, wd, g, impd, rpe=None, choices=None, reps=args.reps):
            out = api.quantize(f, wd, g, impd, rows_per_expert=rpe, choices=choices)
            torch.cuda.synchronize()
            es = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
            ee = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
            ks = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
            ke = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
            for r in range(reps):
                api.time_next_search(ks[r], ke[r])
                es[r].record()
                api.quantize(f, wd, g, impd, rows_per_expert=rpe, choices=choices, out=out)
                ee[r].record()
            torch.cuda.synchronize()
            whole = float(np.median([es[r].elapsed_time(ee[r]) for r in range(reps)]))
            kern = float(np.median([ks[r].elapsed_time(ke[r]) for r in range(reps)]))
            n = wd.shape[0] * wd.shape[1]
            res = {"encode_ms": round(whole, 4), "search_ms": round(kern, 4),
                   "encode_M_elem_s": round(n / whole / 1e3, 1)}
            if choices is None:
                a = OPS_PER_ELEM[f] * n / (kern * 1e-3) / 1e12
                res["search_TOP_s"] = round(a, 2)
                res["roofline_frac"] = round(a / PEAK_TOPS, 4)
            return res

        per = {}
        for f in api.FORMATS:
            g = torch.from_numpy(inputs.grid_for(f, GRID_SEED[f])).to(dev)
            per[f] = time_encode(f, w, g, imp)
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
        threads = min(os.cpu_count() or 1, 16)
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
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extras": extras,
        "source_hash": source_hash(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
