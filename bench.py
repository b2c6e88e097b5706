#!/usr/bin/env python3
"""Benchmark of the MXFP8 MoE expert path on one MI355X.

Workload (the large expert GEMM case): 8192 tokens x hidden 5120, top-2
routing over 16 experts (one expert forced empty) -> 16384 routed rows, ffn
8192, bf16 inputs N(0,1) with 0.1% outliers x1000.  One step = the whole hot
path, forward plus backward (``moe.STAGES``): X rowwise quantize, route +
MXFP8 permute, W rowwise + columnwise quantize, grouped GEMM fwd, dY rowwise
+ columnwise quantize, grouped GEMM dgrad, X columnwise quantize in permuted
order, grouped GEMM wgrad; GEMM outputs in bf16.  Inputs are resident in HBM
before the timed region.

Printed: one JSON line.  ``value`` = GEMM FLOPs of a step (3 x 2*M*N*K over
the real routed rows) / step time (the timed region over ``--steps`` eager
steps, with no instrumentation inside it), in TFLOP/s.  ``stages`` gives
each stage's median duration (HIP events around every stage, in a second
pass of ``--steps`` steps; 70 steps, about 0.2 s each, by default) and
its throughput against the MI355X peak (``frac``: MXFP8 dense 5.0 PFLOP/s,
HBM 8 TB/s) and against the ceilings measured at the start of the run
(``frac_ceiling``; ``ceilings``: a streaming copy and a scaled-MFMA-only
loop, kernels of the library; the row+col quantize stages also carry
``frac_pattern``, against the tile quantizer's loads and stores timed with
no arithmetic).  ``stages_mall_flushed`` times every stage
again after a 512 MB fill that evicts the Infinity Cache.
``small_configs`` times the tiny (forward, microseconds) and mid (forward +
dgrad + wgrad) workloads.
``roofline`` reports the dominant GEMM stage.  ``fused_quant_permute`` times
the same step with the quantize fused into the permute (routing metadata plus
one gathered row+col quantize of the bf16 tokens in place of the X quantize,
the MXFP8 permute and the permuted X columnwise quantize; same bytes out);
the headline keeps the MXFP8 permute, the step that becomes a transfer
between devices when experts are sharded.  ``quantize_bandwidth`` times
the fused rowwise+columnwise quantize and both dequantizes of a
[16*8192, 5120] bf16 tensor.  ``swiglu_layer`` times the full SwiGLU expert
FFN layer (64 experts, top-8, 32768 tokens, hidden 7168, ffn 2048) forward
plus backward, stage by stage, including the router, SwiGLU and combine
glue (and its fused-permute variant).  ``bf16_baseline`` times the same
expert step with bf16 operands (bf16 gather and transposes, bf16-MFMA grouped
GEMMs of the same kernel design) and the MXFP8 speedup over it;
``swiglu_layer.bf16_gemms`` does the same for the layer's six GEMMs.
``graph`` (and ``swiglu_layer.graph``) replays the step captured once in a
HIP graph.
``cpu_baseline`` times the oracle on a bounded sample (three
median-sized experts' share of the step, and the fused quantize of a slice
of the bandwidth workload), with the host's CPU model and core count.
"""

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MXFP8_TFLOPS = 5000.0   # MI355X dense FP8/MXFP8 MFMA
PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense BF16 MFMA
METRIC = "MXFP8 grouped-GEMM TFLOP/s fwd+bwd and quantize GB/s, % of MI355X peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
CALIB_BYTES = 1 << 30        # plain device copy used to scale the FETCH_SIZE / WRITE_SIZE counters

# Counter pass (--counter-pass): every stage runs COUNTER_REPS times, each
# launch bracketed by marker kernels, so that per-dispatch hardware counters
# (rocprofv3 --pmc) can be attributed to stages by position alone.
COUNTER = None
COUNTER_REPS = 3
MARKER_KERNEL = "FillFunctor<long>"   # the marker: a one-element int64 fill (nothing else on the path fills int64)


def counter_mark(label):
    """Counter pass: launch the marker kernel; the launches up to the next
    marker belong to ``label``."""
    COUNTER["labels"].append(label)
    COUNTER["marker"].fill_(len(COUNTER["labels"]))


def counter_work(prefix, nbytes):
    """Counter pass: record the algorithmic bytes of the stages ``prefix + name``."""
    if COUNTER is not None:
        COUNTER["alg"].update({prefix + n: float(v) for n, v in nbytes.items()})


def measured_traffic(stage):
    """HBM bytes per launch of ``stage`` as recorded in profiles/hbm_traffic.txt
    (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a copy of known size), or
    None when no record exists or a kernel source changed since it was taken
    (the record hashes its comma-separated source files, concatenated)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    for line in open(TRAFFIC_FILE):
        if not line.startswith("stage="):
            continue
        kv = dict(f.split("=", 1) for f in line.split())
        if kv.get("stage") != stage:
            continue
        srcs = [os.path.join(ROOT, f) for f in kv["source"].split(",")]
        if not all(os.path.exists(f) for f in srcs):
            return None
        if hashlib.sha256(b"".join(open(f, "rb").read() for f in srcs)).hexdigest() != kv["sha256"]:
            return None
        return {"fetch_bytes": float(kv["fetch_bytes"]), "write_bytes": float(kv["write_bytes"]),
                "bytes": float(kv["fetch_bytes"]) + float(kv["write_bytes"])}
    return None


def ensure_built():
    import mxfp8_block_scaled_07_amd as mxa
    if not os.path.exists(mxa.LIB_PATH):
        from mxfp8_block_scaled_07_amd import _build
        _build.build()


def time_stages(run, names, steps, warmup, flush=None, label=""):
    """Run ``run(name)`` for every name, ``warmup`` untimed then ``steps`` timed
    passes with per-stage HIP events on torch's current stream (the launch
    stream), for the per-stage medians; then (without ``flush``) ``steps``
    more passes with no events inside the timed region, for the time per
    pass, so that the event records between stages do not count in it.
    Returns (ms per pass, per-stage median ms, wall seconds of the pass
    whose time is returned).
    With ``flush`` (a callable), it runs before every stage, outside the
    stage's events (and inside the timed region).  In the counter pass each
    stage instead runs COUNTER_REPS times between markers labelled
    ``label + name`` (the cache-flushed passes are skipped) and the times
    returned are placeholders."""
    import statistics

    import torch
    if COUNTER is not None:
        if flush is None:
            print(f"counter pass: {label}{names[0]} .. {names[-1]}", file=sys.stderr, flush=True)
            for _ in range(COUNTER_REPS):
                for n in names:
                    counter_mark(label + n)
                    run(n)
                    counter_mark("other")
            torch.cuda.synchronize()
        return 1.0, {n: 1.0 for n in names}, 0.0
    for _ in range(warmup):
        for n in names:
            run(n)
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in names]
          for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(steps):
        for j, n in enumerate(names):
            if flush is not None:
                flush()
            ev[i][j][0].record()
            run(n)
            ev[i][j][1].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    per = {n: statistics.median(ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(steps))
           for j, n in enumerate(names)}
    if flush is None:
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t_start.record()
        for i in range(steps):
            for n in names:
                run(n)
        t_end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        total_ms = t_start.elapsed_time(t_end)
    return total_ms / steps, per, wall


def mall_flusher(nbytes=512 << 20):
    """A callable that overwrites ``nbytes`` of device memory (a fill kernel):
    run before a stage, it evicts that stage's inputs from the 256 MB
    Infinity Cache."""
    import torch
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    state = {"v": 0}

    def flush():
        state["v"] ^= 1
        buf.fill_(state["v"])
    return flush


def measure_ceilings(copy_bytes=1344 << 20, reps=7):
    """Measured ceilings of this part (library kernels mx_ceiling_copy,
    mx_ceiling_tile_pattern and mx_ceiling_mfma): the median HBM rate of a
    streaming copy of ``copy_bytes`` (read + write bytes per second; 2.7 GB
    moved, the size of the fused quantize's traffic), the median rate of the
    tile quantizer's access pattern without its arithmetic on the
    quantize-bandwidth tensor [131072, 5120] (bf16 in, both code
    orientations out: 2.7 GB), and the median rate of a loop of scaled FP8
    MFMAs in the grouped GEMMs' register pattern, on random operands (the
    rate the part sustains on real data: their switching power lowers the
    clock) and on near-constant operands (TFLOP/s)."""
    import statistics

    import torch

    import mxfp8_block_scaled_07_amd as mxa
    src = torch.ones(copy_bytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dev = torch.cuda.get_device_properties(0)
    wgs = dev.multi_processor_count
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda:0")
    iters = 20000
    # the tile pattern reads [R, C] bf16 from the copy's source and writes both
    # R x C code arrays into its destination (2 R C <= copy_bytes)
    R, C = 131072, 5120
    row_out, col_out = dst[:R * C], dst[R * C:2 * R * C]
    mxa.mx_ceiling_copy(src, dst, copy_bytes)
    mxa.mx_ceiling_tile_pattern(src, row_out, col_out, R, C)
    mxa.mx_ceiling_mfma(out, wgs, 100, True)
    torch.cuda.synchronize()
    cp, tp, mf, mc = [], [], [], []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        e[0].record()
        mxa.mx_ceiling_copy(src, dst, copy_bytes)
        e[1].record()
        mxa.mx_ceiling_tile_pattern(src, row_out, col_out, R, C)
        e[2].record()
        mxa.mx_ceiling_mfma(out, wgs, iters, True)
        e[3].record()
        mxa.mx_ceiling_mfma(out, wgs, iters, False)
        e[4].record()
        torch.cuda.synchronize()
        cp.append(e[0].elapsed_time(e[1]))
        tp.append(e[1].elapsed_time(e[2]))
        mf.append(e[2].elapsed_time(e[3]))
        mc.append(e[3].elapsed_time(e[4]))
    flops = wgs * 4 * iters * 16 * 131072.0
    res = {"hbm_copy_gbps": round(2 * copy_bytes / (statistics.median(cp) * 1e-3) / 1e9, 1),
           "quant_pattern_gbps": round(4 * R * C / (statistics.median(tp) * 1e-3) / 1e9, 1),
           "mfma_mxfp8_tflops": round(flops / (statistics.median(mf) * 1e-3) / 1e12, 1),
           "mfma_mxfp8_tflops_constant_operands": round(flops / (statistics.median(mc) * 1e-3) / 1e12, 1),
           "copy_bytes_moved": 2 * copy_bytes, "cus": wgs,
           "note": "medians of 7 launches: mx_ceiling_copy (16-byte non-temporal streaming copy, one chunk per "
                   "thread, read + write bytes / time), mx_ceiling_tile_pattern (the row+col tile quantizer's loads "
                   "and stores with no arithmetic, [131072, 5120] bf16 in, 4 bytes per element moved) and "
                   "mx_ceiling_mfma (16 independent 32x32x64 scaled FP8 MFMAs per wave on the GEMM "
                   "step's 4 A + 4 B register fragments, one wave per SIMD); mfma_mxfp8_tflops uses random codes "
                   "and scales (the ceiling on real data), the constant-operand figure shows the clock headroom "
                   "that data-dependent power takes away"}
    del src, dst, out
    torch.cuda.empty_cache()
    return res


def time_graph(g, steps, warmup):
    """ms per replay of a captured step: ``warmup`` untimed replays, then
    ``steps`` replays between two events on torch's current stream."""
    import torch
    if COUNTER is not None:
        return 1.0
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


# stages that quantize a plain bf16 tensor in both orientations: their
# frac_pattern compares them with the tile quantizer's own access pattern
ROWCOL_QUANT_STAGES = ("quant_w", "quant_dy")


def stage_entry(n, ms, work, ceil):
    """Throughput of one stage against the published peak (frac) and the
    measured ceiling (frac_ceiling)."""
    if n in work["gemm_flops"]:
        tf = work["gemm_flops"][n] / (ms * 1e-3) / 1e12
        return {"ms": round(ms, 4), "tflops": round(tf, 1), "frac": round(tf / PEAK_MXFP8_TFLOPS, 4),
                "frac_ceiling": round(tf / ceil["mfma_mxfp8_tflops"], 4)}
    gbs = work["bytes"][n] / (ms * 1e-3) / 1e9
    e = {"ms": round(ms, 4), "gbps": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBPS, 4),
         "frac_ceiling": round(gbs / ceil["hbm_copy_gbps"], 4)}
    if n in ROWCOL_QUANT_STAGES:
        e["frac_pattern"] = round(gbs / ceil["quant_pattern_gbps"], 4)
    return e


def gpu_expert_path(args, c, ceil):
    import numpy as np
    import torch

    from mxfp8_block_scaled_07_amd import MX_OUT_BF16, moe

    T, K, N, E, topk = c["T"], c["K"], c["N"], c["E"], c["topk"]
    dev = "cuda:0"
    x = torch.from_numpy(c["x"].view(np.int16)).to(dev)
    w = torch.from_numpy(c["w"].view(np.int16)).to(dev)
    ids = torch.from_numpy(c["expert_ids"].astype(np.int32)).to(dev)
    dy_full = torch.from_numpy(c["dy_full"].view(np.int16)).to(dev)
    b = moe.ExpertBuffers(T, K, N, E, topk, device=dev, out_dtype=MX_OUT_BF16)
    moe.run_stage("quant_x", b, x, w, None, ids)
    moe.run_stage("permute", b, x, w, None, ids)
    dy = moe.zero_pad_rows(dy_full, b.src)
    del dy_full
    torch.cuda.synchronize()
    M = T * topk
    step_ms, per, wall = time_stages(lambda n: moe.run_stage(n, b, x, w, dy, ids), moe.STAGES, args.steps,
                                     args.warmup)
    work = moe.algorithmic_work(T, K, N, E, topk, M)
    for pre in ("", "fused."):
        counter_work(pre, {**work["bytes"], **work["gemm_operand_bytes"]})
    stages = {}
    for n in moe.STAGES:
        stages[n] = stage_entry(n, per[n], work, ceil)
        tr = measured_traffic(n)
        stages[n]["traffic"] = None if tr is None else tr["bytes"]
    # the same stages each timed after evicting the Infinity Cache (a 512 MB
    # fill before every stage): inputs come from HBM even when they are small
    _, fper, _ = time_stages(lambda n: moe.run_stage(n, b, x, w, dy, ids), moe.STAGES, max(50, args.steps),
                             args.warmup, flush=mall_flusher())
    flushed = {n: stage_entry(n, fper[n], work, ceil) for n in moe.STAGES}
    gemm_total = sum(work["gemm_flops"].values())
    value = gemm_total / (step_ms * 1e-3) / 1e12
    # the same step with the quantize fused into the permute (same bytes out)
    f_ms, f_per, _ = time_stages(lambda n: moe.run_stage(n, b, x, w, dy, ids), moe.FUSED_STAGES, args.steps,
                                 args.warmup, label="fused.")
    fused_stages = {}
    for n in moe.FUSED_STAGES:
        if n in work["gemm_flops"]:
            fused_stages[n] = {"ms": round(f_per[n], 4),
                               "tflops": round(work["gemm_flops"][n] / (f_per[n] * 1e-3) / 1e12, 1)}
        else:
            fused_stages[n] = {"ms": round(f_per[n], 4),
                               "gbps": round(work["bytes"][n] / (f_per[n] * 1e-3) / 1e9, 1)}
    fused = {"ms_per_step": round(f_ms, 4), "tflops": round(gemm_total / (f_ms * 1e-3) / 1e12, 1),
             "stages": fused_stages,
             "note": "routing metadata + one gathered row+col quantize of the bf16 tokens replace quant_x, "
                     "the MXFP8 permute and quant_xt; bit-identical results"}
    # the same step captured once in a HIP graph and replayed (no host launch
    # gaps, no per-stage events)
    graph = None if COUNTER is not None else moe.capture(lambda: moe.expert_step(b, x, w, dy, ids))
    g_ms = time_graph(graph, args.steps, args.warmup)
    del graph
    graph_res = {"ms_per_step": round(g_ms, 4), "tflops": round(sum(work["gemm_flops"].values()) / (g_ms * 1e-3) / 1e12, 1),
                 "note": "the step's launches captured in one HIP graph (torch.cuda.CUDAGraph) and replayed"}
    bf16 = gpu_bf16_step(args, c, x, w, dy, ids, work, step_ms, per)
    dom = max(work["gemm_flops"], key=lambda n: per[n])
    dom_tf = work["gemm_flops"][dom] / (per[dom] * 1e-3) / 1e12
    counts = np.bincount(c["expert_ids"].ravel(), minlength=E)
    tr = measured_traffic(dom)
    result = {
        "value": value, "ms_per_step": step_ms, "stages": stages, "wall_s_timed": wall,
        "stages_mall_flushed": flushed,
        "fused_quant_permute": fused,
        "graph": graph_res,
        "bf16_baseline": bf16,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(dom_tf, 1), "peak": PEAK_MXFP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(dom_tf / PEAK_MXFP8_TFLOPS, 4),
                     "ceiling": ceil["mfma_mxfp8_tflops"],
                     "frac_ceiling": round(dom_tf / ceil["mfma_mxfp8_tflops"], 4),
                     "traffic": None if tr is None else tr["bytes"],
                     "traffic_detail": tr, "algorithmic_operand_bytes": work["gemm_operand_bytes"][dom],
                     "per_launch_flops": work["gemm_flops"][dom], "avg_launch_ms": round(per[dom], 4)},
        "config": {"workload": "large expert GEMM fwd+dgrad+wgrad: T=8192 tokens, top-2 of E=16 experts "
                               "(16384 routed rows, >=1 empty expert), hidden K=5120, ffn N=8192, "
                               "bf16 N(0,1) inputs with 0.1% x1000 outliers, MXFP8 operands, bf16 GEMM outputs",
                   "tokens": T, "topk": topk, "experts": E, "hidden": K, "ffn": N,
                   "routed_rows": M, "capacity_rows": b.cap, "empty_experts": int((counts == 0).sum())},
    }
    del b, x, w, dy
    torch.cuda.empty_cache()
    return result


def gpu_bf16_step(args, c, x, w, dy, ids, work, mx_step_ms, mx_per):
    """The BF16 baseline of the same step on the same bf16 inputs: routing,
    bf16 token gather, bf16 transposes in place of the columnwise quantizes,
    and the three grouped GEMMs on bf16 operands (same kernel design, bf16
    MFMA).  Reports its stages against the bf16 MFMA and HBM peaks and the
    MXFP8 speedup over it (step and per GEMM)."""
    import torch

    from mxfp8_block_scaled_07_amd import MX_OUT_BF16, moe

    T, K, N, E, topk = c["T"], c["K"], c["N"], c["E"], c["topk"]
    b = moe.Bf16Buffers(T, K, N, E, topk, device="cuda:0", out_dtype=MX_OUT_BF16)
    ms, per, _ = time_stages(lambda n: moe.run_bf16_stage(n, b, x, w, dy, ids), moe.BF16_STAGES, args.steps,
                             args.warmup, label="bf16.")
    bw = moe.bf16_work(T, K, N, E, topk)
    counter_work("bf16.", {**bw["bytes"], **bw["gemm_operand_bytes"]})
    stages = {}
    for n in moe.BF16_STAGES:
        if n in work["gemm_flops"]:
            tf = work["gemm_flops"][n] / (per[n] * 1e-3) / 1e12
            stages[n] = {"ms": round(per[n], 4), "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "mxfp8_speedup": round(per[n] / mx_per[n], 3)}
        else:
            gbs = bw["bytes"][n] / (per[n] * 1e-3) / 1e9
            stages[n] = {"ms": round(per[n], 4), "gbps": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBPS, 4)}
        tr = measured_traffic("bf16." + n)
        stages[n]["traffic"] = None if tr is None else tr["bytes"]
    gemm_ms = sum(per[n] for n in work["gemm_flops"])
    mx_gemm_ms = sum(mx_per[n] for n in work["gemm_flops"])
    flops = sum(work["gemm_flops"].values())
    del b
    torch.cuda.empty_cache()
    return {"ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "mxfp8_step_speedup": round(ms / mx_step_ms, 3), "mxfp8_gemm_speedup": round(gemm_ms / mx_gemm_ms, 3),
            "peak_bf16_tflops": PEAK_BF16_TFLOPS, "stages": stages,
            "note": "same step on bf16 operands: routing, bf16 token gather, bf16 transposes of W, dY and X_perm "
                    "(the columnwise quantizes' counterparts), bf16-MFMA grouped GEMMs of the same kernel design"}


def gpu_small_configs(args, ceil):
    """The tiny and mid workloads of the benchmark specification, timed like
    the headline step (medians over >= 50 passes): the tiny case forward only
    (E=4, K=256, N=512, 2048 rows, fp32 output; its kernels are launch-bound,
    so it is reported in microseconds) and the mid case forward + dgrad +
    wgrad (E=8, K=2048, N=1408, 16384 Zipf-sized rows, bf16 outputs)."""
    import numpy as np
    import torch

    import workloads
    from mxfp8_block_scaled_07_amd import MX_OUT_BF16, MX_OUT_F32, moe

    out = {}
    for cfg, stages, od in ((1, ("quant_x", "permute", "quant_w", "gemm_fwd"), MX_OUT_F32),
                            (2, moe.STAGES, MX_OUT_BF16)):
        c = workloads.config(cfg)
        T, K, N, E, topk = c["T"], c["K"], c["N"], c["E"], c["topk"]
        dev = "cuda:0"
        x = torch.from_numpy(c["x"].view(np.int16)).to(dev)
        w = torch.from_numpy(c["w"].view(np.int16)).to(dev)
        ids = torch.from_numpy(c["expert_ids"].astype(np.int32)).to(dev)
        b = moe.ExpertBuffers(T, K, N, E, topk, device=dev, out_dtype=od)
        dy = None
        if "dy_full" in c:
            moe.run_stage("quant_x", b, x, w, None, ids)
            moe.run_stage("permute", b, x, w, None, ids)
            dy = moe.zero_pad_rows(torch.from_numpy(c["dy_full"].view(np.int16)).to(dev), b.src)
        torch.cuda.synchronize()
        step_ms, per, _ = time_stages(lambda n: moe.run_stage(n, b, x, w, dy, ids), stages, max(50, args.steps),
                                      args.warmup, label=f"config{cfg}.")
        work = moe.algorithmic_work(T, K, N, E, topk)
        st = {n: stage_entry(n, per[n], work, ceil) for n in stages}
        for n in st:
            st[n]["us"] = round(per[n] * 1e3, 2)
        flops = sum(work["gemm_flops"][n] for n in stages if n in work["gemm_flops"])
        gemm_ms = sum(per[n] for n in stages if n in work["gemm_flops"])
        out[f"config{cfg}"] = {
            "workload": ("tiny expert GEMM fwd: E=4, K=256, N=512, 2048 rows, fp32 output" if cfg == 1 else
                         "mid expert layer fwd+dgrad+wgrad: E=8, K=2048, N=1408, 16384 Zipf(1.2)-sized rows, "
                         "bf16 outputs"),
            "us_per_step": round(step_ms * 1e3, 2), "gemm_us": round(gemm_ms * 1e3, 2),
            "gemm_tflops": round(flops / (gemm_ms * 1e-3) / 1e12, 1),
            "gemm_frac": round(flops / (gemm_ms * 1e-3) / 1e12 / PEAK_MXFP8_TFLOPS, 4), "stages": st}
        del b, x, w, dy
        torch.cuda.empty_cache()
    out["note"] = ("the tiny case's GEMM is 0.54 GFLOP, far below one launch's latency: its fraction of the "
                   "peak is not meaningful and is reported for completeness")
    return out


def gpu_quantize_bandwidth(args, ceil):
    import numpy as np
    import torch

    import workloads
    import mxfp8_block_scaled_07_amd as mxa

    rows, cols = 16 * 8192, 5120
    xb = workloads.quant_tensor(4, rows, cols)
    x = torch.from_numpy(xb.view(np.int16)).to("cuda:0")
    del xb
    q, s, qt, st = mxa.quantize(x, rowwise=True, colwise=True)
    y = torch.empty_like(x)
    yt = torch.empty((cols, rows), dtype=torch.int16, device=x.device)

    def run(n):
        if n == "quant_rowcol":
            mxa.mx_quantize(x, 1, rows, cols, None, rows, q, s, qt, st)
        elif n == "dequant_row":
            mxa.mx_dequantize(q, s, rows, cols, y)
        else:
            mxa.mx_dequantize(qt, st, cols, rows, yt)

    names = ("quant_rowcol", "dequant_row", "dequant_col")
    _, per, _ = time_stages(run, names, max(50, args.steps), 2, label="quant.")
    n_el = rows * cols
    nbytes = {"quant_rowcol": n_el * (2 + 2 * (1 + 1 / 32)), "dequant_row": n_el * (1 + 1 / 32 + 2),
              "dequant_col": n_el * (1 + 1 / 32 + 2)}
    out = {}
    for n in names:
        gbs = nbytes[n] / (per[n] * 1e-3) / 1e9
        tr = measured_traffic("quant." + n)
        out[n] = {"ms": round(per[n], 4), "gbps": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBPS, 4),
                  "frac_ceiling": round(gbs / ceil["hbm_copy_gbps"], 4), "traffic": None if tr is None else tr["bytes"]}
        if n == "quant_rowcol":
            out[n]["frac_pattern"] = round(gbs / ceil["quant_pattern_gbps"], 4)
    counter_work("quant.", nbytes)
    out["shape"] = [rows, cols]
    del x, q, s, qt, st, y, yt
    torch.cuda.empty_cache()
    return out


def gpu_swiglu_layer(args):
    """The full SwiGLU expert FFN layer of the 64-expert top-8 workload (T=32768
    tokens, hidden 7168, expert ffn 2048), forward plus backward, on the seeded
    synthetic inputs of ``workloads.layer_inputs`` (drawn on the GPU).  Every
    stage is timed like the headline step; the glue kernels (SwiGLU, combine
    and their backwards) are reported against HBM bandwidth."""
    import torch

    from mxfp8_block_scaled_07_amd import moe

    import workloads
    inp = workloads.layer_inputs("cuda:0")
    T, H, F, E, k = inp["T"], inp["H"], inp["F"], inp["E"], inp["topk"]
    dev = "cuda:0"
    logits, x, dout, w1, w2 = inp["logits"], inp["x"], inp["dout"], inp["w1"], inp["w2"]
    del inp
    b = moe.LayerBuffers(T, H, F, E, k, device=dev)
    torch.cuda.synchronize()
    steps = max(3, args.steps // 4)
    step_ms, per, _ = time_stages(lambda n: moe.run_layer_stage(n, b, x, w1, w2, logits, dout),
                                  moe.LAYER_STAGES, steps, 2, label="layer.")
    work = moe.layer_work(T, H, F, E, k)
    for pre in ("layer.", "layer_fused."):
        counter_work(pre, {**work["bytes"], **work["gemm_operand_bytes"]})
    stages = {}
    for n in moe.LAYER_STAGES:
        ms = per[n]
        if n in work["gemm_flops"]:
            tf = work["gemm_flops"][n] / (ms * 1e-3) / 1e12
            stages[n] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac": round(tf / PEAK_MXFP8_TFLOPS, 4)}
        else:
            gbs = work["bytes"][n] / (ms * 1e-3) / 1e9
            stages[n] = {"ms": round(ms, 4), "gbps": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBPS, 4)}
        tr = measured_traffic("layer." + n)
        stages[n]["traffic"] = None if tr is None else tr["bytes"]
    flops = sum(work["gemm_flops"].values())
    tf = flops / (step_ms * 1e-3) / 1e12
    res = {"workload": "SwiGLU expert FFN layer fwd+bwd from router logits: T=32768 tokens, top-8 of E=64 experts "
                       "(262144 routed rows), hidden 7168, expert ffn 2048, bf16 N(0,1) activations, 0.02*N(0,1) "
                       "weights, MXFP8 GEMM operands, bf16 GEMM outputs",
           "steps": steps, "ms_per_step": round(step_ms, 3), "gemm_tflop_per_step": round(flops / 1e12, 3),
           "tflops": round(tf, 1), "frac": round(tf / PEAK_MXFP8_TFLOPS, 4), "stages": stages}
    # the same layer with the quantize fused into the permute (same bytes out)
    f_ms, f_per, _ = time_stages(lambda n: moe.run_layer_stage(n, b, x, w1, w2, logits, dout),
                                 moe.LAYER_FUSED_STAGES, steps, 2, label="layer_fused.")
    res["fused_quant_permute"] = {
        "ms_per_step": round(f_ms, 3), "tflops": round(flops / (f_ms * 1e-3) / 1e12, 1),
        "stages": {n: {"ms": round(f_per[n], 4), "gbps": round(work["bytes"][n] / (f_per[n] * 1e-3) / 1e9, 1)}
                   for n in ("route", "quant_xperm")},
        "replaces": {n: round(per[n], 4) for n in ("quant_x", "permute", "quant_xt")}}
    graph = None if COUNTER is not None else moe.capture(lambda: moe.layer_step(b, x, w1, w2, logits, dout))
    g_ms = time_graph(graph, steps, 2)
    del graph
    res["graph"] = {"ms_per_step": round(g_ms, 3), "tflops": round(flops / (g_ms * 1e-3) / 1e12, 1)}
    res["bf16_gemms"] = layer_bf16_gemms(args, b, x, w1, w2, per, work)
    del b, x, dout, w1, w2, logits
    torch.cuda.empty_cache()
    return res


def layer_bf16_gemms(args, b, x, w1, w2, mx_per, work):
    """The layer's six grouped GEMMs with bf16 operands (the BF16 baseline),
    over the layer's own routing (group offsets of the MXFP8 run): operands
    are the layer's bf16 tensors, gathered / transposed by mx_bf16_gather
    (X_perm, W1^T, W2^T; the MXFP8 run's bf16 dA, dX_perm and H stand in for
    A, dY and dH).  Each GEMM is timed like the MXFP8 stages and reported
    with the MXFP8 speedup over it."""
    import torch

    import mxfp8_block_scaled_07_amd as mxa

    T, H, F, E, cap = b.T, b.H, b.F, b.E, b.cap
    dev, bf = x.device, torch.bfloat16
    e = lambda *s: torch.empty(s, dtype=bf, device=dev)  # noqa: E731
    xp, xt, w1t, w2t, at, dyt, dht = e(cap, H), e(H, cap), e(E, H, 2 * F), e(E, F, H), e(F, cap), e(H, cap), e(2 * F, cap)
    mxa.mx_bf16_gather(x, 1, T, H, b.src, cap, xp, xt)
    mxa.mx_bf16_gather(w1, E, 2 * F, H, None, 2 * F, None, w1t)
    mxa.mx_bf16_gather(w2, E, H, F, None, H, None, w2t)
    a, dy, dh = b.da, b.dxp, b.h
    mxa.mx_bf16_gather(a, 1, cap, F, None, cap, None, at)
    mxa.mx_bf16_gather(dy, 1, cap, H, None, cap, None, dyt)
    mxa.mx_bf16_gather(dh, 1, cap, 2 * F, None, cap, None, dht)
    o_h, o_y, o_da, o_dw2, o_dx, o_dw1 = e(cap, 2 * F), e(cap, H), e(cap, F), e(E, H, F), e(cap, H), e(E, 2 * F, H)
    out = mxa.MX_OUT_BF16

    def run(n):
        if n == "gemm1_fwd":
            mxa.mx_bf16_grouped_gemm_fwd(xp, w1, b.off, E, cap, 2 * F, H, o_h, out)
        elif n == "gemm2_fwd":
            mxa.mx_bf16_grouped_gemm_fwd(a, w2, b.off, E, cap, H, F, o_y, out)
        elif n == "gemm2_dgrad":
            mxa.mx_bf16_grouped_gemm_dgrad(dy, w2t, b.off, E, cap, F, H, o_da, out)
        elif n == "gemm2_wgrad":
            mxa.mx_bf16_grouped_gemm_wgrad(dyt, at, b.off, E, cap, H, F, o_dw2, out)
        elif n == "gemm1_dgrad":
            mxa.mx_bf16_grouped_gemm_dgrad(dh, w1t, b.off, E, cap, H, 2 * F, o_dx, out)
        else:
            mxa.mx_bf16_grouped_gemm_wgrad(dht, xt, b.off, E, cap, 2 * F, H, o_dw1, out)

    names = ("gemm1_fwd", "gemm2_fwd", "gemm2_dgrad", "gemm2_wgrad", "gemm1_dgrad", "gemm1_wgrad")
    M = T * b.topk   # routed rows: every token goes to topk experts
    counter_work("layer_bf16.", {   # bf16 operands read once, bf16 output written once
        "gemm1_fwd": (M * H + E * 2 * F * H) * 2 + M * 2 * F * 2, "gemm2_fwd": (M * F + E * H * F) * 2 + M * H * 2,
        "gemm2_dgrad": (M * H + E * F * H) * 2 + M * F * 2, "gemm2_wgrad": (H * M + F * M) * 2 + E * H * F * 2,
        "gemm1_dgrad": (M * 2 * F + E * H * 2 * F) * 2 + M * H * 2,
        "gemm1_wgrad": (2 * F * M + H * M) * 2 + E * 2 * F * H * 2})
    torch.cuda.synchronize()
    _, per, _ = time_stages(run, names, max(3, args.steps // 4), 2, label="layer_bf16.")
    stages = {}
    for n in names:
        tf = work["gemm_flops"][n] / (per[n] * 1e-3) / 1e12
        tr = measured_traffic("layer_bf16." + n)
        stages[n] = {"ms": round(per[n], 4), "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "mxfp8_speedup": round(per[n] / mx_per[n], 3), "traffic": None if tr is None else tr["bytes"]}
    tot, mx_tot = sum(per[n] for n in names), sum(mx_per[n] for n in names)
    del xp, xt, w1t, w2t, at, dyt, dht, o_h, o_y, o_da, o_dw2, o_dx, o_dw1
    torch.cuda.empty_cache()
    return {"ms": round(tot, 3), "mxfp8_ms": round(mx_tot, 3), "mxfp8_speedup": round(tot / mx_tot, 3),
            "tflops": round(sum(work["gemm_flops"][n] for n in names) / (tot * 1e-3) / 1e12, 1),
            "peak_bf16_tflops": PEAK_BF16_TFLOPS, "stages": stages,
            "note": "the six grouped GEMMs of the layer on bf16 operands, same routing and kernel design; "
                    "GEMMs only (the layer's glue kernels exist in their MXFP8-fused form only)"}


def copy_calibration():
    """A plain device-to-device copy of CALIB_BYTES, three launches: the
    reference the FETCH_SIZE / WRITE_SIZE counters are scaled by."""
    import torch
    a = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        if COUNTER is not None:
            counter_mark("calibration")
        b.copy_(a)
        if COUNTER is not None:
            counter_mark("other")
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), else the machine type."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(args, c):
    """The oracle, as it stands, on three experts' share of the step (about
    10-20 s of host work)."""
    import numpy as np

    from oracle import gemm as og
    from oracle import mxfp8 as mx
    from oracle import routing

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = None
    E = c["E"]
    t0 = time.perf_counter()
    counts, off, dst, src = routing.route(c["expert_ids"], E, c["capacity"])
    order = np.argsort(counts)
    experts = [int(e) for e in order[len(order) // 2 - 1:len(order) // 2 + 2]]   # three median-sized experts
    m = 0
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        rows_src = src[lo:hi]
        xq, xs = mx.quantize_rowwise(c["x"][np.maximum(rows_src, 0)])
        xpq, xps = routing.permute(xq, xs, np.where(rows_src >= 0, np.arange(hi - lo), -1))
        wq, ws = mx.quantize_rowwise(c["w"][e])
        wtq, wts = mx.quantize_colwise(c["w"][e])
        dy = c["dy_full"][lo:hi].copy()
        dy[rows_src < 0] = 0
        dyq, dys = mx.quantize_rowwise(dy)
        dytq, dyts = mx.quantize_colwise(dy)
        xtq, xts = mx.quantize_colwise(c["x"], rows_out=hi - lo, gather=rows_src)
        goff = np.array([0, hi - lo])
        og.grouped_gemm_fwd(xpq, xps, wq[None], ws[None], goff, want_abs=False)
        og.grouped_gemm_dgrad(dyq, dys, wtq[None], wts[None], goff, want_abs=False)
        og.grouped_gemm_wgrad(dytq, dyts, xtq, xts, goff, want_abs=False)
        m += int(counts[e])
    dt = time.perf_counter() - t0
    flops = 3 * 2.0 * m * c["N"] * c["K"]
    cores = len(os.sched_getaffinity(0))
    # the oracle's fused rowwise + columnwise quantize on a slice of the
    # bandwidth workload's tensor (2048 of its 131072 rows, same recipe)
    import workloads
    qrows, qcols = 2048, 5120
    xq = workloads.quant_tensor(4, qrows, qcols)
    tq = time.perf_counter()
    mx.quantize_rowwise(xq)
    mx.quantize_colwise(xq)
    dq = time.perf_counter() - tq
    qgbps = qrows * qcols * (2 + 2 * (1 + 1 / 32)) / dq / 1e9
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": blas_threads or cores,
            "host_cores": cores, "kind": "oracle", "seconds": round(dt, 2),
            "cpu": cpu_model(),
            "quantize_gbps": round(qgbps, 3), "quantize_seconds": round(dq, 2),
            "quantize_sample": f"oracle rowwise + columnwise quantize of a [{qrows}, {qcols}] slice of the "
                               f"bandwidth workload (same recipe; 4.0625 B per element), one process",
            "sample": f"three median-sized experts ({m} routed rows of 16384): routing of all 8192x2 ids, and "
                      f"per expert the rowwise/colwise quantize of its X rows, W_e and dY rows, its permute and "
                      f"the fp64 fwd/dgrad/wgrad GEMMs (value = their GEMM FLOPs / wall time)"}


# kernel sources behind each stage (the traffic record hashes them)
_CS = "mxfp8_block_scaled_07_amd/csrc/"
_SRC_QUANT = [_CS + "quantize.hip", _CS + "tile_quant.h", _CS + "mx_device.h"]


def stage_sources(label):
    pre, n = label.rsplit(".", 1) if "." in label else ("", label)
    if n.startswith("gemm"):
        return [_CS + "gemm.hip"]
    if n in ("permute", "route"):
        return [_CS + "permute.hip"]
    if pre in ("bf16", "layer_bf16") or n == "permute_bf16" or n.startswith("transpose"):
        return [_CS + "bf16.hip", _CS + "mx_device.h"]
    if n in ("router", "router_bwd"):
        return [_CS + "router.hip", _CS + "mx_device.h"]
    if n in ("swiglu", "swiglu_bwd", "combine", "combine_bwd", "unpermute_dx"):
        return [_CS + "glue.hip", _CS + "tile_quant.h", _CS + "mx_device.h"]
    return _SRC_QUANT


def summarize_counters(fetch_csv, write_csv, log, out_path=TRAFFIC_FILE):
    """Write profiles/hbm_traffic.txt from two counter passes (FETCH_SIZE and
    WRITE_SIZE, one counter each) and the counter pass's printed line: the
    dispatches between two markers are one call of the stage the first marker
    names; a stage's bytes are the mean over its calls of the summed counter
    (KiB) of its dispatches, scaled by what the same counter reads for a plain
    copy of CALIB_BYTES."""
    info = [json.loads(ln) for ln in open(log) if ln.startswith('{"counter_pass"')][-1]["counter_pass"]
    labels, alg = info["labels"], info["algorithmic_bytes"]

    f = {lab: d["FETCH_SIZE"] for lab, d in counter_means(fetch_csv, labels).items() if "FETCH_SIZE" in d}
    w = {lab: d["WRITE_SIZE"] for lab, d in counter_means(write_csv, labels).items() if "WRITE_SIZE" in d}
    ff, fw = CALIB_BYTES / (f["calibration"] * 1024), CALIB_BYTES / (w["calibration"] * 1024)
    cmd = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 900 rocprofv3 --pmc {C} -d $GRAFT_REPO_ROOT/gpurun_out/"
           "pmc_{c} -o run --output-format csv -- python3 $GRAFT_REPO_ROOT/bench.py --counter-pass "
           "> $GRAFT_REPO_ROOT/gpurun_out/pmc_{c}.log")
    out = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE): expert step, large workload",
           "# (T=8192, K=5120, N=8192, E=16, top-2); fused. the same step with the quantize fused into the",
           "# permute; bf16. its BF16 baseline; quant. the quantize-bandwidth tensor [131072, 5120]; layer. the",
           "# SwiGLU expert FFN layer (T=32768, top-8 of E=64, hidden 7168, ffn 2048), layer_fused. with the",
           "# fused permute, layer_bf16. its six GEMMs on bf16 operands.",
           "#",
           "# Commands (from the repository root on one MI355X), one counter per run, then the summary:",
           "#   " + cmd.format(C="FETCH_SIZE", c="fetch"),
           "#   " + cmd.format(C="WRITE_SIZE", c="write"),
           "#   python3 bench.py --summarize-counters gpurun_out/pmc_fetch/run_counter_collection.csv "
           "gpurun_out/pmc_write/run_counter_collection.csv gpurun_out/pmc_fetch.log",
           "#",
           f"# The counter pass runs every stage {info['reps']} times, each call between two marker kernels",
           "#   (one-element int64 fills); a stage's bytes are the mean over its calls of the counter summed",
           "#   over the call's dispatches (KiB) x 1024 x the calibration factor.",
           f"# Calibration: a plain copy of {CALIB_BYTES} bytes reads FETCH_SIZE {f['calibration']:.0f} KiB and",
           f"#   WRITE_SIZE {w['calibration']:.0f} KiB per launch; factors fetch x{ff:.4f}, write x{fw:.4f}.",
           "# algorithmic = bytes the stage must move at least once (moe.algorithmic_work, bf16_work,",
           "#   layer_work); GEMM stages count their operands and bf16 output once.",
           "# sha256 = of the kernel sources (in the order listed) when the counters were taken; bench.py ignores",
           "#   a record whose sources changed.",
           "#"]
    for lab in dict.fromkeys(labels):
        if lab in ("other", "calibration") or lab.startswith("config") or lab not in f or lab not in w:
            continue
        fb, wb = f[lab] * 1024 * ff, w[lab] * 1024 * fw
        srcs = stage_sources(lab)
        digest = hashlib.sha256(b"".join(open(os.path.join(ROOT, x), "rb").read() for x in srcs)).hexdigest()
        a = alg.get(lab)
        ratio = f"{(fb + wb) / a:.3f}" if a else "n/a"
        out.append(f"stage={lab} source={','.join(srcs)} sha256={digest} fetch_bytes={fb:.0f} write_bytes={wb:.0f} "
                   f"algorithmic_bytes={a or 0:.0f} ratio={ratio}")
    open(out_path, "w").write("\n".join(out) + "\n")
    print(f"wrote {out_path}: {len(out)} lines")


GEMM_COUNTER_STAGES = ("gemm_fwd", "gemm_dgrad", "gemm_wgrad", "bf16.gemm_fwd", "bf16.gemm_dgrad", "bf16.gemm_wgrad")
GEMM_COUNTER_SETS = (
    "SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VMEM SQ_VMEM_TA_ADDR_FIFO_FULL "
    "SQ_VMEM_TA_CMD_FIFO_FULL SQ_LDS_BANK_CONFLICT TA_BUSY_avr TA_ADDR_STALLED_BY_TC_CYCLES_sum GRBM_GUI_ACTIVE",
    "TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum TCC_TAG_STALL_sum TCP_TCR_TCP_STALL_CYCLES_sum "
    "TCP_PENDING_STALL_CYCLES_sum TCP_UTCL1_TRANSLATION_MISS_sum TCP_UTCL1_TRANSLATION_HIT_sum TD_TD_BUSY_sum "
    "TD_TC_STALL_sum GRBM_GUI_ACTIVE")


def counter_means(path, labels):
    """{label: {counter: mean over the label's calls of the counter summed over the call's dispatches}} from
    a --pmc CSV of a counter pass (marker kernels delimit the calls)."""
    import csv
    import statistics
    rows = sorted(csv.DictReader(open(path)), key=lambda r: (int(r["Dispatch_Id"]), r["Counter_Name"]))
    calls, cur, n_mark, last = {}, None, 0, None
    for r in rows:
        if MARKER_KERNEL in r["Kernel_Name"]:
            if r["Dispatch_Id"] == last:
                continue
            last = r["Dispatch_Id"]
            if n_mark == len(labels):
                raise SystemExit(f"{path}: more marker dispatches than the {len(labels)} labels")
            if cur is not None:
                for k, v in cur[1].items():
                    calls.setdefault(cur[0], {}).setdefault(k, []).append(v)
            cur = (labels[n_mark], {})
            n_mark += 1
        elif cur is not None:
            cur[1][r["Counter_Name"]] = cur[1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if cur is not None:
        for k, v in cur[1].items():
            calls.setdefault(cur[0], {}).setdefault(k, []).append(v)
    if n_mark != len(labels):
        raise SystemExit(f"{path}: {n_mark} marker dispatches for {len(labels)} labels")
    return {lab: {k: statistics.fmean(v) for k, v in d.items()} for lab, d in calls.items()}


def summarize_gemm_counters(log, csvs, out_path):
    """Write the GEMM hardware-counter table (profiles/gemm_counters.md) from
    counter passes of the expert step (one CSV per counter set)."""
    info = [json.loads(ln) for ln in open(log) if ln.startswith('{"counter_pass"')][-1]["counter_pass"]
    m = {}
    for path in csvs:
        for lab, d in counter_means(path, info["labels"]).items():
            m.setdefault(lab, {}).update(d)
    st = GEMM_COUNTER_STAGES
    names = sorted({k for lab in st for k in m.get(lab, {})})
    cmd = ("timeout -s KILL 300 rocprofv3 --pmc {C} -d $GRAFT_REPO_ROOT/gpurun_out/gemm_pmc{i} -o run --output-format "
           "csv -- python3 $GRAFT_REPO_ROOT/bench.py --counter-pass --no-layer --no-quant-bench "
           "> $GRAFT_REPO_ROOT/gpurun_out/gemm_pmc{i}.log")
    out = ["# Hardware counters: grouped GEMMs of the expert step, large workload (T=8192, K=5120, N=8192, E=16, "
           "top-2), MXFP8 and its BF16 baseline", "",
           f"Mean counter value per call over the counter pass's {info['reps']} calls of each stage (rocprofv3 sums "
           "over hardware instances; SQ counts in the units it reports). Calls are delimited by the counter pass's "
           "marker kernels. Commands (from the repository root on one MI355X; one --pmc pass per counter set), then "
           "the summary:", "", "```", "cd /tmp && export TMPDIR=/tmp"]
    out += [cmd.format(C=c, i=i + 1) for i, c in enumerate(GEMM_COUNTER_SETS)]
    out += ["cd $GRAFT_REPO_ROOT && python3 bench.py --summarize-gemm-counters gpurun_out/gemm_pmc1.log "
            "gpurun_out/gemm_pmc1/run_counter_collection.csv gpurun_out/gemm_pmc2/run_counter_collection.csv", "```",
            "", "| counter | " + " | ".join(st) + " |", "|---|" + "---:|" * len(st)]
    for k in names:
        out.append(f"| {k} | " + " | ".join(f"{m.get(lab, {}).get(k, float('nan')):.4g}" for lab in st) + " |")

    def der(lab, f):
        d = m.get(lab, {})
        try:
            return f"{f(d):.2f}"
        except (KeyError, ZeroDivisionError):
            return "n/a"
    rows = [("MFMA busy", lambda d: d["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / (d["GRBM_GUI_ACTIVE"] / 8)),
            ("L2 hit rate", lambda d: d["TCC_HIT_sum"] / (d["TCC_HIT_sum"] + d["TCC_MISS_sum"])),
            ("TD busy", lambda d: d["TD_TD_BUSY_sum"] / 256 / (d["GRBM_GUI_ACTIVE"] / 8)),
            ("TD stalled on L1-L2", lambda d: d["TD_TC_STALL_sum"] / 256 / (d["GRBM_GUI_ACTIVE"] / 8))]
    out += ["", "Derived (SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (GRBM_GUI_ACTIVE / 8 XCDs); TCC_HIT / (TCC_HIT + "
            "TCC_MISS); TD_TD_BUSY and TD_TC_STALL / 256 CUs / (GRBM_GUI_ACTIVE / 8)):", "",
            "| | " + " | ".join(st) + " |", "|---|" + "---:|" * len(st)]
    for name, f in rows:
        out.append(f"| {name} | " + " | ".join(der(lab, f) for lab in st) + " |")
    out += ["", "Notes:",
            "- A bf16 32x32x16 MFMA does a quarter of the work of a scaled FP8 32x32x64 MFMA in half its cycles, so "
            "the bf16 GEMMs count twice the MFMA busy cycles for the same FLOPs (the 2:1 ratio of the two dense "
            "peaks).",
            "- MFMA busy includes the MFMAs of padding rows (the ~1092-row groups fill 5 m-tiles of 256 to 85%) and "
            "of the wgrad ring's padding steps.",
            "- Under the counter pass the kernels run serialized, one call at a time; their durations are not the "
            "bench's.", ""]
    open(out_path, "w").write("\n".join(out))
    print(f"wrote {out_path}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=70)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quant-bench", action="store_true")
    ap.add_argument("--no-layer", action="store_true", help="skip the SwiGLU expert FFN layer workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--no-small-configs", action="store_true", help="skip the tiny and mid workloads")
    ap.add_argument("--counter-pass", action="store_true",
                    help="run every stage a few times between marker kernels, for per-stage hardware counters "
                         "(rocprofv3 --pmc); prints the stage labels instead of timings")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "LOG"),
                    help="write profiles/hbm_traffic.txt from two counter passes (no GPU needed)")
    ap.add_argument("--summarize-gemm-counters", nargs="+", metavar="LOG_THEN_CSVS",
                    help="write profiles/gemm_counters.md from a counter pass's log and its --pmc CSVs")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_gemm_counters:
        summarize_gemm_counters(args.summarize_gemm_counters[0], args.summarize_gemm_counters[1:],
                                os.path.join(ROOT, "profiles", "gemm_counters.md"))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the expert path has no multi-GPU leg "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    ensure_built()
    import workloads
    c = workloads.config(3)
    if args.counter_pass:
        import torch
        global COUNTER
        COUNTER = {"labels": [], "alg": {}, "marker": torch.empty(1, dtype=torch.int64, device="cuda:0")}
        ceil = {"hbm_copy_gbps": 1.0, "quant_pattern_gbps": 1.0, "mfma_mxfp8_tflops": 1.0,
                "mfma_mxfp8_tflops_constant_operands": 1.0}
    else:
        ceil = measure_ceilings()
    res = gpu_expert_path(args, c, ceil)
    line = {
        "metric": METRIC, "value": round(res["value"], 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "mxfp8", "data": "synthetic",
        "config": res["config"], "roofline": res["roofline"], "stages": res["stages"],
        "fused_quant_permute": res["fused_quant_permute"], "graph": res["graph"],
        "bf16_baseline": res["bf16_baseline"], "ceilings": ceil, "stages_mall_flushed": res["stages_mall_flushed"],
    }
    if not args.no_quant_bench:
        line["quantize_bandwidth"] = gpu_quantize_bandwidth(args, ceil)
    if not (args.no_small_configs or args.counter_pass):
        line["small_configs"] = gpu_small_configs(args, ceil)
    if not args.no_layer:
        line["swiglu_layer"] = gpu_swiglu_layer(args)
    if args.copy_calibration or args.counter_pass:
        copy_calibration()
    if args.counter_pass:
        print(json.dumps({"counter_pass": {"labels": COUNTER["labels"], "reps": COUNTER_REPS,
                                           "algorithmic_bytes": COUNTER["alg"]}}), flush=True)
        return
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args, c)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
