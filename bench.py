#!/usr/bin/env python3
"""Throughput of the routed MoE FFN forward pass on one MI355X.

One step = one moe_forward over a batch of synthetic tokens: router product, gate,
statistics, capacity, dispatch, routed expert FFNs, shared experts, combine.  The
default workload is the Mixtral-shaped layer (4096 tokens, d 4096, 8 SwiGLU experts of
width 14336, top-2, bf16), the one the layer's throughput targets are stated on; other
workloads can be chosen with --config.

Prints one JSON line: tokens/s over the timed steps, per-stage times from HIP events
recorded by the library on the launch stream, the roofline position of the dominant
kernel, and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # dense MFMA, MI355X
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0
METRIC = "MoE-layer tokens/s; grouped-GEMM TFLOP/s & % of MFMA peak; dispatch GB/s"
STAGES = ["route", "dispatch", "gemm1", "gemm2", "shared", "combine"]
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "sparse_mixture_experts_forward_amd", "csrc")
# kernel symbol of each stage's launch, as rocprofv3 names it (bf16 workloads)
PACKED_ROWS = 256  # segments averaging this many rows take the packed-weight kernel
CALIB_KERNEL = "MulFunctor"  # the plain float32 copy (x * 1) that scales byte counters


# The sources of the expert GEMM kernels, whose counter-derived traffic the bench reports:
# gemm.hip, common.h and the grouped-GEMM part of kernels.h.
GEMM_SOURCES = ("common.h", "gemm.hip", "kernels.h")
GEMM_HEADER_PART = ("// ---------------------------------------------------------------- grouped GEMM",
                    "// ---------------------------------------------------------------- combine")


def sources_hash() -> str:
    """Hash of the expert GEMM's sources: stored with counter-derived traffic, which is
    reported only while those kernels are unchanged."""
    h = hashlib.sha256()
    for f in sorted(os.path.join(CSRC, n) for n in GEMM_SOURCES):
        with open(f, "rb") as fh:
            text = fh.read()
        if os.path.basename(f) == "kernels.h":
            a, b = (p.encode() for p in GEMM_HEADER_PART)
            text = text[text.index(a):text.index(b)]
        h.update(os.path.basename(f).encode() + text)
    return h.hexdigest()[:16]


SMALL_ROWS = 48  # below this the library takes 32-row tiles


def _avg_rows(cfg, capacity: int) -> int:
    """The library's bound on the kept rows per expert (what picks its GEMM kernels)."""
    rows = cfg.n_tokens * cfg.top_k
    if capacity >= 0:
        rows = min(rows, capacity * cfg.n_experts)
    return rows // cfg.n_experts


def packed_path(cfg, capacity: int, packed: bool) -> bool:
    """Whether the routed expert products read packed weights: every bf16 workload (the
    library then runs a packed-weight kernel for every segment length)."""
    return bool(packed) and cfg.dtype == "bf16"


def _grid_for(max_rows: int, n_seg: int, bm: int, n_ntiles: int) -> int:
    t = (-(-max_rows // bm) + n_seg) * n_ntiles
    return -(-t // 8) * 8


def _f32_tile(cfg, stage: str, capacity: int) -> int:
    """The float32 product's tile side: 64 where 64 x 64 tiles give 512 workgroups or
    more by the library's row bound, else 32."""
    rows = cfg.n_tokens * cfg.top_k
    if capacity >= 0:
        rows = min(rows, capacity * cfg.n_experts)
    n_out = cfg.d_ff if stage == "gemm1" else cfg.d_model
    return 64 if _grid_for(rows, cfg.n_experts, 64, -(-n_out // 64)) >= 512 else 32


def stage_symbol(cfg, stage: str, packed: bool = False, capacity: int = -1):
    """The kernel of a GEMM stage's launch.  (With a capacity limit and a row bound of
    SMALL_ROWS or more per expert, the dispatch picks the tile height on the device; the
    name given is then that of the taller tiles.)"""
    epi = {"gemm1": 2 if cfg.act == "swiglu" else 1, "gemm2": 0}.get(stage)
    if epi is None:
        return None
    if cfg.dtype != "bf16":
        return f"gemm_f32_kernel<{epi}, false, {_f32_tile(cfg, stage, capacity)}>"
    avg = _avg_rows(cfg, capacity)
    if avg < SMALL_ROWS:
        return f"gemm_packed_small_kernel<{epi}>" if packed else f"gemm_bf16_kernel<32, {epi}, false>"
    if packed:
        shape = "128, 8, 8, 0" if avg >= PACKED_ROWS else "256, 16, 4, 1"
        return f"gemm_packed_kernel<PackedShape<{shape}>, {epi}>"
    return f"gemm_bf16_kernel<256, {epi}, false>"


def _pmc_rows(path: str):
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _counter_values(path: str, counter: str) -> dict:
    """{kernel name: [value per dispatch]}, names without the library's namespaces."""
    vals = {}
    for r in _pmc_rows(path):
        if r["Counter_Name"] == counter:
            name = r["Kernel_Name"].replace("moe::(anonymous namespace)::", "")
            vals.setdefault(name, []).append(float(r["Counter_Value"]))
    return vals


def digest_pmc(cfg_name: str, dirs, calib_mib: int) -> dict:
    """Per-dispatch HBM bytes of each stage kernel from rocprofv3 --pmc runs of this
    bench (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the same
    counter reads for the plain copy kernel (--calibrate-copy-mib, its own run) that
    reads and writes calib_mib MiB once.  dirs = (fetch, write, calib_fetch,
    calib_write)."""
    from sparse_mixture_experts_forward_amd import CONFIGS

    cfg = CONFIGS[cfg_name]
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = dirs
    out = {"config": cfg_name, "sources": sources_hash(), "calib_bytes": calib_mib << 20,
           "kernels": {}}
    per = {}
    for counter, path, cpath in (("FETCH_SIZE", fetch_dir, cfetch_dir),
                                 ("WRITE_SIZE", write_dir, cwrite_dir)):
        vals = _counter_values(path, counter)
        calib = [v for name, vs in _counter_values(cpath, counter).items()
                 if CALIB_KERNEL in name for v in vs]
        if len(calib) != 1:
            raise SystemExit(f"expected one {CALIB_KERNEL} dispatch with {counter} in {cpath}")
        scale = (calib_mib << 20) / (calib[0] * 1024.0)  # bytes per counted byte
        per[counter] = (vals, scale)
        out[counter.lower() + "_calib_kib"] = calib[0]
        out[counter.lower() + "_scale"] = round(scale, 4)
    for stage in STAGES:
        syms = [x for x in (stage_symbol(cfg, stage, True), stage_symbol(cfg, stage)) if x]
        if not syms:
            continue
        # the packed-weight kernel where the profiled run used it, else the staged one
        sym = next((x for x in syms
                    if any(x in name for name in per["FETCH_SIZE"][0])), syms[-1])
        rec = {}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            vals, scale = per[counter]
            got = [v for name, vs in vals.items() if sym in name for v in vs]
            if got:
                rec[counter.lower() + "_bytes"] = round(sum(got) / len(got) * 1024.0 * scale)
                rec["dispatches"] = len(got)
        if rec:
            rec["symbol"] = sym
            out["kernels"][stage] = rec
    return out


def stored_traffic(cfg_name: str, stage: str, symbol: str):
    """HBM bytes per launch of a stage kernel from the committed counter digest, or None
    if there is none, it was taken of another kernel, or the kernels changed since."""
    path = os.path.join(PROFILES, f"traffic_{cfg_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("sources") != sources_hash():
        return None
    k = d.get("kernels", {}).get(stage)
    if not k or "fetch_size_bytes" not in k or "write_size_bytes" not in k:
        return None
    if k.get("symbol") != symbol:
        return None
    return k["fetch_size_bytes"] + k["write_size_bytes"]


def describe(cfg) -> str:
    s = (f"{cfg.name}: N={cfg.n_tokens} d={cfg.d_model} E={cfg.n_experts} k={cfg.top_k} "
         f"{cfg.act} d_ff={cfg.d_ff} {cfg.dtype}")
    if cfg.n_shared:
        s += f" +{cfg.n_shared} shared"
    if cfg.alpha:
        s += f" capacity_factor={cfg.alpha}"
    if cfg.logit_bias != "none":
        s += f" logit_bias={cfg.logit_bias}"
    if cfg.bias_selection_only:
        s += " (bias for selection only)"
    if cfg.capacity_rule != "fixed":
        s += f" capacity_rule={cfg.capacity_rule}"
    if cfg.reroute_rounds:
        s += f" overflow re-routed in up to {cfg.reroute_rounds} rounds"
    return s


def kernel_work(cfg, kept: int, touched: int):
    """Algorithmic flops and HBM bytes of each stage (padding and dropped rows excluded)."""
    es = 2 if cfg.dtype == "bf16" else 4
    n, d, f, k = cfg.n_tokens, cfg.d_model, cfg.d_ff, cfg.top_k
    m1 = 2 if cfg.act == "swiglu" else 1
    sh = cfg.n_shared
    w = {}
    w["gemm1"] = dict(flops=2.0 * kept * d * f * m1,
                      bytes=touched * m1 * f * d * es + kept * d * es + kept * f * es)
    w["gemm2"] = dict(flops=2.0 * kept * f * d,
                      bytes=touched * d * f * es + kept * f * es + kept * d * es)
    w["shared"] = dict(flops=2.0 * n * d * f * sh * (m1 + 1),
                       bytes=(sh * (m1 + 1) * f * d * es + n * d * es * 2 + n * sh * f * es * 2)
                       if sh else 0)
    scatter = bool(cfg.fuse & 4) and k == 1 and sh == 0
    gather, wscale = bool(cfg.fuse & 1), bool(cfg.fuse & 2) or scatter
    # dispatch: ids in, slot map out, row map (and row weights) out; the row copy of x
    # only without the gather fusion; with the scatter fusion the output rows of tokens
    # whose slot was dropped are zeroed
    w["dispatch"] = dict(flops=0.0, bytes=n * k * 4 * 2 + kept * 4 + (kept * 8 if wscale else 0)
                         + (0 if gather else n * d * es + kept * d * es)
                         + ((n - kept) * d * es if scatter else 0))
    w["combine"] = dict(flops=0.0, bytes=0 if scatter else
                        kept * d * es + n * k * (4 if wscale else 8) + n * d * es * (2 if sh else 1))
    w["route"] = dict(flops=2.0 * n * d * cfg.n_experts,
                      bytes=n * d * es + d * cfg.n_experts * 4 + n * (cfg.n_experts * 4 + k * 8))
    return w


def roofline(name, work, ms, dtype):
    peak_f = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_F32_TFLOPS
    ridge = peak_f * 1e12 / (PEAK_HBM_GBPS * 1e9)
    fl, by = work["flops"], work["bytes"]
    if fl > 0 and fl / by >= ridge:
        ach = fl / (ms * 1e-3) / 1e12
        return dict(kernel=name, bound="mfma", achieved=round(ach, 2), peak=peak_f, unit="TFLOP/s",
                    frac=round(ach / peak_f, 4), traffic=None, avg_ms=round(ms, 5),
                    algorithmic_flops=fl, algorithmic_bytes=by)
    ach = by / (ms * 1e-3) / 1e9
    return dict(kernel=name, bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                frac=round(ach / PEAK_HBM_GBPS, 4), traffic=None, avg_ms=round(ms, 5),
                algorithmic_flops=fl, algorithmic_bytes=by)


def cpu_baseline(cfg, inp, logits, budget_s: float):
    """The CPU oracle, as it stands, on the first n_s tokens of the same inputs (routing
    and capacity over every token), n_s sized to about budget_s seconds."""
    import numpy as np

    import oracle as O

    def host(t):
        t = t.detach().contiguous()
        if str(t.dtype) == "torch.bfloat16":
            import torch

            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    x = host(inp.x)
    lb = None if inp.logit_bias is None else host(inp.logit_bias)
    wr = host(inp.w_router)
    raw = {}
    for e in range(cfg.n_experts):  # staging copies to host memory: not timed
        raw[e] = {k: host(getattr(inp, k)[e]) for k in ("w1", "w2", "w3", "b1", "b2")
                  if getattr(inp, k) is not None}
    sraw = {}
    for s in range(cfg.n_shared):
        sraw[s] = {k: host(getattr(inp, "s" + k)[s]) for k in ("w1", "w2", "w3")
                   if getattr(inp, "s" + k) is not None}

    def widen_expert(w):
        return O.ExpertWeights(**{k: O.widen(v, cfg.dtype) for k, v in w.items()})

    def run(n_s):
        t0 = time.perf_counter()
        O.forward(x, cfg.dtype, wr, cfg.top_k, lambda e: widen_expert(raw[e]), cfg.n_experts,
                  cfg.act, logit_bias=lb, alpha=cfg.alpha, renormalize=cfg.renormalize,
                  bias_selection_only=cfg.bias_selection_only,
                  capacity_rule=cfg.capacity_rule, reroute_rounds=cfg.reroute_rounds,
                  shared=(lambda s: widen_expert(sraw[s])) if cfg.n_shared else None,
                  n_shared=cfg.n_shared, tokens=np.arange(n_s))
        return time.perf_counter() - t0

    n = cfg.n_tokens
    n_s = min(n, 16)
    t = run(n_s)
    while t < budget_s / 4 and n_s < n:  # the first runs are dominated by fixed costs
        n_s = min(n, n_s * 4)
        t = run(n_s)
    if t < 0.6 * budget_s and n_s < n:
        n_s = int(min(n, max(n_s, n_s * 0.8 * budget_s / t)))
        t = run(n_s)
    # the whole workload in less than the budget: time further whole passes (at most
    # four in all) and report their mean
    passes = 1
    while n_s == n and passes < 4 and t * (passes + 1) / passes <= budget_s:
        t += run(n_s)
        passes += 1
    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    what = (f"all {n} tokens, {passes} passes" if passes > 1 else
            f"first {n_s} of {n} tokens (router product, gate and capacity over all {n})")
    return dict(value=round(n_s * passes / t, 2), unit="tokens/s", cores=int(cores),
                kind="oracle", sample=f"{what}; float64 numpy; {t:.1f} s",
                seconds=round(t, 2))


def dispatch_copy(layer, x, topk_idx, kept: int, reps: int = 20) -> dict:
    """The permuted copy of x that the gather fusion removes, measured through the C
    ABI: moe_dispatch with and without the copy (preallocated buffers, HIP events
    around each call on the launch stream); the difference of the medians is the
    copy's cost, its algorithmic bytes x read once plus the kept rows written."""
    import torch

    from sparse_mixture_experts_forward_amd import _binding as B
    from sparse_mixture_experts_forward_amd.layer import workspace

    cfg = layer.cfg
    n, k = topk_idx.shape
    dev = x.device
    i32 = torch.int32
    offsets = torch.empty(cfg.n_experts + 1, dtype=i32, device=dev)
    row_token = torch.empty(max(n * k, 1), dtype=i32, device=dev)
    slot_row = torch.empty((n, k), dtype=i32, device=dev)
    kept_count = torch.empty(cfg.n_experts, dtype=i32, device=dev)
    dropped = torch.empty(1, dtype=i32, device=dev)
    x_perm = torch.empty((max(n * k, 1), x.shape[1]), dtype=x.dtype, device=dev)
    ws = workspace(B.moe_dispatch_workspace_size(n, k, cfg.n_experts), dev)
    cap = layer.capacity(n)

    def timed(with_copy):
        times = []
        for _ in range(reps + 3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            B.moe_dispatch(topk_idx, cfg.n_experts, cap, x if with_copy else None, offsets,
                           row_token, slot_row, kept_count, dropped,
                           x_perm if with_copy else None, ws)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        times = sorted(times[3:])
        return times[len(times) // 2]

    with_ms, without_ms = timed(True), timed(False)
    es = x.element_size()
    nbytes = n * x.shape[1] * es + kept * x.shape[1] * es
    copy_ms = max(with_ms - without_ms, 1e-6)
    gbps = nbytes / (copy_ms * 1e-3) / 1e9
    return {"dispatch_with_copy_ms": round(with_ms, 5), "dispatch_index_maps_ms": round(without_ms, 5),
            "copy_ms": round(copy_ms, 5), "copy_bytes": nbytes, "copy_gbps": round(gbps, 1),
            "copy_frac_of_hbm": round(gbps / PEAK_HBM_GBPS, 4),
            "stage_gbps_with_copy": round((nbytes + n * k * 8) / (with_ms * 1e-3) / 1e9, 1),
            "note": "standalone moe_dispatch with the permuted copy of x (what the default "
                    "gather fusion skips); copy = with minus without, medians of "
                    f"{reps} calls"}


def _median(v):
    v = sorted(v)
    return v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])


def measure(cfg, dev, steps: int, warmup: int, pack: bool, cold: bool = True) -> dict:
    """Times `steps` moe_forward calls of one workload (after `warmup` untimed ones) on
    inputs resident in HBM: wall clock over the steps, per-stage HIP events recorded by
    the library on the launch stream, the roofline position of every stage kernel.
    With packed weights (where the library's bound picks a packed-weight kernel, i.e.
    every bf16 workload) the routed experts' weights are packed once before the warmup
    and the layer keeps only the packed copy."""
    import torch

    from sparse_mixture_experts_forward_amd import MoELayer, synth
    from sparse_mixture_experts_forward_amd import _binding as B

    inp = synth.DeviceInputs(cfg, dev)
    layer = MoELayer.from_inputs(inp)
    n = cfg.n_tokens
    cap = layer.capacity(n)
    use_packed = packed_path(cfg, cap, pack)
    pack_ms = None
    if use_packed:
        torch.cuda.synchronize()
        tp = time.perf_counter()
        layer.pack_weights(drop_unpacked=True)
        torch.cuda.synchronize()
        pack_ms = (time.perf_counter() - tp) * 1e3
    stats = layer.new_stats(n)
    y = torch.empty_like(inp.x)

    for _ in range(warmup):
        layer.forward(inp.x, y, stats)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(B.MOE_N_STAGE_EVENTS)]
          for _ in range(steps)]
    for row in ev:  # create the events
        for e in row:
            e.record()
    torch.cuda.synchronize()
    handles = [[e.cuda_event for e in row] for row in ev]

    # the timed steps: the layer as a caller runs it, nothing recorded between its launches
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        layer.forward(inp.x, y, stats)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # attribution pass: the same steps with HIP events at the stage boundaries, recorded
    # by the library on the launch stream (each record costs a few microseconds of GPU
    # time, so they stay out of the timed steps)
    for i in range(steps):
        layer.forward(inp.x, y, stats, stage_events=handles[i])
    torch.cuda.synchronize()
    step_gpu_ms = sum(ev[i][0].elapsed_time(ev[i][-1]) for i in range(steps)) / steps
    if cfg.n_shared > 0:
        # the shared experts overlap the routed ones in the timed steps; for per-stage
        # times a second pass runs them after the routed experts, on the same stream
        for i in range(steps):
            layer.forward(inp.x, y, stats, stage_events=handles[i], concurrent_shared=False)
        torch.cuda.synchronize()
    stage_ms = {s: 0.0 for s in STAGES}
    stage_all = {s: [] for s in STAGES}
    for row in ev:
        for j, s in enumerate(STAGES):
            t = row[j].elapsed_time(row[j + 1])
            stage_ms[s] += t / steps
            stage_all[s].append(t)

    cold_out = None
    if cold:
        # each step preceded by a 1 GiB scratch write (outside the stage events)
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cold_all = {s: [] for s in STAGES}
        cold_step = []
        for row in ev:
            scratch.fill_(1.0)
            layer.forward(inp.x, y, stats, stage_events=[e.cuda_event for e in row])
        torch.cuda.synchronize()
        for row in ev:
            for j, s in enumerate(STAGES):
                cold_all[s].append(row[j].elapsed_time(row[j + 1]))
            cold_step.append(row[0].elapsed_time(row[-1]))
        del scratch
        cold_out = {"step_ms_median": round(_median(cold_step), 4),
                    "stages_ms_median": {s: round(_median(v), 5) for s, v in cold_all.items()}}

    kept = int(stats["kept_count"].sum().item())
    touched = int((stats["kept_count"] > 0).sum().item())
    work = kernel_work(cfg, kept, touched)
    kernels = {s: roofline(s, work[s], stage_ms[s], cfg.dtype) for s in STAGES
               if stage_ms[s] > 0 and (work[s]["flops"] > 0 or work[s]["bytes"] > 0)}
    for s, r in kernels.items():
        r["symbol"] = stage_symbol(cfg, s, use_packed, cap)
        r["traffic"] = stored_traffic(cfg.name, s, r["symbol"])
    dominant = max(kernels, key=lambda s: stage_ms[s])
    gemm_ms = stage_ms["gemm1"] + stage_ms["gemm2"] + stage_ms["shared"]
    gemm_flops = work["gemm1"]["flops"] + work["gemm2"]["flops"] + work["shared"]["flops"]
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12 if gemm_ms > 0 else 0.0
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    disp_gbps = work["dispatch"]["bytes"] / (stage_ms["dispatch"] * 1e-3) / 1e9
    comb_gbps = (work["combine"]["bytes"] / (stage_ms["combine"] * 1e-3) / 1e9
                 if stage_ms["combine"] > 0 else None)
    ms_step = elapsed / steps * 1e3
    # weights of the experts that kept a row, once per step: what a weight-bound step
    # must stream from HBM at least
    es = 2 if cfg.dtype == "bf16" else 4
    m1 = 3 if cfg.act == "swiglu" else 2
    touched_bytes = touched * m1 * cfg.d_model * cfg.d_ff * es
    routed_ms = stage_ms["gemm1"] + stage_ms["gemm2"]
    out = {
        "tokens_per_s": round(n * steps / elapsed, 1),
        "ms_per_step": round(ms_step, 4),
        "config": {"workload": describe(cfg), "n_tokens": n, "d_model": cfg.d_model,
                   "d_ff": cfg.d_ff, "n_experts": cfg.n_experts, "top_k": cfg.top_k,
                   "n_shared": cfg.n_shared, "capacity_factor": cfg.alpha,
                   "kept_rows": kept, "experts_touched": touched, "capacity": cap,
                   "n_rerouted": int(stats["n_rerouted"].item()), "fuse": cfg.fuse,
                   "packed_weights": use_packed,
                   "pack_ms_once": None if pack_ms is None else round(pack_ms, 2),
                   "resident_weight_bytes": layer.resident_weight_bytes()},
        "roofline": kernels[dominant],
        "grouped_gemm_tflops": round(gemm_tflops, 2),
        "grouped_gemm_frac_of_peak": round(gemm_tflops / peak, 4),
        "touched_weight_bytes": touched_bytes,
        "touched_weight_gbps_step": round(touched_bytes / (ms_step * 1e-3) / 1e9, 1),
        "touched_weight_gbps_routed_gemms": (round(touched_bytes / (routed_ms * 1e-3) / 1e9, 1)
                                             if routed_ms > 0 else None),
        "touched_weight_frac_of_hbm_step": round(touched_bytes / (ms_step * 1e-3) / 1e9
                                                 / PEAK_HBM_GBPS, 4),
        "dispatch_gbps": round(disp_gbps, 1),
        "dispatch_frac_of_hbm": round(disp_gbps / PEAK_HBM_GBPS, 4),
        "dispatch_note": ("index maps only (capacity ranks, slot and row maps): the kept rows "
                          "of x are gathered inside gemm1, so no row is copied"
                          if cfg.fuse & 1 else
                          "index maps and the permuted copy of the kept rows of x"),
        "combine_gbps": None if comb_gbps is None else round(comb_gbps, 1),
        "stages_ms": {s: round(v, 5) for s, v in stage_ms.items()},
        "stages_note": ("stage times from an attribution pass with the shared experts after "
                        "the routed ones on one stream (the timed steps overlap them and "
                        "record no events)"
                        if cfg.n_shared > 0 else
                        "stage times from an attribution pass of the same steps with HIP "
                        "events at the stage boundaries (the timed steps record none)"),
        "stages_ms_median": {s: round(_median(v), 5) for s, v in stage_all.items()},
        "step_gpu_ms_events": round(step_gpu_ms, 4),
        "kernels": kernels,
        "_layer": layer, "_inputs": inp, "_stats": stats,
    }
    if cold_out is not None:
        cm = cold_out["stages_ms_median"]
        cold_out["dispatch_gbps"] = round(work["dispatch"]["bytes"] / (cm["dispatch"] * 1e-3) / 1e9, 1)
        if cm["combine"] > 0:
            cold_out["combine_gbps"] = round(work["combine"]["bytes"] / (cm["combine"] * 1e-3) / 1e9, 1)
        out["cold"] = cold_out
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-dispatch-copy", action="store_true",
                    help="skip the standalone timing of the permuted copy of x")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tokens", type=int, default=0,
                    help="override the workload's batch (tokens); 0 keeps it")
    ap.add_argument("--no-pack", action="store_true",
                    help="do not pack the routed experts' weights (bf16): the expert "
                         "products then stage both operands through LDS")
    ap.add_argument("--bias-selection-only", action="store_true",
                    help="the logit bias steers selection only (weights from the unbiased "
                         "softmax)")
    ap.add_argument("--reroute-rounds", type=int, default=0,
                    help="re-route overflow to the next preferred experts with room")
    ap.add_argument("--capacity-rule", choices=["fixed", "linear", "log"], default="fixed",
                    help="capacity from the factor, or the batch-dependent rules")
    ap.add_argument("--fuse", type=int, default=None,
                    help="fusion bitmask (1 gather x rows in GEMM1, 2 routing weights in "
                         "GEMM2's epilogue, 4 top-1 rows written straight to the output); "
                         "default: the workload's own")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache pass (a 1 GiB scratch write before each step "
                         "evicts L2 and the 256 MB Infinity Cache; stage times only)")
    ap.add_argument("--workloads", default="switch,deepseek,decode,tiny",
                    help="comma-separated further workloads measured after the headline one "
                         "(each with its own timed steps, no CPU baseline); empty: none")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run only one plain device copy (float32 x * 1) of this many MiB: "
                         "the reference kernel that scales hardware byte counters")
    ap.add_argument("--digest-pmc", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "CALIB_FETCH_DIR", "CALIB_WRITE_DIR"),
                    help="no GPU work: turn rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "this bench and of --calibrate-copy-mib into "
                         "profiles/traffic_<config>.json")
    args = ap.parse_args()
    if args.digest_pmc:
        d = digest_pmc(args.config, args.digest_pmc, args.calibrate_copy_mib or 1024)
        os.makedirs(PROFILES, exist_ok=True)
        with open(os.path.join(PROFILES, f"traffic_{args.config}.json"), "w") as fh:
            json.dump(d, fh, indent=1)
            fh.write("\n")
        print(json.dumps(d))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the layer is measured on a single MI355X); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy_mib > 0:
        # one elementwise kernel that reads and writes calibrate_copy_mib MiB once
        dev = torch.device("cuda:0")
        src = torch.ones((args.calibrate_copy_mib << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": args.calibrate_copy_mib << 20}))
        return

    from sparse_mixture_experts_forward_amd import CONFIGS
    from sparse_mixture_experts_forward_amd import _binding as B

    B.lib()  # fails loudly if the HIP library is not built
    cfg = CONFIGS[args.config]
    if args.tokens > 0:
        cfg = cfg.with_tokens(args.tokens)
    if args.bias_selection_only:
        cfg = cfg.scaled(bias_selection_only=True)
    if args.fuse is not None:
        cfg = cfg.scaled(fuse=args.fuse)
    if args.reroute_rounds or args.capacity_rule != "fixed":
        cfg = cfg.scaled(reroute_rounds=args.reroute_rounds, capacity_rule=args.capacity_rule)
    dev = torch.device("cuda:0")
    m = measure(cfg, dev, args.steps, args.warmup, not args.no_pack, cold=not args.no_cold)
    layer, inp, stats = m.pop("_layer"), m.pop("_inputs"), m.pop("_stats")
    n = cfg.n_tokens
    kept = m["config"]["kept_rows"]
    out = {
        "metric": METRIC,
        "value": m["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded counter-based generator; x ~ N(0,1), weights ~ N(0,1/fan_in))",
    }
    out.update({k: v for k, v in m.items() if k not in ("tokens_per_s", "ms_per_step")})
    if cfg.fuse & 1 and n > 0 and not args.no_dispatch_copy:
        out["dispatch_copy"] = dispatch_copy(layer, inp.x, stats["topk_idx"], kept)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, stats["logits"], args.cpu_seconds)
    del layer, inp, stats
    torch.cuda.empty_cache()
    # the other workloads, each in the configuration it ships with (no CPU baseline)
    names = [w for w in (args.workloads.split(",") if args.workloads else []) if w]
    if names:
        out["workloads"] = {}
    for name in names:
        if name == cfg.name and args.tokens <= 0:
            continue
        w = measure(CONFIGS[name], dev, args.steps, args.warmup, not args.no_pack, cold=False)
        for k in ("_layer", "_inputs", "_stats"):
            w.pop(k)
        out["workloads"][name] = w
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
