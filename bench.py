#!/usr/bin/env python3
"""Benchmark: paged MLA decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole decode path over one batch: the host tile
scheduler (mla_get_metadata) with its upload, then mla_decode_kvcache (split-KV
kernel + combine kernel). Inputs are resident in HBM before timing starts. The
KV pool is replicated R times and steps rotate through the copies so that the
working set exceeds the 256 MB Infinity Cache and the numbers are HBM numbers.

Prints one JSON line. `value` is achieved algorithmic HBM GB/s of the whole
step; TFLOPS and roofline fractions ride along. `roofline` is measured on the
split-KV kernel alone with HIP events on the decode stream. `cpu_baseline`
times the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense BF16 MFMA
INFINITY_CACHE_BYTES = 256 << 20


def algorithmic_work(w):
    """Bytes the method must move and FLOPs it must do (no partials, no re-reads).

    bytes = sum_b h_kv*L_b*bpt + q + o + lse + block-table entries + lengths,
    flops = 2*(576 + 512) * h_q * sum_b sum_s n_allowed(b, s)."""
    L = [int(x) for x in w.cache_seqlens.tolist()]
    B, S, H, Hk = w.batch, w.s_q, w.h_q, w.h_kv
    bpt = 1152 if w.kv_format == "bf16" else 656
    kv = sum(Hk * l * bpt for l in L)
    q = B * S * H * 576 * 2
    o = B * S * H * 512 * 2
    lse = B * S * H * 4
    bt = sum((l + 63) // 64 for l in L) * 4
    byts = kv + q + o + lse + bt + B * 4
    n_allowed = 0
    for l in L:
        for s in range(S):
            n_allowed += max(0, min(l, (l - S + 1 + s) if w.causal else l))
    flops = 2 * (576 + 512) * H * n_allowed
    return byts, flops, kv


class HipEvents:
    """Minimal HIP event API through ctypes (events on the decode stream).

    Events are created without the system-scope fence (hipEventDisableSystemFence):
    a default event's completion writes back and invalidates the GPU caches, which
    put ~16 us of idle time into every step. These events only order timestamps and
    tell the host that a step has read its staging buffer; results are read after a
    full device synchronize."""

    DISABLE_TIMING = 0x2
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self, timing: bool = True):
        e = ctypes.c_void_p()
        flags = self.DISABLE_SYSTEM_FENCE | (0 if timing else self.DISABLE_TIMING)
        if self.lib.hipEventCreateWithFlags(ctypes.byref(e), flags) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e.value

    def record(self, e, stream) -> None:
        if self.lib.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def synchronize(self, e) -> None:
        if self.lib.hipEventSynchronize(ctypes.c_void_p(e)) != 0:
            raise RuntimeError("hipEventSynchronize failed")

    def elapsed_ms(self, a, b) -> float:
        t = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(t.value)

    def destroy(self, e):
        self.lib.hipEventDestroy(ctypes.c_void_p(e))


def cpu_baseline(w, target_s: float = 15.0):
    """Time the oracle on the first sequences of the workload (bounded sample)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    a = w.as_numpy()
    done, t_total, n = [], 0.0, 0
    while t_total < target_s and n < 64 * w.batch:      # cycle through the batch until the time target
        b = n % w.batch
        t0 = time.perf_counter()
        oracle.mla_decode(a["q_bits"], a["kvcache"], w.kv_format, a["block_table"], a["cache_seqlens"],
                          dv=w.dv, causal=w.causal, softmax_scale=w.softmax_scale, batches=[b])
        t_total += time.perf_counter() - t0
        done.append(b)
        n += 1
    L = [int(a["cache_seqlens"][b]) for b in done]
    bpt = 1152 if w.kv_format == "bf16" else 656
    S, H = w.s_q, w.h_q
    byts = sum(w.h_kv * l * bpt for l in L) + len(done) * S * H * (576 * 2 + 512 * 2 + 4) \
        + sum((l + 63) // 64 for l in L) * 4 + 4 * len(done)
    return {"value": round(byts / t_total / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(done)} sequence decodes cycling through the {w.batch} sequences in batch order "
                      f"({sum(L)} cached tokens), {t_total:.2f} s, numpy float64"}


def source_sha256() -> str:
    """Hash of the library sources: a stored counter summary is only used for the same kernels."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_mla_decode_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_file(kernel: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when there is
    none or it was taken on other kernel sources."""
    path = traffic_file(kernel, workload)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_sha256():
        return None
    try:
        return int(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _pmc_rows(d: str):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    rows = []
    for fn in files:
        with open(fn) as f:
            rows.extend(csv.DictReader(f))
    return rows


def _per_dispatch(rows, counter: str, match) -> list:
    """Counter value per dispatch (summed over the instances rocprofv3 reports) for kernels matching."""
    acc = {}
    for r in rows:
        if r["Counter_Name"] == counter and match(r["Kernel_Name"]):
            acc[r["Dispatch_Id"]] = acc.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return list(acc.values())


def pmc_summary(args) -> str:
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the split kernel by what the same
    counters read for the calibration copy of known size."""
    from workloads import named_workload
    w = named_workload(args.workload)
    split_name = split_kernel_name(w)
    is_split = lambda n: (split_name + "(") in n or (split_name + "<") in n
    is_copy = lambda n: "elementwise" in n and "Mul" in n
    fr, wr = _pmc_rows(args.pmc_summary[0]), _pmc_rows(args.pmc_summary[1])
    f_split, w_split = _per_dispatch(fr, "FETCH_SIZE", is_split), _per_dispatch(wr, "WRITE_SIZE", is_split)
    f_copy, w_copy = _per_dispatch(fr, "FETCH_SIZE", is_copy), _per_dispatch(wr, "WRITE_SIZE", is_copy)
    if not (f_split and w_split and f_copy and w_copy):
        raise SystemExit("missing split-kernel or calibration-copy dispatches in the counter files")
    copy_bytes = args.calibrate_copy_mb * (1 << 20)
    if copy_bytes <= 0:
        raise SystemExit("--calibrate-copy-mb must give the calibration copy size")
    fetch_scale = copy_bytes / (sum(f_copy) / len(f_copy) * 1024.0)
    write_scale = copy_bytes / (sum(w_copy) / len(w_copy) * 1024.0)
    fetch = sum(f_split) / len(f_split) * 1024.0 * fetch_scale
    write = sum(w_split) / len(w_split) * 1024.0 * write_scale
    byts, _, _ = algorithmic_work(w)
    lines = [
        f"# HBM traffic of {split_name} on workload {w.name} (rocprofv3 --pmc, scaled by a plain copy)",
        f"kernel: {split_name}",
        f"workload: {w.name}",
        f"source_sha256: {source_sha256()}",
        f"split_dispatches: {len(f_split)} (FETCH_SIZE run), {len(w_split)} (WRITE_SIZE run)",
        f"split_fetch_kib_per_dispatch: {sum(f_split) / len(f_split):.1f}",
        f"split_write_kib_per_dispatch: {sum(w_split) / len(w_split):.1f}",
        f"copy_bytes: {copy_bytes}",
        f"copy_fetch_kib: {sum(f_copy) / len(f_copy):.1f}",
        f"copy_write_kib: {sum(w_copy) / len(w_copy):.1f}",
        f"fetch_scale: {fetch_scale:.4f}",
        f"write_scale: {write_scale:.4f}",
        f"hbm_fetch_bytes_per_launch: {int(fetch)}",
        f"hbm_write_bytes_per_launch: {int(write)}",
        f"hbm_bytes_per_launch: {int(fetch + write)}",
        f"algorithmic_bytes_per_step: {byts}",
        f"traffic_over_algorithmic: {(fetch + write) / byts:.3f}",
    ]
    return "\n".join(lines) + "\n"


MFMA_COUNTERS = "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CYCLES GRBM_GUI_ACTIVE"
SIMDS = 256 * 4
XCDS = 8


def mfma_summary(args) -> str:
    """MFMA utilisation of the split kernel from one rocprofv3 --pmc run with MFMA_COUNTERS:
    matrix-core busy cycles summed over the SIMDs / (GPU-active cycles x SIMDs), and the bf16 MFMA
    work the counters saw against the algorithmic FLOPs. rocprofv3 reports GRBM_GUI_ACTIVE summed
    over the 8 XCDs (each has its own); the per-dispatch medians are used (the first dispatch of a
    run is cold)."""
    from workloads import named_workload
    w = named_workload(args.workload)
    split_name = split_kernel_name(w)
    is_split = lambda n: (split_name + "(") in n or (split_name + "<") in n
    rows = _pmc_rows(args.mfma_summary)
    busy = _per_dispatch(rows, "SQ_VALU_MFMA_BUSY_CYCLES", is_split)
    mops = _per_dispatch(rows, "SQ_INSTS_VALU_MFMA_MOPS_BF16", is_split)
    gui = _per_dispatch(rows, "GRBM_GUI_ACTIVE", is_split)
    if not (busy and mops and gui):
        raise SystemExit("missing split-kernel dispatches or MFMA counters in the counter files")
    med = lambda xs: percentiles(xs, (50,))[0]
    _, flops, _ = algorithmic_work(w)
    active = med(gui) / XCDS
    dur_ns = {}
    for r in rows:
        if is_split(r["Kernel_Name"]):
            dur_ns[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    dur_us = med(list(dur_ns.values())) / 1e3
    util = med(busy) / (active * SIMDS)
    mfma_flops = med(mops) * 512.0
    lines = [
        f"# MFMA utilisation of {split_name} on workload {w.name} (rocprofv3 --pmc)",
        f"kernel: {split_name}",
        f"workload: {w.name}",
        f"source_sha256: {source_sha256()}",
        f"counters: {MFMA_COUNTERS}",
        f"split_dispatches: {len(busy)}",
        f"mfma_busy_cycles_per_dispatch (sum over {SIMDS} SIMDs): {med(busy):.0f}",
        f"gpu_active_cycles_per_dispatch (GRBM_GUI_ACTIVE / {XCDS} XCDs): {active:.0f}",
        f"mfma_util (busy / (active x {SIMDS})): {util:.4f}",
        f"dispatch_duration_us (counter-run timestamps): {dur_us:.1f}",
        f"implied_clock_ghz (active cycles / duration): {active / (dur_us * 1e3):.2f}",
        f"bf16_mfma_flops_per_dispatch (MOPS x 512): {mfma_flops:.4e}",
        f"algorithmic_flops_per_step: {flops:.4e}",
        f"mfma_flops_over_algorithmic: {mfma_flops / flops:.3f}",
    ]
    return "\n".join(lines) + "\n"


def split_kernel_name(w) -> str:
    """Name of the split kernel a workload runs (128-row tiles above 64 rows per KV head:
    the one-barrier kernel for bf16 pages, the two-barrier one for FP8)."""
    if w.heads_per_kv > 64:
        return "splitkv_x1_kernel" if w.kv_format == "bf16" else "splitkv_x_kernel"
    return "splitkv_kernel"


def percentiles(xs, ps):
    """Nearest-rank percentiles of a list of floats."""
    ys = sorted(xs)
    return [ys[min(len(ys) - 1, max(0, math.ceil(p / 100 * len(ys)) - 1))] for p in ps]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="compute_heavy")
    ap.add_argument("--copies", type=int, default=0, help="KV pool replicas to rotate through (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="run one plain fp32 copy kernel (out = in * 1) of this size before timing, as the "
                         "reference for scaling HBM byte counters")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "bench made with --calibrate-copy-mb, and print the traffic summary")
    ap.add_argument("--mfma-summary", metavar="DIR",
                    help="no GPU run: summarise one rocprofv3 --pmc run of this bench with the counters "
                         "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CYCLES GRBM_GUI_ACTIVE")
    args = ap.parse_args()
    if args.pmc_summary:
        print(pmc_summary(args), end="")
        return
    if args.mfma_summary:
        print(mfma_summary(args), end="")
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the decode path shards by sequence with no communication; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_mla_decode_amd as mla
    from workloads import WORKLOAD_SPECS, named_workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = named_workload(args.workload)
    byts, flops, kv_bytes = algorithmic_work(w)
    pool_bytes = w.kvcache.numel() * w.kvcache.element_size()
    copies = args.copies or max(1, math.ceil(2 * INFINITY_CACHE_BYTES / max(pool_bytes, 1)))
    print(f"[bench] {w.name}: {WORKLOAD_SPECS[w.name]['text']}; pool {pool_bytes / 1e6:.1f} MB x {copies} copies",
          file=sys.stderr, flush=True)

    q = w.q.to(dev)
    bt = w.block_table.to(dev)
    L_dev = w.cache_seqlens.to(dev)
    L_host = w.cache_seqlens.clone().pin_memory()
    kvs = [w.kvcache.to(dev) for _ in range(copies)]
    M = w.heads_per_kv
    parts = mla.mla_num_parts(w.batch, M, w.h_kv, w.kv_format)
    flat_dev = torch.empty((parts * 8 + w.batch + 1,), dtype=torch.int32, device=dev)
    meta_dev, splits_dev = mla.split_metadata(flat_dev, w.batch)
    out = torch.empty((w.batch, w.s_q, w.h_q, w.dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.h_q, w.s_q), dtype=torch.float32, device=dev)
    ws = torch.empty((mla.mla_workspace_bytes(w.batch, parts, M, w.h_kv),), dtype=torch.uint8, device=dev)
    _, s_host = mla.mla_get_metadata_host(L_host, M, w.h_kv, kv_format=w.kv_format, num_parts=parts)
    max_splits = mla.max_splits_of(s_host)
    decoders = [mla.MlaDecoder(q, kv, bt, L_dev, w.dv, meta_dev, splits_dev, w.causal, w.softmax_scale,
                               out=out, lse=lse, workspace=ws, max_splits=max_splits) for kv in kvs]
    stream = torch.cuda.current_stream(dev)
    hip = HipEvents()

    # two pinned staging buffers for the host scheduler's output, used in turn; a buffer is
    # rewritten only after the upload that read it two steps earlier has finished
    stage = [torch.empty((parts * 8 + w.batch + 1,), dtype=torch.int32, pin_memory=True) for _ in range(2)]
    stage_done = [None, None]

    def step(i, ev=None):
        # a1: host tile scheduler for this step's lengths, uploaded on the decode stream
        # (metadata rows and num_splits share one pinned buffer: one copy)
        k = i & 1
        if stage_done[k] is not None:
            hip.synchronize(stage_done[k])
        m_h, _ = mla.mla_get_metadata_host(L_host, M, w.h_kv, kv_format=w.kv_format, num_parts=parts,
                                           out=stage[k])
        flat_dev.copy_(stage[k], non_blocking=True)
        if stage_done[k] is None:
            stage_done[k] = hip.create(timing=False)
        hip.record(stage_done[k], stream)
        d = decoders[i % copies]
        d.set_events(ev if ev is not None else (None, None, None))
        d.run(stream)

    if args.calibrate_copy_mb > 0:
        n = args.calibrate_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)            # reads and writes calibrate_copy_mb MiB once
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(hip.create(), hip.create(), hip.create()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    split_ms = [hip.elapsed_ms(e[0], e[1]) for e in evs]
    comb_ms = [hip.elapsed_ms(e[1], e[2]) for e in evs]
    for e in evs:
        for x in e:
            hip.destroy(x)
    for x in stage_done:
        if x is not None:
            hip.destroy(x)
    split_avg = sum(split_ms) / len(split_ms)
    comb_avg = sum(comb_ms) / len(comb_ms)

    gbs = byts / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    split_gbs = byts / (split_avg * 1e-3) / 1e9
    split_tflops = flops / (split_avg * 1e-3) / 1e12
    intensity = flops / byts
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    bound = "hbm" if intensity < ridge else "mfma"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(split_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(split_gbs / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": round(split_tflops, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(split_tflops / BF16_PEAK_TFLOPS, 4), "traffic": None}

    split_name = split_kernel_name(w)
    roof["traffic"] = stored_traffic(split_name, w.name)

    result = {
        "metric": "paged MLA decode achieved HBM GB/s and TFLOPS (+% of roofline), 1 MI355X",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "s_q": w.s_q, "h_q": w.h_q, "h_kv": w.h_kv,
                   "d_qk": 576, "d_v": 512, "page": 64, "kv_format": w.kv_format, "causal": w.causal,
                   "total_kv_tokens": int(w.cache_seqlens.sum()), "num_parts": parts, "kv_copies": copies},
        "tflops": round(tflops, 2),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
        "split_kernel_ms": round(split_avg, 5),
        "split_kernel_ms_p10_p50_p90": [round(x, 5) for x in percentiles(split_ms, (10, 50, 90))],
        "combine_kernel_ms": round(comb_avg, 5),
        "algorithmic_bytes": byts,
        "algorithmic_flops": flops,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
