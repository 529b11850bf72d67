#!/usr/bin/env python3
"""Benchmark: paged MLA decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

The default workload is mtp (batch 128, s_q 2, h_q 128, causal, L ~ U[3072, 5120]):
the largest configuration, with 256 query rows per KV head. One step is one pass
of the whole decode path over one batch: the host tile scheduler
(mla_get_metadata) with its upload, then mla_decode_kvcache (split-KV kernel +
combine kernel). Inputs are resident in HBM before timing starts. The KV pool is
replicated R times and steps rotate through the copies so that the working set
exceeds the 256 MB Infinity Cache and the numbers are HBM numbers.

Prints one JSON line. `value` is achieved algorithmic HBM GB/s of the whole
step; TFLOPS and roofline fractions ride along. `roofline` is measured on the
split-KV kernel alone with HIP events attached to its launch on the decode
stream; `roofline_split_combine` prices the same work over both kernels of the
call. `cpu_baseline` times the CPU oracle on a bounded sample of the same
workload (plus 1-core samples of the small workloads).
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


def is_prefill(w) -> bool:
    return hasattr(w, "kv") and not hasattr(w, "kvcache")


def load_workload(name: str):
    """A decode workload (WORKLOAD_SPECS) or a sparse-prefill one (PREFILL_SPECS) by name."""
    from workloads import PREFILL_SPECS, named_prefill, named_workload
    return named_prefill(name) if name in PREFILL_SPECS else named_workload(name)


def prefill_attended(w):
    """Listed entries of each (query token, KV head) that name a row (not -1)."""
    return int((w.indices >= 0).sum())


def algorithmic_work(w):
    """Bytes the method must move and FLOPs it must do (no partials, no re-reads).

    bytes = sum_b h_kv*L_b*bpt + q + o + lse + block-table entries + lengths,
    flops = 2*(576 + 512) * h_q * sum_b sum_s n_allowed(b, s).
    Sparse prefill: bytes = every kv row once + q + o + lse + indices (a listed row is
    gathered again for every query token that lists it, from cache, not HBM), flops =
    2*(576 + 512) * (h_q / h_kv) * listed rows over all (token, KV head)."""
    if is_prefill(w):
        n_att = prefill_attended(w)
        kv = w.s_kv * w.h_kv * 1152
        byts = kv + w.s_q * w.h_q * (576 * 2 + 512 * 2 + 4) + w.indices.numel() * 4
        return byts, 2 * (576 + 512) * (w.h_q // w.h_kv) * n_att, kv
    L = [int(x) for x in w.cache_seqlens.tolist()]
    B, S, H, Hk = w.batch, w.s_q, w.h_q, w.h_kv
    bpt = 1152 if w.kv_format == "bf16" else 656
    if getattr(w, "indices", None) is not None:
        # sparse: the attended entries of each query token (listed, not -1, inside the causal
        # mask); each one moves its cached row and its block-table entry; the indices are read
        import numpy as np
        idx = w.indices.numpy().astype(np.int64)
        Lb = np.asarray(L, dtype=np.int64)[:, None, None]
        s_ = np.arange(S)[None, :, None]
        att = (idx >= 0) & ((not w.causal) | (idx <= Lb - S + s_))
        n_att = int(att.sum())
        byts = (n_att * Hk * bpt + B * S * H * (576 * 2 + 512 * 2 + 4) + n_att * 4 + idx.size * 4 + B * 4)
        return byts, 2 * (576 + 512) * H * n_att, n_att * Hk * bpt
    kv = sum(Hk * l * bpt for l in L)
    if getattr(w, "vcache", None) is not None:
        kv += sum(Hk * l * w.dv * 2 for l in L)       # the separate V rows
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


def host_cores() -> int:
    """CPU threads this process may use: its affinity set, capped by OMP_NUM_THREADS when set
    (the share of a shared host that the job is given)."""
    n = len(os.sched_getaffinity(0))
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        cap = 0
    return min(n, cap) if cap > 0 else n


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_sample(w, target_s: float):
    """Oracle decodes of one sequence at a time, cycling through the batch, until target_s of
    oracle time is spent; returns (sequences done, seconds, algorithmic bytes of them, cached
    tokens they read)."""
    import numpy as np
    import oracle
    a = w.as_numpy()
    sparse = getattr(w, "indices", None) is not None
    idx = w.indices.numpy() if sparse else None
    done, t_total, n = [], 0.0, 0
    while t_total < target_s and n < max(64 * w.batch, 4096):
        b = n % w.batch
        t0 = time.perf_counter()
        if sparse:
            oracle.mla_decode_sparse(a["q_bits"], a["kvcache"], w.kv_format, a["block_table"], a["cache_seqlens"],
                                     idx, dv=w.dv, causal=w.causal, softmax_scale=w.softmax_scale, batches=[b])
        else:
            oracle.mla_decode(a["q_bits"], a["kvcache"], w.kv_format, a["block_table"], a["cache_seqlens"],
                              dv=w.dv, causal=w.causal, softmax_scale=w.softmax_scale, batches=[b],
                              vcache=a.get("vcache"))
        t_total += time.perf_counter() - t0
        done.append(b)
        n += 1
    bpt = 1152 if w.kv_format == "bf16" else 656
    if sparse:
        # tokens a sequence reads: its attended entries (the accounting of algorithmic_work)
        L = np.asarray(a["cache_seqlens"], dtype=np.int64)[:, None, None]
        att = (idx >= 0) & ((not w.causal) | (idx <= L - w.s_q + np.arange(w.s_q)[None, :, None]))
        per_b = att.reshape(w.batch, -1).sum(axis=1)
        toks = [int(per_b[b]) for b in done]
        byts = sum(w.h_kv * t * bpt + 4 * t for t in toks) + len(done) * w.s_q * (
            w.h_q * (576 * 2 + 512 * 2 + 4) + 4 * w.topk) + 4 * len(done)
        return done, t_total, byts, sum(toks)
    L = [int(a["cache_seqlens"][b]) for b in done]
    if "vcache" in a:
        bpt += w.dv * 2
    byts = sum(w.h_kv * l * bpt for l in L) + len(done) * w.s_q * w.h_q * (576 * 2 + 512 * 2 + 4) \
        + sum((l + 63) // 64 for l in L) * 4 + 4 * len(done)
    return done, t_total, byts, sum(L)


def cpu_baseline(w, target_s: float = 15.0, one_core=("tiny", "compute_heavy", "ragged"), one_core_s: float = 3.0):
    """Time the oracle (as it stands) on a bounded sample of the workload with every host core the
    job may use (BLAS threads set to match), plus 1-core samples of the small workloads."""
    from threadpoolctl import threadpool_limits
    from workloads import named_workload
    cores = host_cores()
    with threadpool_limits(limits=cores):
        done, t_total, byts, toks = _oracle_sample(w, target_s)
    res = {"value": round(byts / t_total / 1e9, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
           "sample": f"{len(done)} sequence decodes cycling through the {w.batch} sequences of {w.name} in batch "
                     f"order ({toks} cached tokens), {t_total:.2f} s, numpy float64",
           "cpu_model": cpu_model(), "one_core": {}}
    for name in one_core:
        w1 = w if name == w.name else named_workload(name)
        with threadpool_limits(limits=1):
            d1, t1, b1, k1 = _oracle_sample(w1, one_core_s)
        res["one_core"][name] = {"value": round(b1 / t1 / 1e9, 4), "unit": "GB/s",
                                 "sample": f"{len(d1)} sequence decodes ({k1} cached tokens), {t1:.2f} s"}
    return res


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
    w = load_workload(args.workload)
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


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F8 "
                 "SQ_INSTS_VALU_MFMA_MOPS_F6F4 SQ_BUSY_CYCLES GRBM_GUI_ACTIVE")
SIMDS = 256 * 4
XCDS = 8


def mfma_summary(args) -> str:
    """MFMA utilisation of the split kernel from one rocprofv3 --pmc run with MFMA_COUNTERS:
    matrix-core busy cycles summed over the SIMDs / (GPU-active cycles x SIMDs), and the bf16 MFMA
    work the counters saw against the algorithmic FLOPs. rocprofv3 reports GRBM_GUI_ACTIVE summed
    over the 8 XCDs (each has its own); the per-dispatch medians are used (the first dispatch of a
    run is cold)."""
    w = load_workload(args.workload)
    split_name = split_kernel_name(w)
    is_split = lambda n: (split_name + "(") in n or (split_name + "<") in n
    rows = _pmc_rows(args.mfma_summary)
    busy = _per_dispatch(rows, "SQ_VALU_MFMA_BUSY_CYCLES", is_split)
    mops = _per_dispatch(rows, "SQ_INSTS_VALU_MFMA_MOPS_BF16", is_split)
    mops8 = _per_dispatch(rows, "SQ_INSTS_VALU_MFMA_MOPS_F8", is_split) or [0.0]
    mops64 = _per_dispatch(rows, "SQ_INSTS_VALU_MFMA_MOPS_F6F4", is_split) or [0.0]
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
    f8_flops = (med(mops8) + med(mops64)) * 512.0
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
        f"bf16_mfma_flops_per_dispatch (MOPS_BF16 x 512): {mfma_flops:.4e}",
        f"fp8_mfma_flops_per_dispatch ((MOPS_F8 + MOPS_F6F4) x 512): {f8_flops:.4e}",
        f"algorithmic_flops_per_step: {flops:.4e}",
        f"mfma_flops_over_algorithmic: {(mfma_flops + f8_flops) / flops:.3f}",
        f"attainable_bf16_tflops_at_this_clock (2.5 PF x clock / 2.4 GHz): "
        f"{BF16_PEAK_TFLOPS * (active / (dur_us * 1e3)) / 2.4:.0f}",
    ]
    return "\n".join(lines) + "\n"


LDS_COUNTERS = ("SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_WAIT_INST_LDS SQ_BUSY_CYCLES "
                "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_INSTS_VALU")


def counter_summary(args) -> str:
    """Per-dispatch medians of every counter of one rocprofv3 --pmc run for the split kernel (LDS
    and wait counters: LDS_COUNTERS), with the wait shares: SQ_WAIT_ANY, SQ_WAIT_INST_LDS and
    SQ_WAVE_CYCLES count in the same units (wave-cycles), so their ratios are the share of wave
    time spent waiting (on anything / on LDS instruction issue)."""
    w = load_workload(args.workload)
    split_name = split_kernel_name(w)
    is_split = lambda n: (split_name + "(") in n or (split_name + "<") in n
    rows = _pmc_rows(args.counter_summary)
    names = sorted({r["Counter_Name"] for r in rows})
    med = lambda xs: percentiles(xs, (50,))[0]
    vals = {}
    for n in names:
        v = _per_dispatch(rows, n, is_split)
        if v:
            vals[n] = med(v)
    if not vals:
        raise SystemExit("no split-kernel dispatches in the counter files")
    lines = [f"# counters of {split_name} on workload {w.name} (rocprofv3 --pmc), median per dispatch",
             f"kernel: {split_name}", f"workload: {w.name}", f"source_sha256: {source_sha256()}",
             f"split_dispatches: {len(_per_dispatch(rows, names[0], is_split))}"]
    lines += [f"{n}: {vals[n]:.6g}" for n in sorted(vals)]
    if "SQ_WAVE_CYCLES" in vals and vals["SQ_WAVE_CYCLES"] > 0:
        if "SQ_WAIT_ANY" in vals:
            lines.append(f"wait_any_over_wave_cycles: {vals['SQ_WAIT_ANY'] / vals['SQ_WAVE_CYCLES']:.3f}")
        if "SQ_WAIT_INST_LDS" in vals:
            lines.append(f"wait_inst_lds_over_wave_cycles: {vals['SQ_WAIT_INST_LDS'] / vals['SQ_WAVE_CYCLES']:.3f}")
    return "\n".join(lines) + "\n"


def trace_summary(args) -> str:
    """kernels_<workload>.txt: rocprofv3 --kernel-trace --stats of a bench run (its
    *kernel_stats.csv, durations in ns), the split kernel's average beside the HIP-event figure
    of the same run, and that run's bench line (the JSON file it printed)."""
    import csv
    import glob
    d, jpath = args.trace_summary
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *kernel_stats.csv under {d}")
    with open(files[0]) as f:
        text = f.read().strip()
    with open(jpath) as f:
        line = [x for x in f.read().splitlines() if x.startswith("{")][-1]
    res = json.loads(line)
    w = load_workload(args.workload)
    name = split_kernel_name(w)
    split_avg = None
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if (name + "(") in r["Name"] or (name + "<") in r["Name"]:
                split_avg = float(r["AverageNs"]) / 1e3
                calls = int(r["Calls"])
    # the timed steps are the last `steps` dispatches (the warmup ones run before the clock settles)
    timed_avg = None
    traces = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if traces:
        with open(traces[0]) as f:
            rows = [r for r in csv.DictReader(f) if (name + "(") in r["Kernel_Name"] or (name + "<") in r["Kernel_Name"]]
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows[-res["steps"]:]]
        if durs:
            timed_avg = sum(durs) / len(durs)
    out = [f"# rocprofv3 kernel-trace statistics, workload {w.name} ({res['steps']} timed + {res['warmup']} warmup steps)",
           "# command (from the repository root on the GPU host):",
           f"#   cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- python3 "
           f"<repo>/bench.py --workload {w.name} --steps {res['steps']} --warmup {res['warmup']} --no-cpu-baseline > <json>",
           f"#   python3 bench.py --trace-summary <dir> <json> --workload {w.name}",
           "# columns as rocprofv3 writes them to its kernel_stats.csv (durations in ns)",
           text, ""]
    if split_avg is not None:
        out.append(f"split kernel ({name}) average (rocprofv3 stats, all {calls} calls): {split_avg:.2f} us")
    if timed_avg is not None:
        out.append(f"split kernel average over the {res['steps']} timed calls (rocprofv3 kernel trace): {timed_avg:.2f} us")
    out.append(f"split kernel average (bench.py HIP events, the same {res['steps']} timed calls): "
               f"{res['split_kernel_ms'] * 1e3:.2f} us")
    out.append(f"bench line of the profiled run: ms_per_step {res['ms_per_step']}, value {res['value']} {res['unit']}, "
               f"roofline {json.dumps(res['roofline'])}")
    if timed_avg is not None:
        byts, flops, _ = algorithmic_work(w)
        rf = roofline(byts, flops, timed_avg * 1e-3)
        out.append(f"roofline from the rocprofv3 timed-call average: {rf['achieved']} {rf['unit']} = {rf['frac']:.4f} "
                   f"of {rf['peak']} (bench line: {res['roofline']['frac']})")
    return "\n".join(out) + "\n"


def split_kernel_name(w) -> str:
    """Name of the split kernel a workload runs: the separate-V-cache kernel when there is a V
    cache, the 128-row one-barrier kernel above 64 rows per KV head and for every sparse
    workload (decode and prefill), else the 64-row kernel."""
    if getattr(w, "vcache", None) is not None:
        return "splitkv_vc_kernel"
    if is_prefill(w) or getattr(w, "indices", None) is not None or w.heads_per_kv > 64:
        return "splitkv_x1_kernel"
    return "splitkv_kernel"


def roofline(byts: int, flops: int, ms: float) -> dict:
    """Algorithmic bytes or FLOPs over a kernel time, against the roofline that bounds the
    workload: HBM below the ridge (2.5 PFLOP/s / 8 TB/s = 312.5 FLOP/B), dense bf16 MFMA above."""
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if flops / byts < ridge:
        gbs = byts / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}
    tf = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": None}


def percentiles(xs, ps):
    """Nearest-rank percentiles of a list of floats."""
    ys = sorted(xs)
    return [ys[min(len(ys) - 1, max(0, math.ceil(p / 100 * len(ys)) - 1))] for p in ps]


def _prefill_oracle_sample(w, target_s: float):
    """Oracle prefill of one query token at a time (strided through the tokens) until target_s of
    oracle time is spent; returns (tokens done, seconds, algorithmic FLOPs of them)."""
    import oracle
    a = w.as_numpy()
    done, t_total, n = [], 0.0, 0
    stride = 997                                # coprime with the token counts used: visits every token
    while t_total < target_s and n < w.s_q:
        s = (n * stride) % w.s_q
        t0 = time.perf_counter()
        oracle.mla_sparse_prefill(a["q_bits"], a["kv_bits"], a["indices"], w.softmax_scale, dv=w.dv, tokens=[s])
        t_total += time.perf_counter() - t0
        done.append(s)
        n += 1
    n_att = int((a["indices"][done] >= 0).sum())
    return done, t_total, 2 * (576 + 512) * (w.h_q // w.h_kv) * n_att


def prefill_cpu_baseline(w, target_s: float = 15.0, one_core_s: float = 3.0):
    from threadpoolctl import threadpool_limits
    cores = host_cores()
    with threadpool_limits(limits=cores):
        done, t_total, fl = _prefill_oracle_sample(w, target_s)
    res = {"value": round(fl / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
           "sample": f"{len(done)} query tokens of {w.name} (all {w.h_q} heads, {w.topk} listed rows each), "
                     f"{t_total:.2f} s, numpy float64",
           "cpu_model": cpu_model()}
    with threadpool_limits(limits=1):
        d1, t1, f1 = _prefill_oracle_sample(w, one_core_s)
    res["one_core"] = {w.name: {"value": round(f1 / t1 / 1e12, 6), "unit": "TFLOP/s",
                                "sample": f"{len(d1)} query tokens, {t1:.2f} s"}}
    return res


def bench_prefill(args, dev):
    """One step = the host scheduler's metadata for the sizes (uploaded) + one sparse prefill
    call (split kernel + combine) over the whole batch of query tokens."""
    import torch
    import paged_mla_decode_amd as mla
    from workloads import PREFILL_SPECS, named_prefill
    w = named_prefill(args.workload)
    byts, flops, _ = algorithmic_work(w)
    print(f"[bench] {w.name}: {PREFILL_SPECS[w.name]['text']}", file=sys.stderr, flush=True)
    q, kv, idx = w.q.to(dev), w.kv.to(dev), w.indices.to(dev)
    parts = mla.mla_num_parts(w.s_q, w.h_q // w.h_kv, w.h_kv, "bf16")
    flat_dev = torch.empty((parts * 8 + w.s_q + 1,), dtype=torch.int32, device=dev)
    meta_dev, splits_dev = mla.split_metadata(flat_dev, w.s_q)

    def host_metadata():
        return mla.mla_get_metadata_sparse(w.s_q, 1, w.topk, w.h_q, w.h_kv, num_parts=parts, host=True)

    _, s_host = host_metadata()
    pre = mla.MlaSparsePrefill(q, kv, idx, w.softmax_scale, w.dv, tile_metadata=meta_dev, num_splits=splits_dev,
                               max_splits=mla.max_splits_of(s_host))
    stream = torch.cuda.current_stream(dev)
    hip = HipEvents()
    stage = [torch.empty((parts * 8 + w.s_q + 1,), dtype=torch.int32, pin_memory=True) for _ in range(2)]
    stage_done = [None, None]

    def step(i, ev=None):
        k = i & 1
        if stage_done[k] is not None:
            hip.synchronize(stage_done[k])
        m_h, _ = host_metadata()
        stage[k].copy_(mla.packed_metadata(m_h))
        flat_dev.copy_(stage[k], non_blocking=True)
        if stage_done[k] is None:
            stage_done[k] = hip.create(timing=False)
        hip.record(stage_done[k], stream)
        pre.set_events(ev if ev is not None else (None, None, None))
        pre.run(stream)

    if args.calibrate_copy_mb > 0:
        n = args.calibrate_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
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
    tflops = flops / (ms * 1e-3) / 1e12
    roof = roofline(byts, flops, split_avg)
    roof["traffic"] = stored_traffic(split_kernel_name(w), w.name)
    roof_call = roofline(byts, flops, split_avg + comb_avg)
    roof_call.pop("traffic")
    result = {
        "metric": "sparse MLA prefill achieved TFLOPS (+% of roofline), 1 MI355X",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "s_q": w.s_q, "s_kv": w.s_kv, "h_q": w.h_q, "h_kv": w.h_kv, "topk": w.topk,
                   "d_qk": 576, "d_v": 512, "num_parts": parts},
        "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
        "split_kernel_ms": round(split_avg, 5),
        "split_kernel_ms_p10_p50_p90": [round(x, 5) for x in percentiles(split_ms, (10, 50, 90))],
        "combine_kernel_ms": round(comb_avg, 5),
        "algorithmic_bytes": byts,
        "algorithmic_flops": flops,
        "roofline": roof,
        "roofline_split_combine": roof_call,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = prefill_cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mtp")
    ap.add_argument("--copies", type=int, default=0, help="KV pool replicas to rotate through (0: auto)")
    ap.add_argument("--metadata", choices=("host", "device"), default="host",
                    help="where each step's tile-scheduler metadata is computed: on the host (then uploaded) or "
                         "by the device scheduler kernel from the device lengths (no host work, no copy; the "
                         "combine then runs without the host's piece-count hint)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="run one plain fp32 copy kernel (out = in * 1) of this size before timing, as the "
                         "reference for scaling HBM byte counters")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "bench made with --calibrate-copy-mb, and print the traffic summary")
    ap.add_argument("--trace-summary", nargs=2, metavar=("DIR", "JSON"),
                    help="no GPU run: summarise one rocprofv3 --kernel-trace --stats run of this bench (DIR) "
                         "with the JSON line that run printed")
    ap.add_argument("--counter-summary", metavar="DIR",
                    help="no GPU run: per-dispatch medians of the counters of one rocprofv3 --pmc run of this "
                         "bench (LDS_COUNTERS: LDS use and wait shares)")
    ap.add_argument("--mfma-summary", metavar="DIR",
                    help="no GPU run: summarise one rocprofv3 --pmc run of this bench with the counters of "
                         "MFMA_COUNTERS (busy cycles, bf16 / fp8 / fp6-fp4 MOPs, SQ busy, GUI active)")
    args = ap.parse_args()
    if args.pmc_summary:
        print(pmc_summary(args), end="")
        return
    if args.mfma_summary:
        print(mfma_summary(args), end="")
        return
    if args.trace_summary:
        print(trace_summary(args), end="")
        return
    if args.counter_summary:
        print(counter_summary(args), end="")
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the decode path shards by sequence with no communication; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_mla_decode_amd as mla
    from workloads import PREFILL_SPECS, WORKLOAD_SPECS, named_workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload in PREFILL_SPECS:
        if args.metadata == "device":
            raise SystemExit("--metadata device: the sparse metadata depends only on the sizes (host)")
        bench_prefill(args, dev)
        return
    w = named_workload(args.workload)
    byts, flops, kv_bytes = algorithmic_work(w)
    pool_bytes = w.kvcache.numel() * w.kvcache.element_size()
    if w.vcache is not None:
        pool_bytes += w.vcache.numel() * w.vcache.element_size()
    copies = args.copies or max(1, math.ceil(2 * INFINITY_CACHE_BYTES / max(pool_bytes, 1)))
    print(f"[bench] {w.name}: {WORKLOAD_SPECS[w.name]['text']}; pool {pool_bytes / 1e6:.1f} MB x {copies} copies",
          file=sys.stderr, flush=True)

    q = w.q.to(dev)
    bt = w.block_table.to(dev)
    L_dev = w.cache_seqlens.to(dev)
    L_host = w.cache_seqlens.clone().pin_memory()
    kvs = [w.kvcache.to(dev) for _ in range(copies)]
    vcs = [w.vcache.to(dev) if w.vcache is not None else None for _ in range(copies)]
    M = w.heads_per_kv
    sparse = getattr(w, "indices", None) is not None
    nseq = w.batch * w.s_q if sparse else w.batch
    parts = mla.mla_num_parts(nseq, w.h_q // w.h_kv if sparse else M, w.h_kv, w.kv_format)
    flat_dev = torch.empty((parts * 8 + nseq + 1,), dtype=torch.int32, device=dev)
    meta_dev, splits_dev = mla.split_metadata(flat_dev, nseq)
    idx_dev = w.indices.to(dev) if sparse else None
    out = torch.empty((w.batch, w.s_q, w.h_q, w.dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.h_q, w.s_q), dtype=torch.float32, device=dev)
    from paged_mla_decode_amd import _lib as mla_lib
    ws_bytes = (mla_lib.load().mla_workspace_bytes_sparse(w.batch, w.s_q, parts, w.h_q, w.h_kv) if sparse
                else mla.mla_workspace_bytes(w.batch, parts, M, w.h_kv))
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    max_blocks = int(w.block_table.shape[1])

    def host_metadata(out_buf=None):
        """a1 on the host: the scheduler's metadata for this step (sparse: from the sizes alone)"""
        if sparse:
            m_h, s_h = mla.mla_get_metadata_sparse(w.batch, w.s_q, w.topk, w.h_q, w.h_kv, kv_format=w.kv_format,
                                                   num_parts=parts, host=True)
            if out_buf is not None:
                out_buf.copy_(mla.packed_metadata(m_h))
            return m_h, s_h
        return mla.mla_get_metadata_host(L_host, M, w.h_kv, kv_format=w.kv_format, num_parts=parts,
                                         max_blocks_per_seq=max_blocks, out=out_buf)

    _, s_host = host_metadata()
    max_splits = mla.max_splits_of(s_host)
    decoders = [mla.MlaDecoder(q, kv, bt, L_dev, w.dv, meta_dev, splits_dev, w.causal, w.softmax_scale,
                               out=out, lse=lse, workspace=ws, max_splits=max_splits, indices=idx_dev, vcache=vc)
                for kv, vc in zip(kvs, vcs)]
    stream = torch.cuda.current_stream(dev)
    hip = HipEvents()

    # two pinned staging buffers for the host scheduler's output, used in turn; a buffer is
    # rewritten only after the upload that read it two steps earlier has finished
    stage = [torch.empty((parts * 8 + nseq + 1,), dtype=torch.int32, pin_memory=True) for _ in range(2)]
    stage_done = [None, None]

    if args.metadata == "device" and sparse:
        raise SystemExit("--metadata device: the sparse metadata depends only on the sizes (host)")
    if args.metadata == "device":
        for d in decoders:
            d.args.max_splits = 0                 # the device path has no host-side piece count
    meta_ev = []

    def step(i, ev=None):
        if args.metadata == "device":
            # a1 on the device: the scheduler kernel reads the device lengths, writes the metadata
            if ev is not None:
                e0, e1 = hip.create(), hip.create()
                hip.record(e0, stream)
            mla.mla_get_metadata_device(L_dev, M, w.h_kv, kv_format=w.kv_format, num_parts=parts, out=flat_dev,
                                        stream=stream)
            if ev is not None:
                hip.record(e1, stream)
                meta_ev.append((e0, e1))
            d = decoders[i % copies]
            d.set_events(ev if ev is not None else (None, None, None))
            d.run(stream)
            return
        # a1: host tile scheduler for this step's lengths, uploaded on the decode stream
        # (metadata rows and num_splits share one pinned buffer: one copy)
        k = i & 1
        if stage_done[k] is not None:
            hip.synchronize(stage_done[k])
        host_metadata(stage[k])
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
    meta_ms = [hip.elapsed_ms(a, b) for a, b in meta_ev]
    for a, b in meta_ev:
        hip.destroy(a)
        hip.destroy(b)
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
    roof = roofline(byts, flops, split_avg)
    split_name = split_kernel_name(w)
    roof["traffic"] = stored_traffic(split_name, w.name)
    # the same algorithmic work over the decode call's two kernels (split + combine)
    roof_call = roofline(byts, flops, split_avg + comb_avg)
    roof_call.pop("traffic")

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
                   "total_kv_tokens": int(w.cache_seqlens.sum()), "num_parts": parts, "kv_copies": copies,
                   **({"topk": w.topk} if sparse else {}), **({"vcache": True} if w.vcache is not None else {})},
        "tflops": round(tflops, 2),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
        "split_kernel_ms": round(split_avg, 5),
        "split_kernel_ms_p10_p50_p90": [round(x, 5) for x in percentiles(split_ms, (10, 50, 90))],
        "combine_kernel_ms": round(comb_avg, 5),
        "metadata": args.metadata,
        "algorithmic_bytes": byts,
        "algorithmic_flops": flops,
        "roofline": roof,
        "roofline_split_combine": roof_call,
    }
    if meta_ms:
        result["metadata_kernel_ms"] = round(sum(meta_ms) / len(meta_ms), 5)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
