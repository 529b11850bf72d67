"""Host-side checks of bench.py (no GPU): its refusal of several GPUs, the
algorithmic work it prices the roofline with (counted here by enumerating the
mask), and the committed counter summaries it reads."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import make_workload  # noqa: E402


def test_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("fmt,bpt", [("bf16", 1152), ("fp8", 656)])
@pytest.mark.parametrize("causal", [False, True])
def test_algorithmic_work_by_enumeration(fmt, bpt, causal):
    L = [1, 5, 64, 130]
    B, S, H = len(L), 2, 16
    w = make_workload(name="work", batch=B, s_q=S, h_q=H, h_kv=1, seqlens=L, causal=causal, kv_format=fmt, seed=7,
                      pool_pages=sum((x + 63) // 64 for x in L) + 1)
    byts, flops, kv = bench.algorithmic_work(w)
    # query token s may read key t < L, and with the bottom-right causal mask only t <= L - S + s
    pairs = sum(1 for l in L for s in range(S) for t in range(l) if not causal or t <= l - S + s)
    assert flops == 2 * (576 + 512) * H * pairs
    assert kv == sum(L) * bpt
    pages = sum((x + 63) // 64 for x in L)
    assert byts == kv + B * S * H * (576 * 2 + 512 * 2 + 4) + pages * 4 + B * 4


def test_committed_counter_summaries_parse():
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.txt")))
    assert files, "no traffic summaries under profiles/"
    for f in files:
        kv = {}
        for line in open(f):
            if ":" in line and not line.startswith(("#", " ")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        for key in ("kernel", "workload", "source_sha256", "hbm_bytes_per_launch", "algorithmic_bytes_per_step",
                    "fetch_scale", "write_scale"):
            assert key in kv, f"{os.path.basename(f)} lacks {key}"
        ratio = int(kv["hbm_bytes_per_launch"]) / int(kv["algorithmic_bytes_per_step"])
        # sparse prefill: the algorithmic bytes count each listed kv row once, but every query token
        # gathers its own topk rows (2048 of 8192 for each of 4096 tokens), and the 9.4 MB kv array
        # does not stay in one XCD's 4 MB L2, so the L2-miss counters see up to s_q * topk rows
        limit = 10.0 if kv["workload"] == "sparse_prefill" else 3.0
        assert 0.9 < ratio < limit, f"{os.path.basename(f)}: traffic / algorithmic bytes = {ratio:.3f}"
        got = bench.stored_traffic(kv["kernel"], kv["workload"])
        assert got is None or got == int(kv["hbm_bytes_per_launch"])


def test_roofline_picks_the_bound_of_the_workload():
    # below the ridge (312.5 FLOP/B) the bound is HBM, above it dense bf16 MFMA
    r = bench.roofline(8_000_000, 8_000_000 * 100, 0.001)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and abs(r["achieved"] - 8000.0) < 1e-6 and r["frac"] == 1.0
    r = bench.roofline(1_000_000, 2_500_000_000, 0.001)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and abs(r["achieved"] - 2500.0) < 1e-6


def test_host_cores_follow_affinity_and_thread_cap(monkeypatch):
    n = len(os.sched_getaffinity(0))
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    assert bench.host_cores() == 1
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.host_cores() == n
    assert isinstance(bench.cpu_model(), str)
