"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Tolerances: BF16 cache -- O max-abs <= 1e-2 and cosine >= 0.9999 (flattened,
float64), LSE max-abs <= 1e-3; FP8 cache -- O max-abs <= 3e-2 against the
oracle run on the same records (dequantised exactly), LSE max-abs <= 1e-3.
Rows with no allowed key must give O = 0 and LSE = -inf on both sides.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import make_workload, named_workload, permute_pages, poison_unused

pytestmark = pytest.mark.gpu

TOL_O = {"bf16": 1e-2, "fp8": 3e-2}
TOL_LSE = 1e-3
DEV = "cuda"


def run_gpu(w, num_parts=0, causal=None):
    import paged_mla_decode_amd as mla
    meta, splits = mla.mla_get_metadata(w.cache_seqlens, w.heads_per_kv, w.h_kv, kv_format=w.kv_format,
                                        num_parts=num_parts, device=torch.device(DEV))
    o, lse = mla.mla_decode_kvcache(w.q.to(DEV), w.kvcache.to(DEV), w.block_table.to(DEV), w.cache_seqlens.to(DEV),
                                    w.dv, meta, splits, causal=w.causal if causal is None else causal,
                                    softmax_scale=w.softmax_scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def compare(w, O, LSE, O_ref, LSE_ref, batches=None, label=""):
    if batches is not None:
        b = np.asarray(list(batches))
        O, LSE, O_ref, LSE_ref = O[b], LSE[b], O_ref[b], LSE_ref[b]
    empty = np.isneginf(LSE_ref)
    assert np.array_equal(np.isneginf(LSE), empty), f"{label}: -inf LSE pattern differs"
    assert np.all(np.isfinite(O)), f"{label}: non-finite O"
    dO = float(np.max(np.abs(O - O_ref))) if O.size else 0.0
    fin = ~empty
    dL = float(np.max(np.abs(LSE[fin] - LSE_ref[fin]))) if fin.any() else 0.0
    a, r = O.ravel(), O_ref.ravel()
    na, nr = np.linalg.norm(a), np.linalg.norm(r)
    cos = float(a @ r / (na * nr)) if na > 0 and nr > 0 else 1.0
    print(f"[parity] {label or w.name}: max|dO|={dO:.3e} cos={cos:.6f} max|dLSE|={dL:.3e} "
          f"max|O_ref|={float(np.max(np.abs(O_ref))) if O_ref.size else 0:.3f}", flush=True)
    assert dO <= TOL_O[w.kv_format], f"{label}: max|dO| = {dO}"
    assert dL <= TOL_LSE, f"{label}: max|dLSE| = {dL}"
    if w.kv_format == "bf16":
        assert cos >= 0.9999, f"{label}: cosine {cos}"
    # rows with no allowed key: O exactly 0
    Oe = np.moveaxis(O, 2, 1)                     # [B, H, S, dv] to line up with LSE [B, H, S]
    assert np.all(Oe[empty] == 0), f"{label}: empty rows must be exactly 0"


SMALL = [
    # name, batch, s_q, h_q, h_kv, lengths, causal, fmt
    ("rows16", 5, 1, 16, 1, [1, 63, 64, 65, 1000], False, "bf16"),
    ("rows8", 2, 1, 8, 1, [129, 3], False, "bf16"),
    ("rows32_causal", 3, 2, 16, 1, [2, 130, 777], True, "bf16"),
    ("rows48", 2, 1, 48, 1, [70, 500], False, "bf16"),
    ("rows128", 3, 1, 128, 1, [5, 300, 2000], False, "bf16"),
    ("rows256_causal", 2, 2, 128, 1, [100, 1500], True, "bf16"),
    ("rows80", 2, 1, 80, 1, [33, 97], False, "bf16"),
    ("rows192_causal", 2, 3, 64, 1, [31, 161], True, "bf16"),
    ("hkv2_rows128", 2, 1, 256, 2, [65, 320], False, "bf16"),
    ("hkv2", 2, 1, 32, 2, [90, 400], False, "bf16"),
    ("fp8_rows16", 3, 1, 16, 1, [64, 200, 1025], False, "fp8"),
    ("fp8_rows128", 2, 1, 128, 1, [33, 1100], False, "fp8"),
    ("fp8_rows256_causal", 2, 2, 128, 1, [3, 700], True, "fp8"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("num_parts", [0, 1, 7])
def test_small_cases(case, num_parts):
    name, B, S, H, Hk, L, causal, fmt = case
    w = make_workload(name=name, batch=B, s_q=S, h_q=H, h_kv=Hk, seqlens=L, causal=causal, kv_format=fmt,
                      seed=100 + len(name), pool_pages=sum((x + 63) // 64 for x in L) + 5)
    print(f"[case] {name} num_parts={num_parts}", flush=True)
    O, LSE = run_gpu(w, num_parts=num_parts)
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(w, O, LSE, O_ref, LSE_ref, label=f"{name}/parts={num_parts}")


_FULL = {}


def full(name):
    if name not in _FULL:
        _FULL.clear()
        _FULL[name] = named_workload(name)
    return _FULL[name]


# (workload, sequences the oracle checks: None = all)
FULL_CASES = [
    ("tiny", None),
    ("compute_heavy", None),
    ("mtp", [0, 1, 37, 64, 100, 127]),
    ("ragged", None),
    ("uniform_long", [0, 5, 63, 64, 100, 127]),
    ("fp8", [0, 1, 31, 62, 63]),
]


@pytest.mark.parametrize("name,batches", FULL_CASES, ids=[c[0] for c in FULL_CASES])
def test_full_size_workloads(name, batches):
    w = full(name)
    print(f"[case] full {name}: {w.meta.get('text')} pages={w.num_pages}", flush=True)
    O, LSE = run_gpu(w)
    if name == "ragged":
        batches = None
    O_ref, LSE_ref = oracle.mla_decode_workload(w, batches=batches)
    compare(w, O, LSE, O_ref, LSE_ref, batches=batches, label=f"full {name}")
    if name == "ragged":
        long_b = int(np.argmax(w.cache_seqlens.numpy()))
        compare(w, O, LSE, O_ref, LSE_ref, batches=[long_b], label="full ragged, the 32768-token sequence")


def test_full_compute_heavy_causal_flag_is_noop():
    w = full("compute_heavy")
    O1, L1 = run_gpu(w, causal=False)
    O2, L2 = run_gpu(w, causal=True)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


@pytest.mark.parametrize("num_parts", [1, 3, 64, 256, 1024])
def test_num_parts_invariance(num_parts):
    w = make_workload(name="parts", batch=6, s_q=2, h_q=64, seqlens=[1, 64, 500, 3000, 0, 129], causal=True, seed=55,
                      pool_pages=80)
    O, LSE = run_gpu(w, num_parts=num_parts)
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(w, O, LSE, O_ref, LSE_ref, label=f"num_parts={num_parts}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_page_permutation_and_determinism(fmt):
    w = make_workload(name="perm", batch=4, s_q=1, h_q=128, seqlens=[700, 64, 2000, 9], kv_format=fmt, seed=56,
                      pool_pages=60)
    O1, L1 = run_gpu(w)
    O1b, L1b = run_gpu(w)
    assert np.array_equal(O1, O1b) and np.array_equal(L1, L1b), "run-to-run results differ"
    O2, L2 = run_gpu(permute_pages(w, 3))
    bitwise = np.array_equal(O1, O2) and np.array_equal(L1, L2)
    print(f"[perm] {fmt}: bitwise identical after page permutation: {bitwise}", flush=True)
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(w, O2, L2, O_ref, LSE_ref, label=f"permuted {fmt}")
    assert bitwise


@pytest.mark.parametrize("h_q", [16, 128])
@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_poisoned_tails_and_unused_pages(fmt, h_q):
    w = make_workload(name="poison", batch=3, s_q=2, h_q=h_q, seqlens=[100, 37, 640], causal=True, kv_format=fmt,
                      seed=57, max_blocks=12)
    O1, L1 = run_gpu(w)
    O2, L2 = run_gpu(poison_unused(w))
    assert np.all(np.isfinite(O2))
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_single_token_gives_value_row_exactly():
    w = make_workload(name="L1", batch=4, s_q=1, h_q=128, seqlens=[1, 1, 1, 1], seed=58, pool_pages=9)
    O, LSE = run_gpu(w)
    a = w.as_numpy()
    for b in range(4):
        v = oracle.bf16_bits_to_f64(a["kvcache"][a["block_table"][b, 0], 0, 0, :512])
        assert np.array_equal(O[b, 0], np.broadcast_to(v, O[b, 0].shape))
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(w, O, LSE, O_ref, LSE_ref, label="L=1")


@pytest.mark.parametrize("h_q", [16, 32, 128])
def test_empty_and_fully_masked_rows(h_q):
    w = make_workload(name="empty", batch=4, s_q=2, h_q=h_q, seqlens=[0, 1, 2, 70], causal=True, seed=59,
                      max_blocks=3)
    for parts in (0, 1, 9):
        O, LSE = run_gpu(w, num_parts=parts)
        O_ref, LSE_ref = oracle.mla_decode_workload(w)
        compare(w, O, LSE, O_ref, LSE_ref, label=f"empty rows parts={parts}")
        assert np.all(O[0] == 0) and np.all(np.isneginf(LSE[0]))
        assert np.all(O[1, 0] == 0) and np.all(np.isneginf(LSE[1, :, 0]))


@pytest.mark.parametrize("h_q", [16, 32, 64])
def test_sequences_without_pages_between_pages(h_q):
    # ranges that start with, and step over, sequences of length 0: the page ring keeps the
    # next pages in flight across them while their (empty) outputs and merges are written
    w = make_workload(name="gaps", batch=8, s_q=1, h_q=h_q, seqlens=[0, 0, 65, 0, 1, 0, 130, 0], seed=63,
                      max_blocks=3)
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    for parts in (0, 1, 2, 3):
        O, LSE = run_gpu(w, num_parts=parts)
        compare(w, O, LSE, O_ref, LSE_ref, label=f"gaps h_q={h_q} parts={parts}")


@pytest.mark.parametrize("h_q", [16, 128])
def test_invalid_block_table_entry_poisons_only_its_sequence(h_q):
    w = make_workload(name="badpage", batch=3, s_q=1, h_q=h_q, seqlens=[100, 200, 50], seed=60)
    w.block_table[1, 2] = 10_000
    O, LSE = run_gpu(w)
    assert np.all(np.isnan(O[1])) and np.all(np.isnan(LSE[1]))
    w_ok = make_workload(name="badpage", batch=3, s_q=1, h_q=h_q, seqlens=[100, 200, 50], seed=60)
    O_ref, LSE_ref = oracle.mla_decode_workload(w_ok, batches=[0, 2])
    compare(w_ok, O, LSE, O_ref, LSE_ref, batches=[0, 2], label="sequences next to a bad page")


@pytest.mark.parametrize("h_q", [32, 128])
def test_noncontiguous_q_and_custom_scale(h_q):
    w = make_workload(name="strided", batch=2, s_q=2, h_q=h_q, seqlens=[333, 90], causal=True, seed=61,
                      softmax_scale=0.07)
    big = torch.zeros(2, 2, h_q + 8, 576, dtype=torch.bfloat16)
    big[:, :, 4:4 + h_q] = w.q
    w.q = big[:, :, 4:4 + h_q]                   # head stride 576, batch stride 2*(h_q+8)*576
    assert not w.q.is_contiguous()
    import paged_mla_decode_amd as mla
    meta, splits = mla.mla_get_metadata(w.cache_seqlens, w.heads_per_kv, 1, device=torch.device(DEV))
    o, lse = mla.mla_decode_kvcache(big.to(DEV)[:, :, 4:4 + h_q], w.kvcache.to(DEV), w.block_table.to(DEV),
                                    w.cache_seqlens.to(DEV), 512, meta, splits, causal=True, softmax_scale=0.07)
    torch.cuda.synchronize()
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(w, o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), O_ref, LSE_ref,
            label="strided q, scale 0.07")
