"""Pins for the oracle's token-level sparse decode (oracle.mla_decode_sparse), each tying
it to something other than itself:

* the pure-Python brute force (tests/bruteforce.py) on tiny cases with duplicates, -1
  padding, both causal flags, h_kv in {1, 2}, BF16 and FP8;
* listing every cached token once gives the dense oracle's result (itself pinned by brute
  force, SDPA and closed forms), and listing the first k tokens gives dense decode over a
  sequence of length k;
* invariants of the definition: reordering a row's list changes nothing, listing every entry
  twice leaves O and adds ln 2 to LSE, -1 entries change nothing;
* errors and empty rows.
Planted mistakes in the sparse path must each fail one of these.
"""
import inspect
import math
import types

import numpy as np
import pytest
import torch

import oracle
import oracle.mla_oracle as base
from bruteforce import brute_force_sparse_decode
from workloads import dense_as_sparse, draw_indices, make_sparse_workload, make_workload

CASES = [
    # (batch, s_q, h_q, h_kv, lengths, causal, fmt, topk, duplicates, padding, seed)
    (2, 1, 4, 1, [70, 130], False, "bf16", 9, 0.3, 0.2, 31),
    (2, 2, 4, 2, [65, 3], True, "bf16", 6, 0.2, 0.1, 32),
    (1, 2, 2, 1, [129], True, "fp8", 7, 0.3, 0.0, 33),
    (2, 1, 3, 1, [1, 64], False, "fp8", 5, 0.0, 0.3, 34),
]


def _sparse(w, m=base, indices=None):
    a = w.as_numpy()
    idx = (w.indices if indices is None else indices).numpy()
    return m.mla_decode_sparse(a["q_bits"], a["kvcache"], w.kv_format, a["block_table"], a["cache_seqlens"], idx,
                               dv=w.dv, causal=w.causal, softmax_scale=w.softmax_scale)


def _case(c):
    B, S, H, Hk, L, causal, fmt, topk, dup, pad, seed = c
    w = make_sparse_workload(name="sp", batch=B, s_q=S, h_q=H, h_kv=Hk, seqlens=L, causal=causal, kv_format=fmt,
                             seed=seed, topk=topk, duplicates=dup, padding=pad,
                             pool_pages=sum((x + 63) // 64 for x in L) + 2)
    if causal:
        # positions drawn from the whole sequence, so that the causal mask drops some of them
        w.indices = draw_indices(L, S, topk, False, np.random.default_rng(seed), dup, pad)
    return w


def _brute(w):
    a = w.as_numpy()
    return brute_force_sparse_decode(a["q_bits"].tolist(), a["kvcache"].tolist(), w.kv_format,
                                     a["block_table"].tolist(), a["cache_seqlens"].tolist(),
                                     w.indices.numpy().tolist(), dv=w.dv, causal=w.causal, scale=w.softmax_scale)


def _close(a, b, tol):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    both_inf = np.isneginf(a) & np.isneginf(b)
    return np.array_equal(np.isneginf(a), np.isneginf(b)) and np.all(np.abs(a[~both_inf] - b[~both_inf]) <= tol)


@pytest.mark.parametrize("c", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_sparse_oracle_matches_bruteforce(c):
    w = _case(c)
    O, LSE = _sparse(w)
    Ob, Lb = _brute(w)
    assert _close(O, Ob, 1e-12) and _close(LSE, Lb, 1e-12)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
def test_every_token_once_equals_dense(fmt, causal):
    w = make_workload(name="d", batch=3, s_q=2, h_q=8, h_kv=2, seqlens=[1, 130, 64], causal=causal, kv_format=fmt,
                      seed=35)
    O, LSE = oracle.mla_decode_workload(w)
    Os, Ls = oracle.mla_decode_workload(dense_as_sparse(w))
    assert _close(Os, O, 1e-12) and _close(Ls, LSE, 1e-12)


def test_first_k_tokens_equal_a_shorter_sequence():
    w = make_workload(name="pre", batch=2, s_q=1, h_q=4, seqlens=[200, 100], seed=36)
    k = [77, 100]
    idx = torch.full((2, 1, 100), -1, dtype=torch.int32)
    for b in range(2):
        idx[b, 0, :k[b]] = torch.arange(k[b])
    Os, Ls = _sparse(w, indices=idx)
    a = w.as_numpy()
    O, LSE = oracle.mla_decode(a["q_bits"], a["kvcache"], "bf16", a["block_table"], np.asarray(k),
                               softmax_scale=w.softmax_scale)
    assert _close(Os, O, 1e-12) and _close(Ls, LSE, 1e-12)


def test_reordering_duplicating_and_padding():
    w = _case(CASES[0])
    O, LSE = _sparse(w)
    rng = np.random.default_rng(37)
    perm = torch.from_numpy(np.stack([rng.permutation(w.topk) for _ in range(w.batch * w.s_q)]))
    idx_p = torch.gather(w.indices.view(-1, w.topk), 1, perm).view_as(w.indices)
    Op, Lp = _sparse(w, indices=idx_p)
    assert _close(Op, O, 1e-12) and _close(Lp, LSE, 1e-12)
    Od, Ld = _sparse(w, indices=torch.cat([w.indices, w.indices], dim=2))
    fin = np.isfinite(LSE)
    assert _close(Od, O, 1e-12) and np.all(np.abs(Ld[fin] - LSE[fin] - math.log(2.0)) <= 1e-12)
    pad = torch.full((w.batch, w.s_q, 5), -1, dtype=torch.int32)
    Oq, Lq = _sparse(w, indices=torch.cat([pad, w.indices, pad], dim=2))
    assert np.array_equal(Oq, O) and np.array_equal(Lq, LSE)


def test_errors_and_empty_rows():
    w = make_sparse_workload(name="e", batch=2, s_q=2, h_q=2, seqlens=[10, 3], causal=True, seed=38, topk=4)
    bad = w.indices.clone()
    bad[1, 0, 0] = 3                      # L_1 = 3: positions 0..2 only
    with pytest.raises(ValueError):
        _sparse(w, indices=bad)
    bad[1, 0, 0] = -2
    with pytest.raises(ValueError):
        _sparse(w, indices=bad)
    none = torch.full_like(w.indices, -1)
    none[0, 1, 2] = 9                     # one key for (0, 1); causal: 9 <= 10 - 2 + 1
    none[1, 0, 0] = 2                     # dropped by the causal mask: 2 > 3 - 2 + 0
    O, LSE = _sparse(w, indices=none)
    assert np.all(O[0, 0] == 0) and np.all(np.isneginf(LSE[0, :, 0]))
    assert np.all(O[1, 0] == 0) and np.all(np.isneginf(LSE[1, :, 0]))
    assert np.all(np.isfinite(LSE[0, :, 1]))


SPARSE_MUTANTS = {
    "dedupe": ("sel = row[row != -1]", "sel = np.unique(row[row != -1])"),
    "no_causal": ("            if causal:\n                sel = sel[sel <= L - S + s]",
                  "            if False:\n                sel = sel[sel <= L - S + s]"),
    "causal_top_left": ("sel = sel[sel <= L - S + s]", "sel = sel[sel <= s]"),
    "slot": ("kv[pages, sel % PAGE]", "kv[pages, (sel + 1) % PAGE]"),
    "page": ("pages = bt[b, sel // PAGE]", "pages = bt[b, sel // PAGE // 2]"),
    "value_from_key_tail": ("o, lse = attend(Qs, Kh, Kh[:, :dv], scale)",
                            "o, lse = attend(Qs, Kh, Kh[:, -dv:], scale)"),
    "head_map": ("Qs = bf16_bits_to_f64(q[b, s, heads, :])", "Qs = bf16_bits_to_f64(q[b, s, kvh::Hk, :])"),
    "lse_layout": ("LSE[b, heads, s] = lse", "LSE[b, heads, S - 1 - s] = lse"),
}


def _mutant(name):
    old, new = SPARSE_MUTANTS[name]
    src = inspect.getsource(base)
    assert src.count(old) == 1, f"mutant {name} no longer matches the oracle source"
    mod = types.ModuleType(f"oracle_sparse_mutant_{name}")
    exec(compile(src.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


def _sparse_pins_fail(m):
    for c in CASES:
        w = _case(c)
        try:
            O, LSE = _sparse(w, m)
        except Exception:
            return True
        Ob, Lb = _brute(w)
        if not (_close(O, Ob, 1e-12) and _close(LSE, Lb, 1e-12)):
            return True
    return False


def test_unmutated_sparse_oracle_passes():
    assert not _sparse_pins_fail(base)


@pytest.mark.parametrize("name", sorted(SPARSE_MUTANTS))
def test_sparse_mutant_is_caught(name):
    assert _sparse_pins_fail(_mutant(name)), f"no pin caught the planted mistake {name!r}"
