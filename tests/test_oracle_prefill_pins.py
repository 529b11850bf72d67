"""Pins for the oracle's sparse prefill (oracle.mla_sparse_prefill):

* the pure-Python brute force on tiny cases (duplicates, -1 padding, h_kv in {1, 2});
* listing every row of kv equals dense attention over all rows: torch
  scaled_dot_product_attention in float64 and scipy's logsumexp;
* reordering, duplicating (LSE + ln 2) and padding invariants; errors; rows with no key.
Planted mistakes in the prefill path must each fail one of these.
"""
import inspect
import math
import types

import numpy as np
import pytest
import torch

import oracle.mla_oracle as base
from bruteforce import brute_force_sparse_prefill
from workloads import make_prefill_workload

CASES = [
    # s_q, h_q, h_kv, s_kv, topk, duplicates, padding, seed
    (3, 4, 1, 70, 9, 0.3, 0.2, 41),
    (2, 4, 2, 130, 6, 0.2, 0.1, 42),
    (2, 2, 1, 5, 8, 0.0, 0.0, 43),
]


def _run(w, m=base, idx=None):
    a = w.as_numpy()
    return m.mla_sparse_prefill(a["q_bits"], a["kv_bits"], a["indices"] if idx is None else idx, w.softmax_scale,
                                dv=w.dv)


def _case(c):
    Sq, H, Hk, Skv, k, dup, pad, seed = c
    return make_prefill_workload(name="pf", s_q=Sq, h_q=H, h_kv=Hk, s_kv=Skv, topk=k, duplicates=dup, padding=pad,
                                 seed=seed)


def _close(a, b, tol):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    inf = np.isneginf(a) & np.isneginf(b)
    return np.array_equal(np.isneginf(a), np.isneginf(b)) and np.all(np.abs(a[~inf] - b[~inf]) <= tol)


def _brute(w):
    a = w.as_numpy()
    return brute_force_sparse_prefill(a["q_bits"].tolist(), a["kv_bits"].tolist(), a["indices"].tolist(),
                                      w.softmax_scale, dv=w.dv)


@pytest.mark.parametrize("c", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_prefill_oracle_matches_bruteforce(c):
    w = _case(c)
    O, L = _run(w)
    Ob, Lb = _brute(w)
    assert _close(O, Ob, 1e-12) and _close(L, Lb, 1e-12)


def test_all_rows_listed_equals_dense_attention():
    from scipy.special import logsumexp
    w = make_prefill_workload(name="all", s_q=5, h_q=8, h_kv=2, s_kv=150, topk=150, seed=44)
    O, LSE = _run(w)
    kv = w.kv.to(torch.float64)
    q = w.q.to(torch.float64)
    G = 4
    for kvh in range(2):
        K = kv[:, kvh, :]
        Q = q[:, kvh * G:(kvh + 1) * G, :].reshape(-1, 576)
        o = torch.nn.functional.scaled_dot_product_attention(Q[None, None], K[None, None],
                                                             K[:, :512].contiguous()[None, None],
                                                             scale=w.softmax_scale)[0, 0]
        z = (w.softmax_scale * (Q @ K.T)).numpy()
        assert np.max(np.abs(O[:, kvh * G:(kvh + 1) * G, :].reshape(-1, 512) - o.numpy())) <= 1e-10
        assert np.max(np.abs(LSE[:, kvh * G:(kvh + 1) * G].reshape(-1) - logsumexp(z, axis=1))) <= 1e-10


def test_prefill_invariants_errors_and_empty_rows():
    w = _case(CASES[0])
    O, L = _run(w)
    idx = w.indices.numpy()
    rng = np.random.default_rng(45)
    perm = np.stack([rng.permutation(idx.shape[2]) for _ in range(idx.shape[0] * idx.shape[1])])
    Op, Lp = _run(w, idx=np.take_along_axis(idx.reshape(-1, idx.shape[2]), perm, 1).reshape(idx.shape))
    assert _close(Op, O, 1e-12) and _close(Lp, L, 1e-12)
    Od, Ld = _run(w, idx=np.concatenate([idx, idx], axis=2))
    fin = np.isfinite(L)
    assert _close(Od, O, 1e-12) and np.all(np.abs(Ld[fin] - L[fin] - math.log(2.0)) <= 1e-12)
    Oq, Lq = _run(w, idx=np.concatenate([np.full(idx.shape[:2] + (3,), -1), idx], axis=2))
    assert np.array_equal(Oq, O) and np.array_equal(Lq, L)
    bad = idx.copy()
    bad[1, 0, 0] = w.s_kv
    with pytest.raises(ValueError):
        _run(w, idx=bad)
    none = np.full_like(idx, -1)
    none[0, 0, 0] = 3
    Oe, Le = _run(w, idx=none)
    assert np.all(Oe[1:] == 0) and np.all(np.isneginf(Le[1:])) and np.all(np.isfinite(Le[0]))


PREFILL_MUTANTS = {
    "kv_head": ("K = bf16_bits_to_f64(kv[sel, kvh, :])", "K = bf16_bits_to_f64(kv[sel, 0, :])"),
    "dedupe": ("sel = row[keep]", "sel = np.unique(row[keep])"),
    "padding_kept": ("keep = row != -1", "keep = row != -2"),
    "value_tail": ("o, lse = attend(bf16_bits_to_f64(q[s, heads, :]), K, K[:, :dv], float(softmax_scale))",
                   "o, lse = attend(bf16_bits_to_f64(q[s, heads, :]), K, K[:, -dv:], float(softmax_scale))"),
    "scale_twice": ("K, K[:, :dv], float(softmax_scale))", "K, K[:, :dv], float(softmax_scale) ** 2)"),
    "head_map": ("heads = slice(kvh * G, (kvh + 1) * G)\n            o, lse",
                 "heads = slice(kvh, H, Hk)\n            o, lse"),
}


def _mutant(name):
    old, new = PREFILL_MUTANTS[name]
    src = inspect.getsource(base)
    assert src.count(old) == 1, f"mutant {name} no longer matches the oracle source"
    mod = types.ModuleType(f"oracle_prefill_mutant_{name}")
    exec(compile(src.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


def _fails(m):
    for c in CASES:
        w = _case(c)
        try:
            O, L = _run(w, m)
        except Exception:
            return True
        Ob, Lb = _brute(w)
        if not (_close(O, Ob, 1e-12) and _close(L, Lb, 1e-12)):
            return True
    return False


def test_unmutated_prefill_oracle_passes():
    assert not _fails(base)


@pytest.mark.parametrize("name", sorted(PREFILL_MUTANTS))
def test_prefill_mutant_is_caught(name):
    assert _fails(_mutant(name)), f"no pin caught the planted mistake {name!r}"
