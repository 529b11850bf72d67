"""Pins for the oracle's separate V cache (mla_decode(..., vcache=...)):

* the pure-Python brute force with V rows from the V cache (BF16 and FP8 keys, causal, h_kv = 2);
* a V cache holding the keys' first 512 dims gives exactly the result without one;
* closed forms: every V row equal to c gives O = c, and the LSE never depends on V;
* O is linear in V (exact bf16 sums of values on a coarse grid);
* page permutation and poisoned unused bytes leave the result unchanged; bad shapes raise.
Planted mistakes in the V-cache path must each fail one of these.
"""
import inspect
import types

import numpy as np
import pytest
import torch

import oracle
import oracle.mla_oracle as base
from bruteforce import brute_force_decode
from workloads import make_workload, permute_pages, poison_unused

CASES = [
    # (batch, s_q, h_q, h_kv, lengths, causal, fmt, seed)
    (2, 1, 4, 1, [1, 130], False, "bf16", 51),
    (2, 2, 4, 2, [65, 128], True, "bf16", 52),
    (1, 1, 3, 1, [129], False, "fp8", 53),
]


def _case(c, **kw):
    B, S, H, Hk, L, causal, fmt, seed = c
    return make_workload(name="vc", batch=B, s_q=S, h_q=H, h_kv=Hk, seqlens=L, causal=causal, kv_format=fmt,
                         seed=seed, pool_pages=sum((x + 63) // 64 for x in L) + 2, vcache=True, **kw)


def _run(w, m=base, vcache="w"):
    a = w.as_numpy()
    vc = a.get("vcache") if isinstance(vcache, str) else vcache
    return m.mla_decode(a["q_bits"], a["kvcache"], w.kv_format, a["block_table"], a["cache_seqlens"], dv=w.dv,
                        causal=w.causal, softmax_scale=w.softmax_scale, vcache=vc)


def _brute(w):
    a = w.as_numpy()
    return brute_force_decode(a["q_bits"].tolist(), a["kvcache"].tolist(), w.kv_format, a["block_table"].tolist(),
                              a["cache_seqlens"].tolist(), dv=w.dv, causal=w.causal, scale=w.softmax_scale,
                              vcache=a["vcache"].tolist())


def _close(a, b, tol):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    inf = np.isneginf(a) & np.isneginf(b)
    return np.array_equal(np.isneginf(a), np.isneginf(b)) and bool(np.all(np.abs(a[~inf] - b[~inf]) <= tol))


@pytest.mark.parametrize("c", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_vcache_oracle_matches_bruteforce(c):
    w = _case(c)
    O, L = _run(w)
    Ob, Lb = _brute(w)
    assert _close(O, Ob, 1e-12) and _close(L, Lb, 1e-12)


def test_vcache_holding_the_keys_equals_no_vcache():
    w = _case(CASES[1])
    kv = w.kvcache
    vc = kv[..., :512].contiguous().view(torch.int16).numpy().view(np.uint16)
    O1, L1 = _run(w, vcache=vc)
    O0, L0 = _run(w, vcache=None)
    assert np.array_equal(O1, O0) and np.array_equal(L1, L0)


def test_constant_values_and_lse_independent_of_v():
    w = _case(CASES[1])
    c = np.linspace(-2.0, 2.0, 512).astype(np.float32)
    cbits = (torch.from_numpy(c).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    vc = np.broadcast_to(cbits, w.vcache.shape).copy()
    O, L = _run(w, vcache=vc)
    cval = torch.from_numpy(c).to(torch.bfloat16).double().numpy()
    fin = np.isfinite(L)
    assert np.max(np.abs(O[np.moveaxis(fin, 1, 2)] - cval)) <= 1e-12
    _, L0 = _run(w, vcache=None)
    assert np.array_equal(L, L0)


def test_linear_in_v():
    w = _case(CASES[0])
    rng = np.random.default_rng(54)
    v1 = rng.integers(-64, 65, size=w.vcache.shape) / 64.0          # exact in bf16, and so are the sums
    v2 = rng.integers(-64, 65, size=w.vcache.shape) / 64.0
    tob = lambda v: torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    O1, _ = _run(w, vcache=tob(v1))
    O2, _ = _run(w, vcache=tob(v2))
    O12, _ = _run(w, vcache=tob(v1 + v2))
    assert np.max(np.abs(O12 - (O1 + O2))) <= 1e-12


def test_vcache_invariants_and_errors():
    w = _case(CASES[1])
    O, L = _run(w)
    Op, Lp = _run(permute_pages(w, 55))
    assert _close(Op, O, 1e-12) and _close(Lp, L, 1e-12)
    Oq, Lq = _run(poison_unused(w))
    assert _close(Oq, O, 1e-12) and _close(Lq, L, 1e-12)
    with pytest.raises(ValueError):
        _run(w, vcache=w.as_numpy()["vcache"][:, :, :, :256])


VC_MUTANTS = {
    "ignore_vcache": ("            if Vsep is not None:\n                Vh = Vsep[:, kvh, :]",
                      "            if False:\n                Vh = Vsep[:, kvh, :]"),
    "v_head0": ("Vh = Vsep[:, kvh, :]", "Vh = Vsep[:, 0, :]"),
    "v_slot": ("return bf16_bits_to_f64(np.asarray(vcache)[page_of, t % PAGE])",
               "return bf16_bits_to_f64(np.asarray(vcache)[page_of, (t + 1) % PAGE])"),
    "v_page": ("page_of = np.asarray(block_table_row).astype(np.int64)[t // PAGE]",
               "page_of = np.asarray(block_table_row).astype(np.int64)[t // PAGE][::-1]"),
}


def _mutant(name):
    old, new = VC_MUTANTS[name]
    src = inspect.getsource(base)
    assert src.count(old) == 1, f"mutant {name} no longer matches the oracle source"
    mod = types.ModuleType(f"oracle_vc_mutant_{name}")
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


def test_unmutated_vcache_oracle_passes():
    assert not _fails(base)


@pytest.mark.parametrize("name", sorted(VC_MUTANTS))
def test_vcache_mutant_is_caught(name):
    assert _fails(_mutant(name)), f"no pin caught the planted mistake {name!r}"
