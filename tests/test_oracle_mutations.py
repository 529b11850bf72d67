"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is one textual edit of oracle/mla_oracle.py (a dropped term, a
wrong sign, index or offset, a wrong base), executed as a throw-away module on
the CPU. The pins it is run against are the independent ones from
test_oracle_pins.py: the pure-Python brute force, torch SDPA with an explicit
mask, the one-key closed form, the split merge and the e4m3fn table.
"""
import functools
import inspect
import math
import types

import numpy as np
import pytest
import torch

import oracle.mla_oracle as base
from bruteforce import brute_force_decode
from workloads import make_workload

MUTANTS = {
    "slot_index": ("rows = kvcache[pages, t % PAGE]", "rows = kvcache[pages, t % 32]"),
    "page_index": ("[t // PAGE].astype(np.int64)", "[t // 32 % block_table_row.shape[0]].astype(np.int64)"),
    "head_map": ("q[b, s, kvh * G:(kvh + 1) * G, :]", "q[b, s, kvh::Hk, :]"),
    "causal_top_left": ("last = (L - S + s) if causal", "last = s if causal"),
    "value_slice": ("Vh = Kh[:, :dv]", "Vh = Kh[:, -dv:]"),
    "dropped_rope_term": ("z = scale * (Q @ K.T)", "z = scale * (Q[:, :512] @ K[:, :512].T)"),
    "scale_twice": ("z = scale * (Q @ K.T)", "z = scale * scale * (Q @ K.T)"),
    "lse_base2": ("lse = mx + np.log(np.exp", "lse = mx + np.log2(np.exp"),
    "unnormalised": ("p = np.exp(z - lse[:, None])", "p = np.exp(z - mx[:, None])"),
    "fp8_scale_order": ("scales[..., :, None]", "scales[..., ::-1, None]"),
    "fp8_rope_offset": ("rope_bits = r[..., 528:656]", "rope_bits = r[..., 526:654]"),
    "e4m3_bias": ("np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    "e4m3_subnormal": ("(m / 8.0) * 2.0 ** -6", "(m / 8.0) * 2.0 ** -7"),
    "e4m3_sign": ("sign = np.where(c & 0x80, -1.0, 1.0)", "sign = np.where(c & 0x40, -1.0, 1.0)"),
    "combine_sign": ("w = np.where(finite, np.exp(L[i] - np.where(finite, lse, 0.0)), 0.0)",
                     "w = np.where(finite, np.exp(np.where(finite, lse, 0.0) - L[i]), 0.0)"),
    "lse_layout": ("LSE[b, kvh * G:(kvh + 1) * G, s] = lse", "LSE[b, kvh * G:(kvh + 1) * G, S - 1 - s] = lse"),
    "bf16_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
}


def _mutant_module(name):
    old, new = MUTANTS[name]
    src = inspect.getsource(base)
    assert src.count(old) == 1, f"mutant {name} no longer matches the oracle source"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


@functools.lru_cache(maxsize=None)
def _cases():
    out = []
    for (B, S, H, Hk, L, causal, fmt, seed) in [(2, 2, 4, 2, [65, 128], True, "bf16", 41),
                                                (2, 2, 2, 1, [2, 70], True, "fp8", 42)]:
        w = make_workload(name="m", batch=B, s_q=S, h_q=H, h_kv=Hk, seqlens=L, causal=causal, kv_format=fmt,
                          seed=seed, pool_pages=sum((x + 63) // 64 for x in L) + 2)
        a = w.as_numpy()
        Ob, Lb = brute_force_decode(a["q_bits"].tolist(), a["kvcache"].tolist(), fmt, a["block_table"].tolist(),
                                    a["cache_seqlens"].tolist(), causal=causal, scale=w.softmax_scale)
        out.append((w, np.asarray(Ob), np.asarray(Lb)))
    return out


def _pins_fail(m) -> list:
    failed = []
    # brute force
    for w, Ob, Lb in _cases():
        a = w.as_numpy()
        try:
            O, L = m.mla_decode(a["q_bits"], a["kvcache"], w.kv_format, a["block_table"], a["cache_seqlens"],
                                causal=w.causal, softmax_scale=w.softmax_scale)
            if not (np.max(np.abs(O - Ob)) <= 1e-12 and np.max(np.abs(L - Lb)) <= 1e-12):
                failed.append("bruteforce")
        except Exception:
            failed.append("bruteforce-raised")
    # split merge
    g = np.random.default_rng(5)
    Q, K = g.standard_normal((3, 576)), g.standard_normal((90, 576))
    O, l = m.attend(Q, K, K[:, :512], 0.05)
    O1, l1 = m.attend(Q, K[:40], K[:40, :512], 0.05)
    O2, l2 = m.attend(Q, K[40:], K[40:, :512], 0.05)
    Oc, lc = m.combine_partials([O1, O2], [l1, l2])
    if not (np.max(np.abs(Oc - O)) <= 1e-12 and np.max(np.abs(lc - l)) <= 1e-12):
        failed.append("split-merge")
    # e4m3fn table
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = m.e4m3fn_to_f64(codes)
    ok = ~np.isnan(ref)
    if not np.array_equal(ours[ok], ref[ok]):
        failed.append("e4m3fn")
    return failed


def test_unmutated_oracle_passes_every_pin():
    assert _pins_fail(base) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert _pins_fail(_mutant_module(name)), f"no pin caught the planted mistake {name!r}"
