"""GPU parity of decode with a separate V cache (vcache) against the oracle
(mla_decode(..., vcache=...)).

Tolerances as for the BF16 decode: O max-abs <= 1e-2, cosine >= 0.9999, LSE <= 1e-3; rows with
no allowed key give O = 0, LSE = -inf; a bad block-table entry makes its sequence NaN."""
import numpy as np
import pytest
import torch

import oracle
from workloads import make_workload, named_workload, permute_pages, poison_unused

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")


def run_vc(w, num_parts=0, vcache=None):
    import paged_mla_decode_amd as mla
    vc = (w.vcache if vcache is None else vcache).to(DEV)
    meta, splits = mla.mla_get_metadata(w.cache_seqlens, w.heads_per_kv, w.h_kv, kv_format="bf16",
                                        max_blocks_per_seq=int(w.block_table.shape[1]), num_parts=num_parts,
                                        device=DEV)
    o, lse = mla.mla_decode_kvcache(w.q.to(DEV), w.kvcache.to(DEV), w.block_table.to(DEV), w.cache_seqlens.to(DEV),
                                    w.dv, meta, splits, causal=w.causal, softmax_scale=w.softmax_scale, vcache=vc)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def compare(O, LSE, O_ref, LSE_ref, label):
    assert not np.any(np.isnan(O)) and not np.any(np.isinf(O)), f"{label}: non-finite O"
    assert not np.any(np.isnan(LSE)) and not np.any(np.isposinf(LSE)), f"{label}: NaN or +inf LSE"
    empty = np.isneginf(LSE_ref)
    assert np.array_equal(np.isneginf(LSE), empty), f"{label}: -inf LSE pattern differs"
    dO = float(np.max(np.abs(O - O_ref))) if O.size else 0.0
    dL = float(np.max(np.abs(LSE[~empty] - LSE_ref[~empty]))) if (~empty).any() else 0.0
    a, r = O.ravel(), O_ref.ravel()
    na, nr = np.linalg.norm(a), np.linalg.norm(r)
    cos = float(a @ r / (na * nr)) if na > 0 and nr > 0 else 1.0
    print(f"[parity] {label}: max|dO|={dO:.3e} cos={cos:.6f} max|dLSE|={dL:.3e}", flush=True)
    assert dO <= 1e-2 and dL <= 1e-3 and cos >= 0.9999, label
    assert np.all(np.moveaxis(O, 2, 1)[empty] == 0), f"{label}: rows without keys must be 0"


SMALL = [
    # name, batch, s_q, h_q, h_kv, lengths, causal
    ("rows16", 6, 1, 16, 1, [1, 31, 32, 33, 64, 1000], False),
    ("rows32_causal", 3, 2, 16, 1, [2, 130, 777], True),
    ("rows64", 2, 1, 64, 1, [70, 500], False),
    ("rows128", 3, 1, 128, 1, [5, 300, 2000], False),
    ("rows256_causal", 2, 2, 128, 1, [100, 1500], True),
    ("hkv2", 2, 2, 32, 2, [65, 400], True),
    ("hkv2_rows96", 2, 1, 192, 2, [129, 64], False),
    ("empty", 3, 1, 16, 1, [0, 40, 0], False),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("num_parts", [0, 1, 7])
def test_vcache_small_cases(case, num_parts):
    name, B, S, H, Hk, L, causal = case
    w = make_workload(name=name, batch=B, s_q=S, h_q=H, h_kv=Hk, seqlens=L, causal=causal, seed=400 + len(name),
                      pool_pages=sum((x + 63) // 64 for x in L) + 2, vcache=True)
    print(f"[case] vcache {name} parts={num_parts}", flush=True)
    O, LSE = run_vc(w, num_parts)
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(O, LSE, O_ref, LSE_ref, f"vcache {name}/parts={num_parts}")


def test_full_vcache_workload_every_sequence():
    w = named_workload("vcache")
    print(f"[case] full vcache: {w.meta.get('text')}", flush=True)
    O, LSE = run_vc(w)
    O2, LSE2 = run_vc(w)
    assert np.array_equal(O, O2) and np.array_equal(LSE, LSE2), "run-to-run results differ"
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(O, LSE, O_ref, LSE_ref, f"full vcache (all {w.batch} sequences)")


def test_vcache_holding_the_keys_matches_plain_decode():
    import paged_mla_decode_amd as mla
    w = make_workload(name="same", batch=3, s_q=2, h_q=64, seqlens=[70, 640, 1000], causal=True, seed=410)
    vc = w.kvcache[..., :512].contiguous()
    O, LSE = run_vc(w, vcache=vc)
    meta, splits = mla.mla_get_metadata(w.cache_seqlens, w.heads_per_kv, 1, device=DEV)
    o, l = mla.mla_decode_kvcache(w.q.to(DEV), w.kvcache.to(DEV), w.block_table.to(DEV), w.cache_seqlens.to(DEV),
                                  512, meta, splits, causal=True)
    torch.cuda.synchronize()
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(O, LSE, O_ref, LSE_ref, "vcache = keys")
    compare(o.float().cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64), O_ref, LSE_ref,
            "plain decode")


def test_vcache_page_permutation_poison_and_bad_page():
    w = make_workload(name="perm", batch=3, s_q=1, h_q=128, seqlens=[200, 65, 900], seed=411,
                      pool_pages=22, vcache=True)
    O, LSE = run_vc(w)
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(O, LSE, O_ref, LSE_ref, "vcache base")
    wp = permute_pages(w, 412)
    Op, Lp = run_vc(wp)
    compare(Op, Lp, O_ref, LSE_ref, "vcache permuted pages")
    wq = poison_unused(w)
    Oq, Lq = run_vc(wq)
    compare(Oq, Lq, O_ref, LSE_ref, "vcache poisoned unused bytes")
    wb = make_workload(name="badpg", batch=2, s_q=1, h_q=16, seqlens=[130, 100], seed=413, vcache=True)
    wb.block_table[1, 1] = 10_000
    Ob, Lb = run_vc(wb)
    assert np.all(np.isnan(Ob[1])) and np.all(np.isnan(Lb[1]))
    assert np.all(np.isfinite(Ob[0])) and np.all(np.isfinite(Lb[0]))
