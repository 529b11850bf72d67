"""GPU parity of token-level sparse decode against the oracle (mla_decode_sparse).

Tolerances as for dense decode: BF16 cache O max-abs <= 1e-2, cosine >= 0.9999, LSE <= 1e-3;
FP8 cache O <= 3e-2 against the oracle on the same records, LSE <= 1e-3. Rows with no
attended key give O = 0, LSE = -inf; an invalid entry makes that query token's rows NaN."""
import numpy as np
import pytest
import torch

import oracle
from workloads import dense_as_sparse, draw_indices, make_sparse_workload, make_workload, named_workload

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")
TOL_O = {"bf16": 1e-2, "fp8": 3e-2}


def run_sparse(w, num_parts=0, indices=None):
    import paged_mla_decode_amd as mla
    idx = (w.indices if indices is None else indices).to(DEV)
    meta, splits = mla.mla_get_metadata_sparse(w.batch, w.s_q, int(idx.shape[2]), w.h_q, w.h_kv,
                                               kv_format=w.kv_format, num_parts=num_parts, device=DEV)
    o, lse = mla.mla_decode_kvcache(w.q.to(DEV), w.kvcache.to(DEV), w.block_table.to(DEV), w.cache_seqlens.to(DEV),
                                    w.dv, meta, splits, causal=w.causal, softmax_scale=w.softmax_scale, indices=idx)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def compare(w, O, LSE, O_ref, LSE_ref, label):
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
    assert dO <= TOL_O[w.kv_format] and dL <= 1e-3, label
    if w.kv_format == "bf16":
        assert cos >= 0.9999, label
    assert np.all(np.moveaxis(O, 2, 1)[empty] == 0), f"{label}: rows without keys must be 0"


SMALL = [
    # name, batch, s_q, h_q, h_kv, lengths, causal, fmt, topk, duplicates, padding
    ("bf16_h128", 3, 1, 128, 1, [100, 2000, 700], False, "bf16", 300, 0.0, 0.0),
    ("bf16_h128_mtp", 2, 2, 128, 1, [900, 1500], True, "bf16", 257, 0.1, 0.1),
    ("bf16_h16", 3, 1, 16, 1, [64, 1000, 33], False, "bf16", 33, 0.2, 0.2),
    ("bf16_h64_hkv2", 2, 2, 128, 2, [400, 150], True, "bf16", 100, 0.0, 0.3),
    ("fp8_h128", 3, 1, 128, 1, [100, 3000, 700], False, "fp8", 512, 0.0, 0.0),
    ("fp8_h128_mtp", 2, 2, 128, 1, [1200, 2049], True, "fp8", 300, 0.1, 0.1),
    ("fp8_h64", 2, 1, 64, 1, [5000, 64], False, "fp8", 129, 0.3, 0.2),
    ("fp8_h256", 2, 1, 256, 1, [600, 300], False, "fp8", 64, 0.0, 0.0),
    ("fp8_topk1", 4, 1, 128, 1, [1, 2, 70, 9], False, "fp8", 1, 0.0, 0.0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("num_parts", [0, 1, 7])
def test_sparse_small_cases(case, num_parts):
    name, B, S, H, Hk, L, causal, fmt, topk, dup, pad = case
    w = make_sparse_workload(name=name, batch=B, s_q=S, h_q=H, h_kv=Hk, seqlens=L, causal=causal, kv_format=fmt,
                             seed=200 + len(name), topk=topk, duplicates=dup, padding=pad)
    if causal:   # positions from the whole sequence: the causal mask drops some of them
        w.indices = draw_indices(L, S, topk, False, np.random.default_rng(len(name)), dup, pad)
    print(f"[case] sparse {name} parts={num_parts}", flush=True)
    O, LSE = run_sparse(w, num_parts)
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(w, O, LSE, O_ref, LSE_ref, f"sparse {name}/parts={num_parts}")


def test_full_sparse_workload():
    w = named_workload("sparse_fp8")
    print(f"[case] full sparse_fp8: {w.meta.get('text')}", flush=True)
    O, LSE = run_sparse(w)
    O2, LSE2 = run_sparse(w)
    assert np.array_equal(O, O2) and np.array_equal(LSE, LSE2), "run-to-run results differ"
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(w, O, LSE, O_ref, LSE_ref, f"full sparse_fp8 (all {w.batch} sequences)")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_listing_every_token_matches_dense(fmt):
    import paged_mla_decode_amd as mla
    w = make_workload(name="all", batch=3, s_q=2, h_q=128, seqlens=[70, 640, 1000], causal=True, kv_format=fmt,
                      seed=211)
    ws = dense_as_sparse(w)
    O, LSE = run_sparse(ws)
    meta, splits = mla.mla_get_metadata(w.cache_seqlens, w.heads_per_kv, 1, kv_format=fmt, device=DEV)
    o, l = mla.mla_decode_kvcache(w.q.to(DEV), w.kvcache.to(DEV), w.block_table.to(DEV), w.cache_seqlens.to(DEV),
                                  512, meta, splits, causal=True)
    torch.cuda.synchronize()
    Od, Ld = o.float().cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64)
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(ws, O, LSE, O_ref, LSE_ref, f"every token listed ({fmt})")
    compare(w, Od, Ld, O_ref, LSE_ref, f"dense ({fmt})")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_invalid_entries_and_bad_pages_poison_only_their_query_token(fmt):
    w = make_sparse_workload(name="bad", batch=3, s_q=2, h_q=128, seqlens=[300, 200, 500], kv_format=fmt, seed=212,
                             topk=40)
    idx = w.indices.clone()
    idx[0, 1, 7] = 300                       # L_0 = 300: out of range
    idx[2, 0, 3] = -5                        # below -1
    O, LSE = run_sparse(w, indices=idx)
    for b, s in [(0, 1), (2, 0)]:
        assert np.all(np.isnan(O[b, s])) and np.all(np.isnan(LSE[b, :, s])), (b, s)
    ok = [(0, 0), (1, 0), (1, 1), (2, 1)]
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    for b, s in ok:
        assert np.max(np.abs(O[b, s] - O_ref[b, s])) <= TOL_O[fmt] and np.max(np.abs(LSE[b, :, s] - LSE_ref[b, :, s])) <= 1e-3
    # a block-table entry outside the pool behind an attended position
    w2 = make_sparse_workload(name="badpg", batch=2, s_q=1, h_q=128, seqlens=[200, 200], kv_format=fmt, seed=213,
                              topk=50)
    w2.indices[1, 0, :] = torch.arange(50, dtype=torch.int32)      # sequence 1 reads page entries 0
    w2.block_table[1, 0] = 10_000
    O, LSE = run_sparse(w2)
    assert np.all(np.isnan(O[1])) and np.all(np.isnan(LSE[1]))
    assert np.all(np.isfinite(O[0]))


def test_rows_without_keys():
    w = make_sparse_workload(name="none", batch=2, s_q=2, h_q=128, seqlens=[50, 3], causal=True, seed=214, topk=8)
    idx = torch.full_like(w.indices, -1)
    idx[0, 1, :3] = torch.tensor([0, 49, 20], dtype=torch.int32)   # (0, 1) attends 3 keys
    idx[1, 0, 0] = 2                                               # dropped by the causal mask (2 > 3 - 2 + 0)
    O, LSE = run_sparse(w, indices=idx)
    O_ref, LSE_ref = oracle.mla_decode_sparse(w.as_numpy()["q_bits"], w.as_numpy()["kvcache"], "bf16",
                                              w.block_table.numpy(), w.cache_seqlens.numpy(), idx.numpy(),
                                              causal=True, softmax_scale=w.softmax_scale)
    w.indices = idx
    compare(w, O, LSE, O_ref, LSE_ref, "rows without keys")
    assert np.all(O[0, 0] == 0) and np.all(np.isneginf(LSE[0, :, 0]))
