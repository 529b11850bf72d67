"""GPU parity of sparse prefill (flash_mla_sparse_fwd through mla_sparse_prefill_fwd) against
the oracle (mla_sparse_prefill).

Tolerances as for BF16 decode: O max-abs <= 1e-2, cosine >= 0.9999, LSE <= 1e-3. Tokens with
no listed row give O = 0, LSE = -inf; an entry outside [-1, s_kv) makes the rows of that
(token, KV head) NaN."""
import numpy as np
import pytest
import torch

import oracle
from workloads import make_prefill_workload, named_prefill

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")


def run_prefill(w, num_parts=0, indices=None):
    import paged_mla_decode_amd as mla
    idx = (w.indices if indices is None else indices).to(DEV)
    o, lse = mla.flash_mla_sparse_fwd(w.q.to(DEV), w.kv.to(DEV), idx, w.softmax_scale, w.dv, num_parts=num_parts)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def ref(w, indices=None, tokens=None):
    a = w.as_numpy()
    idx = a["indices"] if indices is None else indices.numpy()
    return oracle.mla_sparse_prefill(a["q_bits"], a["kv_bits"], idx, w.softmax_scale, dv=w.dv, tokens=tokens)


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
    assert np.all(O[empty] == 0), f"{label}: rows without keys must be 0"


SMALL = [
    # name, s_q, h_q, h_kv, s_kv, topk, duplicates, padding
    ("h128", 5, 128, 1, 1000, 300, 0.0, 0.0),
    ("h128_ragged", 7, 128, 1, 333, 129, 0.2, 0.2),
    ("h128_topk_over_skv", 3, 128, 1, 70, 200, 0.0, 0.0),      # every row, then -1 padding
    ("h16", 6, 16, 1, 2000, 64, 0.1, 0.1),
    ("h64_hkv2", 4, 64, 2, 500, 100, 0.0, 0.3),
    ("h256", 2, 256, 1, 640, 65, 0.0, 0.0),
    ("topk1", 9, 128, 1, 10, 1, 0.0, 0.0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("num_parts", [0, 1, 5])
def test_prefill_small_cases(case, num_parts):
    name, Sq, H, Hk, Skv, topk, dup, pad = case
    w = make_prefill_workload(name=name, s_q=Sq, h_q=H, h_kv=Hk, s_kv=Skv, topk=topk, duplicates=dup, padding=pad,
                              seed=300 + len(name))
    print(f"[case] prefill {name} parts={num_parts}", flush=True)
    O, LSE = run_prefill(w, num_parts)
    O_ref, LSE_ref = ref(w)
    compare(O, LSE, O_ref, LSE_ref, f"prefill {name}/parts={num_parts}")


def test_full_prefill_workload_sampled_tokens():
    w = named_prefill("sparse_prefill")
    print(f"[case] full sparse_prefill: {w.meta.get('text')}", flush=True)
    O, LSE = run_prefill(w)
    O2, LSE2 = run_prefill(w)
    assert np.array_equal(O, O2) and np.array_equal(LSE, LSE2), "run-to-run results differ"
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(LSE))
    rng = np.random.default_rng(301)
    tokens = sorted({0, w.s_q - 1, *rng.choice(w.s_q, 46, replace=False).tolist()})
    O_ref, LSE_ref = ref(w, tokens=tokens)
    compare(O[tokens], LSE[tokens], O_ref, LSE_ref, f"full sparse_prefill ({len(tokens)} tokens)")


def test_invalid_entries_poison_only_their_token_and_kv_head():
    w = make_prefill_workload(name="bad", s_q=4, h_q=64, h_kv=2, s_kv=300, topk=40, seed=302)
    idx = w.indices.clone()
    idx[1, 0, 7] = 300                       # s_kv = 300: out of range
    idx[3, 1, 3] = -5                        # below -1
    O, LSE = run_prefill(w, indices=idx)
    assert np.all(np.isnan(O[1, :32])) and np.all(np.isnan(LSE[1, :32]))
    assert np.all(np.isnan(O[3, 32:])) and np.all(np.isnan(LSE[3, 32:]))
    O_ref, LSE_ref = ref(w)
    for s, heads in [(0, slice(0, 64)), (1, slice(32, 64)), (2, slice(0, 64)), (3, slice(0, 32))]:
        assert np.max(np.abs(O[s, heads] - O_ref[s, heads])) <= 1e-2
        assert np.max(np.abs(LSE[s, heads] - LSE_ref[s, heads])) <= 1e-3


def test_tokens_without_rows():
    w = make_prefill_workload(name="none", s_q=3, h_q=128, s_kv=50, topk=8, seed=303)
    idx = torch.full_like(w.indices, -1)
    idx[1, 0, :3] = torch.tensor([0, 49, 20], dtype=torch.int32)
    O, LSE = run_prefill(w, indices=idx)
    O_ref, LSE_ref = ref(w, indices=idx)
    compare(O, LSE, O_ref, LSE_ref, "tokens without rows")
    assert np.all(O[0] == 0) and np.all(np.isneginf(LSE[2]))


def test_prefill_matches_sparse_decode_on_the_same_rows():
    """The same attention posed as sparse decode (one sequence of s_kv cached tokens, every
    query token its own query position) gives the same bits: both run the same kernels over
    the same entries."""
    import paged_mla_decode_amd as mla
    w = make_prefill_workload(name="eq", s_q=6, h_q=128, s_kv=700, topk=150, seed=304)
    O, LSE = run_prefill(w)
    Skv = w.s_kv
    npg = (Skv + 63) // 64
    pool = torch.zeros((npg * 64, 1, 576), dtype=torch.bfloat16)
    pool[:Skv] = w.kv
    kvcache = pool.view(npg, 64, 1, 576).to(DEV)
    bt = torch.arange(npg, dtype=torch.int32).view(1, npg)
    q = w.q.view(1, w.s_q, w.h_q, 576)
    idx = w.indices.view(1, w.s_q, w.topk)
    meta, splits = mla.mla_get_metadata_sparse(1, w.s_q, w.topk, w.h_q, 1, device=DEV)
    o, lse = mla.mla_decode_kvcache(q.to(DEV), kvcache, bt.to(DEV), torch.tensor([Skv], dtype=torch.int32, device=DEV),
                                    512, meta, splits, causal=False, softmax_scale=w.softmax_scale, indices=idx.to(DEV))
    torch.cuda.synchronize()
    Od = o.float().cpu().numpy().astype(np.float64)[0]
    Ld = lse.cpu().numpy().astype(np.float64)[0].T
    assert np.array_equal(O, Od) and np.array_equal(LSE, Ld)
