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


def run_gpu(w, num_parts=0, causal=None, meta_lengths=None, edit_splits=None):
    """Decode `w` on the GPU. meta_lengths: build the metadata for these lengths instead
    (unchecked against the block table); edit_splits(num_splits_host) may rewrite num_splits."""
    import paged_mla_decode_amd as mla
    dev = torch.device(DEV)
    if meta_lengths is None and edit_splits is None:
        meta, splits = mla.mla_get_metadata(w.cache_seqlens, w.heads_per_kv, w.h_kv, kv_format=w.kv_format,
                                            max_blocks_per_seq=int(w.block_table.shape[1]), num_parts=num_parts,
                                            device=dev)
    else:
        L = w.cache_seqlens if meta_lengths is None else torch.tensor(meta_lengths, dtype=torch.int32)
        meta_h, splits_h = mla.mla_get_metadata_host(L, w.heads_per_kv, w.h_kv, kv_format=w.kv_format,
                                                     num_parts=num_parts)
        if edit_splits is not None:
            edit_splits(splits_h)
        meta, splits = meta_h.to(dev), splits_h.to(dev)
    o, lse = mla.mla_decode_kvcache(w.q.to(DEV), w.kvcache.to(DEV), w.block_table.to(DEV), w.cache_seqlens.to(DEV),
                                    w.dv, meta, splits, causal=w.causal if causal is None else causal,
                                    softmax_scale=w.softmax_scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def compare(w, O, LSE, O_ref, LSE_ref, batches=None, label=""):
    # every output is checked for NaN/inf before any subset is taken
    assert not np.any(np.isnan(O)) and not np.any(np.isinf(O)), f"{label}: non-finite O"
    assert not np.any(np.isnan(LSE)) and not np.any(np.isposinf(LSE)), f"{label}: NaN or +inf LSE"
    if batches is not None:
        b = np.asarray(list(batches))
        O, LSE, O_ref, LSE_ref = O[b], LSE[b], O_ref[b], LSE_ref[b]
    empty = np.isneginf(LSE_ref)
    assert np.array_equal(np.isneginf(LSE), empty), f"{label}: -inf LSE pattern differs"
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
    ("fp8_rows8", 2, 1, 8, 1, [129, 3], False, "fp8"),
    ("fp8_rows32_causal", 3, 2, 16, 1, [2, 130, 777], True, "fp8"),
    ("fp8_rows48", 2, 1, 48, 1, [70, 500], False, "fp8"),
    ("fp8_rows64", 2, 1, 64, 1, [65, 900], False, "fp8"),
    ("fp8_rows64_causal", 2, 2, 32, 1, [3, 600], True, "fp8"),
    ("fp8_rows80", 2, 1, 80, 1, [33, 97], False, "fp8"),
    ("fp8_rows128", 2, 1, 128, 1, [33, 1100], False, "fp8"),
    ("fp8_rows192_causal", 2, 3, 64, 1, [31, 161], True, "fp8"),
    ("fp8_rows256_causal", 2, 2, 128, 1, [3, 700], True, "fp8"),
    ("fp8_hkv2", 2, 1, 32, 2, [90, 400], False, "fp8"),
    ("fp8_hkv2_rows64", 2, 1, 128, 2, [200, 70], False, "fp8"),
    ("fp8_hkv2_rows128", 2, 1, 256, 2, [65, 320], False, "fp8"),
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


FULL_CASES = ["tiny", "compute_heavy", "mtp", "ragged", "uniform_long", "fp8"]


@pytest.mark.parametrize("name", FULL_CASES)
def test_full_size_workloads(name):
    """Every sequence of every full-size workload against the oracle, in the launch
    configuration the benchmark times (default number of ranges); a second run must be
    bitwise identical."""
    w = full(name)
    print(f"[case] full {name}: {w.meta.get('text')} pages={w.num_pages}", flush=True)
    O, LSE = run_gpu(w)
    O2, LSE2 = run_gpu(w)
    assert np.array_equal(O, O2) and np.array_equal(LSE, LSE2), f"full {name}: run-to-run results differ"
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(w, O, LSE, O_ref, LSE_ref, label=f"full {name} (all {w.batch} sequences)")
    if name == "ragged":
        long_b = int(np.argmax(w.cache_seqlens.numpy()))
        compare(w, O, LSE, O_ref, LSE_ref, batches=[long_b], label="full ragged, the 32768-token sequence")


@pytest.mark.parametrize("h_q,s_q", [(16, 1), (16, 2), (32, 1), (64, 1)])
def test_fp8_narrow_tiles_many_pieces(h_q, s_q):
    """FP8 records with up to 64 query rows per KV head (the 64-row kernels' FP8 variants, e.g.
    16 heads per GPU) at a size where every sequence spans many pages and, in the default launch
    configuration, several pieces (one with more than 16), so the fp32 partials and the
    many-piece combine run; every sequence against the oracle, and a bitwise rerun."""
    rng = np.random.default_rng(71 + h_q + s_q)
    lens = [int(x) for x in rng.integers(600, 3000, size=23)] + [12000]
    w = make_workload(name=f"fp8_narrow_h{h_q}_s{s_q}", batch=24, s_q=s_q, h_q=h_q, seqlens=lens,
                      causal=s_q > 1, kv_format="fp8", seed=72 + h_q)
    O, LSE = run_gpu(w)
    O2, LSE2 = run_gpu(w)
    assert np.array_equal(O, O2) and np.array_equal(LSE, LSE2), "run-to-run results differ"
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(w, O, LSE, O_ref, LSE_ref, label=f"fp8 h_q={h_q} s_q={s_q}, 24 sequences")


MANY = [
    # name, batch, s_q, h_q, h_kv, lengths, causal, fmt, num_parts, pieces of the longest sequence (at least)
    ("many_rows5", 3, 1, 5, 1, [5000, 300, 2500], False, "bf16", 256, 65),
    ("many_hkv2", 2, 1, 32, 2, [4500, 900], False, "bf16", 200, 65),
    ("many_rows128_causal", 3, 2, 64, 1, [5000, 64, 2000], True, "bf16", 300, 65),
    ("many_fp8_rows16", 2, 1, 16, 1, [6000, 100], False, "fp8", 256, 65),
    ("many_fp8_rows128", 2, 1, 128, 1, [4100, 700], False, "fp8", 256, 65),
    # a partial 128-row tile (fp16 partials) whose last row pair holds one row
    ("many_rows75", 2, 1, 75, 1, [5000, 700], False, "bf16", 256, 65),
    ("many_fp8_rows75_causal", 2, 3, 25, 1, [4300, 900], True, "fp8", 256, 65),
    ("many_hkv2_rows128", 2, 1, 256, 2, [4500, 300], False, "bf16", 256, 65),
    ("many_fp8_hkv2_rows64", 2, 1, 128, 2, [4200, 500], False, "fp8", 256, 65),
]


def _pieces(w, num_parts):
    import paged_mla_decode_amd as mla
    _, splits = mla.mla_get_metadata_host(w.cache_seqlens, w.heads_per_kv, w.h_kv, kv_format=w.kv_format,
                                          num_parts=num_parts)
    return np.diff(splits.numpy())


@pytest.mark.parametrize("case", MANY, ids=[c[0] for c in MANY])
def test_sequences_of_many_pieces(case):
    """Sequences cut into more than 8 pieces (merged by the combine's helper workgroups), here
    more than 64 (two rounds of loads), with row counts that do not fill the helpers' row
    pairs, two KV heads, fp32 and fp16 partials."""
    name, B, S, H, Hk, L, causal, fmt, parts, least = case
    w = make_workload(name=name, batch=B, s_q=S, h_q=H, h_kv=Hk, seqlens=L, causal=causal, kv_format=fmt,
                      seed=80 + len(name), pool_pages=sum((x + 63) // 64 for x in L) + 5)
    n = _pieces(w, parts)
    print(f"[case] {name} num_parts={parts} pieces={n.tolist()}", flush=True)
    assert n.max() >= least
    O, LSE = run_gpu(w, num_parts=parts)
    O2, LSE2 = run_gpu(w, num_parts=parts)
    assert np.array_equal(O, O2) and np.array_equal(LSE, LSE2), "run-to-run results differ"
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(w, O, LSE, O_ref, LSE_ref, label=f"{name}/parts={parts}")


def test_more_than_256_sequences_of_many_pieces():
    """300 sequences of 9-11 pieces each: the combine's helpers list them in two chunks."""
    rng = np.random.default_rng(81)
    lens = [int(x) for x in rng.integers(560, 700, size=300)]
    w = make_workload(name="many_chunks", batch=300, s_q=1, h_q=16, seqlens=lens, seed=82)
    n = _pieces(w, 4000)
    print(f"[case] many_chunks: {int((n > 8).sum())} sequences of more than 8 pieces", flush=True)
    assert (n > 8).sum() > 256
    O, LSE = run_gpu(w, num_parts=4000)
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(w, O, LSE, O_ref, LSE_ref, label="300 sequences of 9-11 pieces")


@pytest.mark.parametrize("h_q", [16, 128])
def test_invalid_page_in_a_sequence_of_many_pieces(h_q):
    w = make_workload(name="badpage_many", batch=3, s_q=1, h_q=h_q, seqlens=[100, 3000, 50], seed=83)
    w_ok = make_workload(name="badpage_many", batch=3, s_q=1, h_q=h_q, seqlens=[100, 3000, 50], seed=83)
    assert _pieces(w, 256)[1] > 8
    w.block_table[1, 20] = 10_000
    O, LSE = run_gpu(w, num_parts=256)
    _compare_except(w_ok, O, LSE, [1], f"a bad page in a sequence of many pieces (h_q={h_q})")


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


@pytest.mark.parametrize("h_q", [16, 32, 64, 128])
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
@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_empty_and_fully_masked_rows(fmt, h_q):
    w = make_workload(name="empty", batch=4, s_q=2, h_q=h_q, seqlens=[0, 1, 2, 70], causal=True, seed=59,
                      max_blocks=3, kv_format=fmt)
    for parts in (0, 1, 9):
        O, LSE = run_gpu(w, num_parts=parts)
        O_ref, LSE_ref = oracle.mla_decode_workload(w)
        compare(w, O, LSE, O_ref, LSE_ref, label=f"empty rows parts={parts}")
        assert np.all(O[0] == 0) and np.all(np.isneginf(LSE[0]))
        assert np.all(O[1, 0] == 0) and np.all(np.isneginf(LSE[1, :, 0]))


@pytest.mark.parametrize("h_q", [16, 32, 64, 128])
@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_sequences_without_pages_between_pages(fmt, h_q):
    # ranges that start with, and step over, sequences of length 0: the page ring keeps the
    # next pages in flight across them while their (empty) outputs and merges are written
    w = make_workload(name="gaps", batch=8, s_q=1, h_q=h_q, seqlens=[0, 0, 65, 0, 1, 0, 130, 0], seed=63,
                      max_blocks=3, kv_format=fmt)
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    for parts in (0, 1, 2, 3):
        O, LSE = run_gpu(w, num_parts=parts)
        compare(w, O, LSE, O_ref, LSE_ref, label=f"gaps h_q={h_q} parts={parts}")


def _compare_except(w, O, LSE, nan_batches, label):
    """The sequences in nan_batches must be NaN everywhere; every other one matches the oracle."""
    nan_batches = sorted(set(nan_batches))
    for b in nan_batches:
        assert np.all(np.isnan(O[b])) and np.all(np.isnan(LSE[b])), f"{label}: sequence {b} must be NaN"
    ok = [b for b in range(w.batch) if b not in nan_batches]
    O_ref, LSE_ref = oracle.mla_decode_workload(w, batches=ok)
    if ok:
        compare(w, O[ok], LSE[ok], O_ref[ok], LSE_ref[ok], label=label)


@pytest.mark.parametrize("h_q", [16, 48, 128])
@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_invalid_block_table_entry_poisons_only_its_sequence(fmt, h_q):
    w = make_workload(name="badpage", batch=3, s_q=1, h_q=h_q, seqlens=[100, 200, 50], seed=60, kv_format=fmt)
    w_ok = make_workload(name="badpage", batch=3, s_q=1, h_q=h_q, seqlens=[100, 200, 50], seed=60, kv_format=fmt)
    w.block_table[1, 2] = 10_000
    O, LSE = run_gpu(w)
    _compare_except(w_ok, O, LSE, [1], f"sequences next to a bad page ({fmt}, h_q={h_q})")


@pytest.mark.parametrize("h_q", [16, 48, 128])
@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_length_beyond_the_block_table_poisons_only_its_sequence(fmt, h_q):
    # metadata built without the block-table check: the decode must not read past the row
    # (4 entries = 256 tokens) and must report the sequence as NaN
    w = make_workload(name="toolong", batch=3, s_q=1, h_q=h_q, seqlens=[100, 256, 50], seed=64, kv_format=fmt,
                      max_blocks=4)
    w_ok = make_workload(name="toolong", batch=3, s_q=1, h_q=h_q, seqlens=[100, 256, 50], seed=64, kv_format=fmt,
                         max_blocks=4)
    w.cache_seqlens[1] = 300
    O, LSE = run_gpu(w, meta_lengths=[100, 300, 50], num_parts=5)
    _compare_except(w_ok, O, LSE, [1], f"next to an over-long sequence ({fmt}, h_q={h_q})")


@pytest.mark.parametrize("h_q", [16, 48, 128])
@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_stale_metadata_is_detected(fmt, h_q):
    # metadata built for other page counts: every sequence is either NaN or correct for the
    # lengths the decode was given, and the sequence whose page count changed is NaN
    w = make_workload(name="stale", batch=4, s_q=1, h_q=h_q, seqlens=[100, 300, 50, 700], seed=65, kv_format=fmt,
                      max_blocks=12)
    for parts in (0, 3):
        O, LSE = run_gpu(w, meta_lengths=[100, 200, 50, 700], num_parts=parts)
        nan_b = [b for b in range(4) if np.all(np.isnan(O[b]))]
        print(f"[stale] {fmt} h_q={h_q} parts={parts}: NaN sequences {nan_b}", flush=True)
        assert 1 in nan_b
        _compare_except(w, O, LSE, nan_b, f"stale metadata ({fmt}, h_q={h_q}, parts={parts})")
    # lengths that change within the same page counts keep the metadata valid
    O, LSE = run_gpu(w, meta_lengths=[70, 257, 1, 641], num_parts=3)
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(w, O, LSE, O_ref, LSE_ref, label=f"same page counts ({fmt}, h_q={h_q})")


@pytest.mark.parametrize("h_q", [16, 128])
def test_sequence_without_pieces_is_nan(h_q):
    # num_splits that gives a sequence no piece: nothing is written for it by the split
    # kernel, and the combine reports NaN instead of leaving the outputs unwritten
    w = make_workload(name="nopiece", batch=3, s_q=1, h_q=h_q, seqlens=[100, 2000, 50], seed=66)

    def edit(splits):
        d = (splits[1:] - splits[:-1]).tolist()
        assert d[0] == 1 and d[2] == 1 and d[1] > 1, d
        splits[:] = torch.tensor([0, 1, 1, 2], dtype=torch.int32)

    O, LSE = run_gpu(w, num_parts=7, edit_splits=edit)
    _compare_except(w, O, LSE, [1], f"sequence without pieces (h_q={h_q})")


@pytest.mark.parametrize("h_q", [32, 128])
def test_noncontiguous_q_and_custom_scale(h_q):
    w = make_workload(name="strided", batch=2, s_q=2, h_q=h_q, seqlens=[333, 90], causal=True, seed=61,
                      softmax_scale=0.07)
    big = torch.zeros(2, 2, h_q + 8, 576, dtype=torch.bfloat16)
    big[:, :, 4:4 + h_q] = w.q
    w.q = big[:, :, 4:4 + h_q]                   # head stride 576, batch stride 2*(h_q+8)*576
    assert not w.q.is_contiguous()
    import paged_mla_decode_amd as mla
    meta, splits = mla.mla_get_metadata(w.cache_seqlens, w.heads_per_kv, 1, max_blocks_per_seq=w.block_table.shape[1],
                                        device=torch.device(DEV))
    o, lse = mla.mla_decode_kvcache(big.to(DEV)[:, :, 4:4 + h_q], w.kvcache.to(DEV), w.block_table.to(DEV),
                                    w.cache_seqlens.to(DEV), 512, meta, splits, causal=True, softmax_scale=0.07)
    torch.cuda.synchronize()
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    compare(w, o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), O_ref, LSE_ref,
            label="strided q, scale 0.07")
