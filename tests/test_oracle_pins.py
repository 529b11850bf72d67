"""Pins for the CPU oracle: each check ties it to something other than itself.

* brute force (pure Python, tests/bruteforce.py) on tiny cases that cross
  page boundaries, both causal flags, h_kv in {1, 2}, s_q in {1, 2}, BF16 and FP8;
* torch's scaled_dot_product_attention in float64 with an explicit
  bottom-right mask, and scipy's logsumexp;
* closed forms (one key, zero query, identical keys, a hand-worked example);
* invariants (page permutation, head permutation, causal rows, split merge);
* the e4m3fn decoder against torch.float8_e4m3fn for all 256 codes.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from bruteforce import brute_force_decode, bf16_bits_to_float, e4m3fn_code_to_float
from workloads import make_workload, named_workload, permute_pages, poison_unused, quantize_fp8_records

TINY_CASES = [
    # (batch, s_q, h_q, h_kv, lengths, causal, fmt, seed)
    (2, 1, 4, 1, [1, 130], False, "bf16", 11),
    (2, 2, 4, 2, [65, 128], True, "bf16", 12),
    (1, 2, 2, 1, [130], False, "bf16", 13),
    (2, 2, 2, 1, [2, 64], True, "fp8", 14),
    (1, 1, 3, 1, [129], False, "fp8", 15),
]


def _brute(w):
    a = w.as_numpy()
    return brute_force_decode(a["q_bits"].tolist(), a["kvcache"].tolist(), w.kv_format,
                              a["block_table"].tolist(), a["cache_seqlens"].tolist(),
                              dv=w.dv, causal=w.causal, scale=w.softmax_scale)


@pytest.mark.parametrize("case", TINY_CASES, ids=lambda c: f"B{c[0]}S{c[1]}H{c[2]}Hk{c[3]}L{c[4]}{'c' if c[5] else ''}{c[6]}")
def test_oracle_matches_bruteforce(case):
    B, S, H, Hk, L, causal, fmt, seed = case
    w = make_workload(name="tiny", batch=B, s_q=S, h_q=H, h_kv=Hk, seqlens=L, causal=causal,
                      kv_format=fmt, seed=seed, pool_pages=sum((x + 63) // 64 for x in L) + 3)
    O, LSE = oracle.mla_decode_workload(w)
    Ob, LSEb = _brute(w)
    assert np.max(np.abs(O - np.asarray(Ob))) <= 1e-12
    assert np.max(np.abs(LSE - np.asarray(LSEb))) <= 1e-12


def _sdpa_reference(w, batches):
    """torch SDPA in float64 with an explicit bottom-right boolean mask."""
    a = w.as_numpy()
    out = {}
    G = w.h_q // w.h_kv
    for b in batches:
        L = int(a["cache_seqlens"][b])
        # contiguous K via a per-token index walk written with torch ops
        t = torch.arange(L)
        pages = torch.from_numpy(a["block_table"][b].astype(np.int64))[t // 64]
        if w.kv_format == "bf16":
            K = w.kvcache[pages, t % 64].to(torch.float64)                      # [L, Hk, 576]
        else:
            raw = w.kvcache[pages, t % 64]                                         # [L, Hk, 656]
            lat = raw[..., :512].contiguous().view(torch.float8_e4m3fn).to(torch.float64)
            sc = raw[..., 512:528].contiguous().view(torch.float32).to(torch.float64)
            rope = raw[..., 528:].contiguous().view(torch.bfloat16).to(torch.float64)
            lat = (lat.view(L, w.h_kv, 4, 128) * sc.view(L, w.h_kv, 4, 1)).view(L, w.h_kv, 512)
            K = torch.cat([lat, rope], dim=-1)
        q = w.q[b].to(torch.float64)                                               # [S, H, 576]
        for kvh in range(w.h_kv):
            Kh = K[:, kvh, :]
            Vh = Kh[:, :w.dv].contiguous()
            Q = q[:, kvh * G:(kvh + 1) * G, :].reshape(w.s_q * G, 576)
            rows_s = torch.arange(w.s_q).repeat_interleave(G)
            last = (L - w.s_q + rows_s) if w.causal else torch.full_like(rows_s, L - 1)
            mask = torch.arange(L)[None, :] <= last[:, None]
            o = torch.nn.functional.scaled_dot_product_attention(
                Q[None, None], Kh[None, None], Vh[None, None], attn_mask=mask[None, None],
                scale=w.softmax_scale)[0, 0]
            from scipy.special import logsumexp
            z = (w.softmax_scale * (Q @ Kh.T)).numpy()
            z = np.where(mask.numpy(), z, -np.inf)
            lse = logsumexp(z, axis=1)
            out[(b, kvh)] = (o.numpy().reshape(w.s_q, G, w.dv), lse.reshape(w.s_q, G))
    return out


@pytest.mark.parametrize("which", ["tiny", "mtp_small", "fp8_small"])
def test_oracle_matches_sdpa(which):
    if which == "tiny":
        w = named_workload("tiny")
    elif which == "mtp_small":
        # the speculative-decode shape (s_q=2, h_q=128, causal, L ~ 4096 +- 25%) at batch 2
        rng = np.random.Generator(np.random.PCG64(3))
        w = make_workload(name="mtp_small", batch=2, s_q=2, h_q=128, seqlens=rng.integers(3072, 5121, 2).tolist(),
                          causal=True, seed=3)
    else:
        w = make_workload(name="fp8_small", batch=2, s_q=1, h_q=128, seqlens=[700, 8192 // 4], kv_format="fp8", seed=5)
    O, LSE = oracle.mla_decode_workload(w)
    ref = _sdpa_reference(w, range(w.batch))
    G = w.h_q // w.h_kv
    for (b, kvh), (o, lse) in ref.items():
        assert np.max(np.abs(O[b, :, kvh * G:(kvh + 1) * G, :] - o)) <= 1e-10
        assert np.max(np.abs(LSE[b, kvh * G:(kvh + 1) * G, :].T - lse)) <= 1e-10


def test_single_key_gives_that_value_row():
    w = make_workload(name="L1", batch=3, s_q=1, h_q=8, seqlens=[1, 1, 1], seed=21, pool_pages=7)
    O, LSE = oracle.mla_decode_workload(w)
    a = w.as_numpy()
    for b in range(3):
        k = oracle.bf16_bits_to_f64(a["kvcache"][a["block_table"][b, 0], 0, 0])
        for h in range(8):
            qv = oracle.bf16_bits_to_f64(a["q_bits"][b, 0, h])
            assert np.array_equal(O[b, 0, h], k[:512])
            z = math.fsum((qv * k).tolist()) * w.softmax_scale
            assert abs(LSE[b, h, 0] - z) <= 1e-12


def test_zero_query_averages_allowed_values():
    w = make_workload(name="q0", batch=2, s_q=2, h_q=4, seqlens=[70, 3], causal=True, seed=22)
    w.q.zero_()
    O, LSE = oracle.mla_decode_workload(w)
    a = w.as_numpy()
    for b, L in enumerate([70, 3]):
        rows = np.stack([oracle.bf16_bits_to_f64(a["kvcache"][a["block_table"][b, t // 64], t % 64, 0])
                         for t in range(L)])
        for s in range(2):
            n = L - 2 + s + 1
            assert np.max(np.abs(O[b, s, :, :] - rows[:n, :512].mean(axis=0))) <= 1e-12
            assert np.max(np.abs(LSE[b, :, s] - math.log(n))) <= 1e-12


def test_identical_keys():
    w = make_workload(name="same", batch=1, s_q=1, h_q=4, seqlens=[150], seed=23)
    w.kvcache[:] = w.kvcache[int(w.block_table[0, 0]), 0]
    O, LSE = oracle.mla_decode_workload(w)
    a = w.as_numpy()
    k = oracle.bf16_bits_to_f64(a["kvcache"][0, 0, 0])
    for h in range(4):
        qv = oracle.bf16_bits_to_f64(a["q_bits"][0, 0, h])
        z = w.softmax_scale * math.fsum((qv * k).tolist())
        assert np.max(np.abs(O[0, 0, h] - k[:512])) <= 1e-12
        assert abs(LSE[0, h, 0] - (z + math.log(150))) <= 1e-12


def test_hand_worked_example():
    """tests/golden/hand_example.txt: two keys, logits 0 and ln 3, so weights 1/4 and 3/4."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "hand_example.txt")
    vals = {}
    for line in open(path, encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split("=", 1)
            vals[k.strip()] = float(v)
    # q = e_0 (first dim 1), key 0 = 0 vector, key 1 has first dim c so that scale*c = ln 3.
    # Build it in bf16-exact values: choose scale = ln(3) / 2 and c = 2 (both exact in fp64/bf16).
    scale = vals["scale"]
    q = torch.zeros(1, 1, 1, 576, dtype=torch.bfloat16)
    q[0, 0, 0, 0] = 1.0
    kv = torch.zeros(1, 64, 1, 576, dtype=torch.bfloat16)
    kv[0, 1, 0, 0] = vals["key1_dim0"]
    kv[0, 0, 0, 1] = vals["value0_dim1"]          # key 0 dim 1 does not touch the logit (q dim 1 = 0)
    kv[0, 1, 0, 1] = vals["value1_dim1"]
    bt = np.zeros((1, 1), dtype=np.int32)
    O, LSE = oracle.mla_decode(q.view(torch.int16).numpy().view(np.uint16), kv.view(torch.int16).numpy().view(np.uint16),
                               "bf16", bt, np.array([2]), softmax_scale=scale)
    assert abs(O[0, 0, 0, 1] - vals["expected_o_dim1"]) <= 1e-14
    assert abs(O[0, 0, 0, 0] - vals["expected_o_dim0"]) <= 1e-14
    assert abs(LSE[0, 0, 0] - vals["expected_lse"]) <= 1e-14


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_page_permutation_invariance(fmt):
    w = make_workload(name="perm", batch=3, s_q=2, h_q=8, seqlens=[300, 64, 1], causal=True, kv_format=fmt,
                      seed=24, pool_pages=12)
    O1, L1 = oracle.mla_decode_workload(w)
    O2, L2 = oracle.mla_decode_workload(permute_pages(w, 99))
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_poisoned_unused_bytes_do_not_leak():
    w = make_workload(name="poison", batch=2, s_q=2, h_q=4, seqlens=[100, 37], causal=True, seed=25, max_blocks=4)
    O1, L1 = oracle.mla_decode_workload(w)
    O2, L2 = oracle.mla_decode_workload(poison_unused(w))
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_head_permutation_within_group():
    w = make_workload(name="heads", batch=1, s_q=1, h_q=8, h_kv=2, seqlens=[90], seed=26)
    O1, L1 = oracle.mla_decode_workload(w)
    perm = torch.tensor([2, 0, 3, 1, 5, 7, 4, 6])       # stays inside each group of 4
    w.q = w.q[:, :, perm].contiguous()
    O2, L2 = oracle.mla_decode_workload(w)
    assert np.array_equal(O2, O1[:, :, perm.numpy()])
    assert np.array_equal(L2, L1[:, perm.numpy()])


def test_causal_rows_equal_shorter_noncausal():
    L = 200
    w = make_workload(name="causal", batch=1, s_q=2, h_q=4, seqlens=[L], causal=True, seed=27)
    Oc, Lc = oracle.mla_decode_workload(w)
    a = w.as_numpy()
    for s in range(2):
        O, LSE = oracle.mla_decode(a["q_bits"][:, s:s + 1], a["kvcache"], "bf16", a["block_table"],
                                   np.array([L - 1 + s]), causal=False, softmax_scale=w.softmax_scale)
        assert np.array_equal(O[0, 0], Oc[0, s]) and np.array_equal(LSE[0, :, 0], Lc[0, :, s])
    # with s_q = 1, causal is a no-op
    w1 = make_workload(name="causal1", batch=2, s_q=1, h_q=4, seqlens=[77, 5], causal=True, seed=28)
    O1, L1 = oracle.mla_decode_workload(w1)
    w1.causal = False
    O2, L2 = oracle.mla_decode_workload(w1)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


@pytest.mark.parametrize("cut", [1, 64, 100, 199])
def test_split_merge_equals_whole(cut):
    w = make_workload(name="split", batch=1, s_q=1, h_q=16, seqlens=[200], seed=29)
    a = w.as_numpy()
    K = oracle.gather_sequence(a["kvcache"], "bf16", a["block_table"][0], 200)[:, 0]
    Q = oracle.bf16_bits_to_f64(a["q_bits"][0, 0])
    O, lse = oracle.attend(Q, K, K[:, :512], w.softmax_scale)
    O1, l1 = oracle.attend(Q, K[:cut], K[:cut, :512], w.softmax_scale)
    O2, l2 = oracle.attend(Q, K[cut:], K[cut:, :512], w.softmax_scale)
    Oc, lc = oracle.combine_partials([O1, O2], [l1, l2])
    assert np.max(np.abs(Oc - O)) <= 1e-12 and np.max(np.abs(lc - lse)) <= 1e-12
    # a part over an empty key set carries no weight; all-empty gives O = 0, LSE = -inf
    Oe, le = oracle.attend(Q, K[:0], K[:0, :512], w.softmax_scale)
    Oc2, lc2 = oracle.combine_partials([O1, Oe, O2], [l1, le, l2])
    assert np.max(np.abs(Oc2 - O)) <= 1e-12
    Oc3, lc3 = oracle.combine_partials([Oe, Oe], [le, le])
    assert np.all(Oc3 == 0) and np.all(np.isneginf(lc3))


def test_empty_and_fully_masked_rows():
    w = make_workload(name="empty", batch=3, s_q=2, h_q=2, seqlens=[0, 1, 2], causal=True, seed=30, max_blocks=2)
    O, LSE = oracle.mla_decode_workload(w)
    assert np.all(O[0] == 0) and np.all(np.isneginf(LSE[0]))          # L = 0
    assert np.all(O[1, 0] == 0) and np.all(np.isneginf(LSE[1, :, 0]))  # L = 1, row s = 0 sees nothing
    assert np.all(np.isfinite(LSE[1, :, 1])) and np.all(np.isfinite(LSE[2]))


def test_invalid_inputs_raise():
    w = make_workload(name="bad", batch=1, s_q=1, h_q=2, seqlens=[10], seed=31)
    a = w.as_numpy()
    with pytest.raises(ValueError):
        oracle.mla_decode(a["q_bits"], a["kvcache"], "bf16", a["block_table"], np.array([65]))
    with pytest.raises(ValueError):
        oracle.mla_decode(a["q_bits"], a["kvcache"], "bf16", a["block_table"], np.array([-1]))
    bt = a["block_table"].copy()
    bt[0, 0] = 5
    with pytest.raises(ValueError):
        oracle.mla_decode(a["q_bits"], a["kvcache"], "bf16", bt, np.array([10]))


def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(codes[nan].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    brute = np.array([e4m3fn_code_to_float(c) for c in range(256)])
    assert np.array_equal(ours[~nan], brute[~nan])
    # closed-form points of the OCP E4M3FN format
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9 and ours[0x38] == 1.0
    assert ours[0x00] == 0.0 and ours[0x80] == 0.0 and math.copysign(1, ours[0x80]) == -1


def test_fp8_record_roundtrip_and_layout():
    g = torch.Generator().manual_seed(7)
    x = torch.randn(5, 512, generator=g)
    rope = torch.randn(5, 64, generator=g).to(torch.bfloat16)
    rec = quantize_fp8_records(x, rope).numpy()
    assert rec.shape == (5, 656)
    dec = oracle.decode_fp8_records(rec)
    # RoPE dims are carried exactly
    assert np.array_equal(dec[:, 512:], rope.to(torch.float64).numpy())
    # latent: e4m3 keeps 3 mantissa bits, so relative error <= 2^-4 within each chunk's range
    xs = x.double().numpy().reshape(5, 4, 128)
    amax = np.abs(xs).max(axis=-1, keepdims=True)
    err = np.abs(dec[:, :512].reshape(5, 4, 128) - xs)
    assert np.all(err <= np.maximum(np.abs(xs) * 2.0 ** -4, amax / 448 * 2.0 ** -9) + 1e-12)
    # scale bytes sit at [512, 528) and multiply 128-dim chunks in order
    sc = rec[:, 512:528].copy().view("<f4")
    assert np.allclose(sc, amax[..., 0] / 448.0, rtol=1e-6)
    brute = np.array([__import__("bruteforce").fp8_record_to_floats(bytes(r.tolist())) for r in rec])
    assert np.array_equal(brute, dec)


def test_named_workloads_shapes():
    w = named_workload("tiny")
    assert w.q.shape == (2, 1, 16, 576) and w.kvcache.shape == (16, 64, 1, 576)
    assert w.cache_seqlens.tolist() == [100, 257] and w.block_table.shape == (2, 5)
    ids = w.block_table[0, :2].tolist() + w.block_table[1, :5].tolist()
    assert len(set(ids)) == 7 and all(0 <= i < 16 for i in ids)
    assert w.block_table[0, 2:].tolist() == [0, 0, 0]
    assert abs(w.softmax_scale - 1 / 24) < 1e-15
