"""Host tile scheduler (mla_get_metadata) invariants, on the CPU.

The layout of the metadata is this library's own (the pages give only its
shape), so the tests check what must hold for any correct schedule: every
(sequence, page) in exactly one range, in order; every sequence in at least
one range; piece indices 0..k-1 in order; num_splits prefix sums; balance.
"""
import ctypes

import numpy as np
import pytest

from paged_mla_decode_amd import _lib


def schedule(L, M=16, hkv=1, fmt=0, cus=256, parts=0):
    lib = _lib.load()
    B = len(L)
    Ls = (ctypes.c_int32 * B)(*[int(x) for x in L])
    if parts == 0:
        parts = lib.mla_num_parts(B, M, hkv, fmt, cus)
    meta = (ctypes.c_int32 * (parts * 8))()
    splits = (ctypes.c_int32 * (B + 1))()
    got = ctypes.c_int(0)
    st = lib.mla_get_metadata(Ls, B, M, hkv, fmt, cus, parts, meta, splits, ctypes.byref(got))
    assert st == _lib.MLA_OK, lib.mla_last_error()
    assert got.value == parts
    return np.array(meta, dtype=np.int64).reshape(parts, 8), np.array(splits, dtype=np.int64)


def check_schedule(L, meta, splits):
    L = np.asarray(L, dtype=np.int64)
    B = len(L)
    npg = (L + 63) // 64
    seen = [[] for _ in range(B)]          # (part, page) in visit order
    pieces = [[] for _ in range(B)]        # split index per covering part
    last = (-1, -1)
    for p, m in enumerate(meta):
        bb, bp, eb, ep, s0 = (int(x) for x in m[:5])
        assert all(int(x) == 0 for x in m[5:])
        if bb < 0:
            continue
        assert 0 <= bb <= eb < B
        for b in range(bb, eb + 1):
            p0 = bp if b == bb else 0
            p1 = ep if b == eb else int(npg[b])
            assert 0 <= p0 <= p1 <= npg[b]
            if npg[b] > 0:
                assert p0 < p1, "a covered sequence with pages must get at least one page"
            pieces[b].append(s0 if b == bb else 0)
            for i in range(p0, p1):
                assert (b, i) > last, "ranges must run in (sequence, page) order"
                last = (b, i)
                seen[b].append(i)
    for b in range(B):
        assert seen[b] == list(range(int(npg[b]))), f"sequence {b}: pages {seen[b]} != 0..{npg[b]-1}"
        assert len(pieces[b]) >= 1, f"sequence {b} is in no range"
        assert pieces[b] == list(range(len(pieces[b]))), f"sequence {b}: piece indices {pieces[b]}"
    assert splits[0] == 0
    assert list(np.diff(splits)) == [len(pc) for pc in pieces]
    return pieces


@pytest.mark.parametrize("L", [
    [100, 257],
    [0],
    [0, 0, 0],
    [1],
    [64, 65, 63, 0, 128, 1],
    [32768],
    [8192] * 128,
])
@pytest.mark.parametrize("parts", [0, 1, 3, 64, 256, 1024])
def test_schedule_covers_everything_once(L, parts):
    meta, splits = schedule(L, parts=parts)
    check_schedule(L, meta, splits)


@pytest.mark.parametrize("M,hkv,fmt", [(16, 1, 0), (32, 1, 0), (128, 1, 0), (256, 1, 0), (128, 1, 1), (64, 2, 0)])
def test_schedule_random_lengths(M, hkv, fmt):
    rng = np.random.default_rng(M + hkv + fmt)
    for trial in range(20):
        B = int(rng.integers(1, 200))
        L = rng.integers(0, 5000, size=B)
        if trial % 3 == 0:
            L[rng.integers(0, B)] = 32768
        meta, splits = schedule(L, M=M, hkv=hkv, fmt=fmt)
        check_schedule(L, meta, splits)


def test_balance_on_ragged_lengths():
    rng = np.random.default_rng(4)
    L = rng.integers(256, 1025, size=128)
    L[17] = 32768
    meta, splits = schedule(L, M=16)
    pieces = check_schedule(L, meta, splits)
    npg = (L + 63) // 64
    # cost of each range = its pages + a fixed cost per piece (the scheduler's
    # split cost: 3 pages for tiles of up to 64 rows)
    split_cost = 3
    costs = []
    for m in meta:
        bb, bp, eb, ep = (int(x) for x in m[:4])
        if bb < 0:
            costs.append(0)
            continue
        c = 0
        for b in range(bb, eb + 1):
            p0 = bp if b == bb else 0
            p1 = ep if b == eb else int(npg[b])
            c += (p1 - p0) + split_cost
        costs.append(c)
    total = int(npg.sum()) + split_cost * len(L)
    target = total / len(meta)
    assert max(costs) <= target + 2 * split_cost + 1
    # the long sequence is spread over many ranges
    assert len(pieces[17]) >= 32


def test_metadata_independent_of_nothing_but_inputs():
    L = [300, 5, 0, 9000]
    a = schedule(L, parts=37)
    b = schedule(L, parts=37)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_default_parts_fill_the_chip():
    lib = _lib.load()
    # one workgroup per CU: up to 64 rows one tile, more than 64 rows 128-row
    # tiles (256 rows: two per range), for bf16 and FP8 pages alike.
    assert lib.mla_num_parts(64, 16, 1, 0, 256) == 256
    assert lib.mla_num_parts(64, 64, 1, 0, 256) == 256
    assert lib.mla_num_parts(64, 128, 1, 0, 256) == 256
    assert lib.mla_num_parts(64, 256, 1, 0, 256) == 128
    assert lib.mla_num_parts(64, 128, 1, 1, 256) == 256
    assert lib.mla_num_parts(64, 256, 1, 1, 256) == 128
    assert lib.mla_num_parts(64, 16, 1, 0, 0) in (-1, 256, lib.mla_device_cu_count(0))
