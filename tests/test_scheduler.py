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


def schedule(L, M=16, hkv=1, fmt=0, cus=256, parts=0, maxb=0):
    lib = _lib.load()
    B = len(L)
    Ls = (ctypes.c_int32 * B)(*[int(x) for x in L])
    if parts == 0:
        parts = lib.mla_num_parts(B, M, hkv, fmt, cus)
    meta = (ctypes.c_int32 * (parts * 8))()
    splits = (ctypes.c_int32 * (B + 1))()
    got = ctypes.c_int(0)
    st = lib.mla_get_metadata(Ls, B, M, hkv, fmt, maxb, cus, parts, meta, splits, ctypes.byref(got))
    assert st == _lib.MLA_OK, lib.mla_last_error()
    assert got.value == parts
    return np.array(meta, dtype=np.int64).reshape(parts, 8), np.array(splits, dtype=np.int64)


def range_checksum(npages):
    """Field 5 of a non-empty range: the page counts of its sequences folded in
    order with h = (h ^ n) * 0x9E3779B1 + 0x7F4A7C15 (mod 2^32) from 0x6D6C6131,
    as a signed int32."""
    h = 0x6D6C6131
    for n in npages:
        h = (((h ^ (int(n) & 0xFFFFFFFF)) * 0x9E3779B1) + 0x7F4A7C15) & 0xFFFFFFFF
    return h - (1 << 32) if h >= (1 << 31) else h


def check_schedule(L, meta, splits):
    L = np.asarray(L, dtype=np.int64)
    B = len(L)
    npg = (L + 63) // 64
    seen = [[] for _ in range(B)]          # (part, page) in visit order
    pieces = [[] for _ in range(B)]        # split index per covering part
    last = (-1, -1)
    for p, m in enumerate(meta):
        bb, bp, eb, ep, s0 = (int(x) for x in m[:5])
        assert int(m[6]) == B and int(m[7]) == 0
        if bb < 0:
            assert int(m[5]) == 0
            continue
        assert 0 <= bb <= eb < B
        assert int(m[5]) == range_checksum(npg[bb:eb + 1]), f"range {p}: checksum"

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


def test_checksum_detects_any_single_page_count_change():
    rng = np.random.default_rng(9)
    for _ in range(200):
        n = rng.integers(0, 300, size=int(rng.integers(1, 8)))
        k = int(rng.integers(0, len(n)))
        m = n.copy()
        m[k] += int(rng.integers(1, 50)) * (1 if rng.random() < 0.5 or m[k] == 0 else -1)
        m[k] = max(m[k], 0)
        if m[k] == n[k]:
            continue
        assert range_checksum(n) != range_checksum(m)


def test_lengths_beyond_the_block_table_are_rejected():
    lib = _lib.load()
    B = 3
    for L, ok in (([64, 128, 0], True), ([64, 129, 0], False), ([0, 0, 128], True)):
        Ls = (ctypes.c_int32 * B)(*L)
        meta = (ctypes.c_int32 * (4 * 8))()
        splits = (ctypes.c_int32 * (B + 1))()
        st = lib.mla_get_metadata(Ls, B, 16, 1, 0, 2, 256, 4, meta, splits, None)
        assert (st == _lib.MLA_OK) == ok, (L, lib.mla_last_error())
        if not ok:
            assert st == _lib.MLA_ERR_INVALID_ARGUMENT and b"exceeds the block table" in lib.mla_last_error()
        # unchecked (0): accepted; the decode reports such a sequence as NaN
        assert lib.mla_get_metadata(Ls, B, 16, 1, 0, 0, 256, 4, meta, splits, None) == _lib.MLA_OK
    Ls = (ctypes.c_int32 * B)(1, 2, 3)
    assert lib.mla_get_metadata(Ls, B, 16, 1, 0, -1, 256, 4, meta, splits, None) == _lib.MLA_ERR_INVALID_ARGUMENT


def cost_line_schedule(L, split_cost, parts):
    """The cost-line form of the greedy fill that the device scheduler (scheduler_device.hip)
    builds on, in plain Python: on the cost line where sequence b spans [S_b, S_b+1) with
    S_b+1 - S_b = split_cost + pages_b, a range starting at V ends at E = V + budget and the next
    one starts at S_e if E - S_e <= split_cost (e: the sequence holding E), else at
    E - split_cost; the budget is the smallest in [ceil(W / P), ceil(W / P) + split_cost] that
    places all the work. The device computes the same range starts in parallel
    (parallel_range_starts below); the rows, piece indices and counts follow as here."""
    import bisect
    B = len(L)
    npg = [(int(x) + 63) // 64 for x in L]
    S = [0]
    for n in npg:
        S.append(S[-1] + split_cost + n)
    W = S[-1]
    lo = max(1, -(-W // parts))
    for c in range(split_cost + 1):
        bd, v, V, ok = lo + c, 0, [], True
        while v < W:
            if len(V) == parts or bd <= split_cost:
                ok = False
                break
            V.append(v)
            E = v + bd
            if E >= W:
                nv = W
            else:
                e = bisect.bisect_right(S, E) - 1
                nv = S[e] if E - S[e] <= split_cost else E - split_cost
            v = nv
        if ok:
            break
    assert ok, "the window always holds a feasible budget"
    n = len(V)
    V = V + [W]
    meta = np.zeros((parts, 8), dtype=np.int64)
    meta[:, 6] = B
    seq_at = lambda x: bisect.bisect_right(S[:B], x) - 1
    count_le = lambda x: bisect.bisect_right(V[:n], x)
    count_lt = lambda x: bisect.bisect_left(V[:n], x)
    for p in range(parts):
        if p >= n:
            meta[p, :5] = [-1, 0, -2, 0, 0]
            continue
        v0, v1 = V[p], V[p + 1]
        bb = seq_at(v0)
        if v1 >= W:
            eb, ep = B - 1, npg[B - 1]
        else:
            a = seq_at(v1)
            eb, ep = (a - 1, npg[a - 1]) if v1 == S[a] else (a, v1 - S[a])
        meta[p, :6] = [bb, v0 - S[bb], eb, ep, p - (count_le(S[bb]) - 1), range_checksum(npg[bb:eb + 1])]
    pieces = [count_lt(S[b + 1]) - (count_le(S[b]) - 1) for b in range(B)]
    return meta, np.concatenate([[0], np.cumsum(pieces)]).astype(np.int64)


def test_cost_line_algorithm_matches_the_greedy_scheduler():
    # the device scheduler's formulation must give the host scheduler's metadata bit for bit
    rng = np.random.default_rng(21)
    for trial in range(400):
        B = int(rng.integers(1, 300))
        kind = trial % 4
        if kind == 0:
            L = rng.integers(0, 5000, size=B)
        elif kind == 1:
            L = rng.integers(0, 200, size=B)
        elif kind == 2:
            L = np.full(B, int(rng.integers(0, 9000)))
        else:
            L = rng.integers(256, 1025, size=B)
            L[rng.integers(0, B)] = 32768
        if rng.random() < 0.2:
            L[rng.random(B) < 0.3] = 0
        M = int(rng.choice([16, 32, 64, 128, 256]))
        P = int(rng.choice([1, 2, 3, 7, 64, 128, 256, 1024]))
        meta, splits = schedule(L, M=M, parts=P)
        m2, s2 = cost_line_schedule(L, 8 if M > 64 else 3, P)
        assert np.array_equal(meta, m2) and np.array_equal(splits, s2), (B, M, P)


def run_table(S, W, bd, split_cost):
    """Runs of the cost-line walk with budget bd (the device scheduler's first step): from the
    start S_e of sequence e the range starts are S_e + k (bd - split_cost) until the end E of a
    range falls within split_cost of a later sequence start S_a (the walk snaps to S_a: the next
    run starts there) or reaches W. Returns, per sequence e, the number of range starts of the run
    and the sequence it snaps to (len(S) - 1 = the end)."""
    B = len(S) - 1
    step = bd - split_cost
    K, nx = [0] * (B + 1), [B] * (B + 1)
    for e in range(B):
        E0 = S[e] + bd
        if E0 >= W:
            K[e], nx[e] = 1, B
            continue
        a = e
        while a + 1 < B and S[a + 1] <= E0:
            a += 1
        k, E = 0, E0
        while True:
            if E - S[a] <= split_cost:                   # snap to the start of sequence a
                K[e], nx[e] = k + 1, a
                break
            target = S[a + 1] if a + 1 < B else W        # the next start (or the end)
            k = k + 1 + (target - E - 1) // step         # first k with E0 + k step >= target
            E = E0 + k * step
            if E >= W:
                K[e], nx[e] = k + 1, B
                break
            a += 1
            while a + 1 < B and S[a + 1] <= E:
                a += 1
    return K, nx


def parallel_range_starts(L, split_cost, parts):
    """The device scheduler's formulation: per candidate budget, the runs, then the number of
    ranges as the sum of the run lengths along the chain of snaps from sequence 0 (pointer
    jumping); the smallest feasible budget; then every range start at once by binary lifting
    over the chain (range p lies in the run of the last chain node whose first range <= p)."""
    B = len(L)
    npg = [(int(x) + 63) // 64 for x in L]
    S = [0]
    for n in npg:
        S.append(S[-1] + split_cost + n)
    W = S[-1]
    lo = max(1, -(-W // parts))
    for c in range(split_cost + 1):
        bd = lo + c
        if bd <= split_cost:
            continue
        K, nx = run_table(S, W, bd, split_cost)
        nxt, tot = list(nx), list(K)
        for _ in range(max(1, B.bit_length()) + 1):      # pointer jumping: tot[e] = ranges from e to the end
            nxt, tot = [nxt[nxt[e]] for e in range(B + 1)], [tot[e] + tot[nxt[e]] for e in range(B + 1)]
        if tot[0] <= parts:
            break
    n = tot[0]
    up, cnt = [list(nx)], [list(K)]                      # lifting tables: 2^k snaps ahead, ranges covered
    for _ in range(max(1, B.bit_length())):
        u, t = up[-1], cnt[-1]
        up.append([u[u[e]] for e in range(B + 1)])
        cnt.append([t[e] + t[u[e]] for e in range(B + 1)])
    V = []
    for p in range(n):
        cur, acc = 0, 0
        for k in reversed(range(len(up))):
            if up[k][cur] != B and acc + cnt[k][cur] <= p:
                acc += cnt[k][cur]
                cur = up[k][cur]
        V.append(S[cur] + (p - acc) * (bd - split_cost))
    return bd, V + [W]


def test_parallel_formulation_matches_the_walk():
    # the device scheduler's parallel form (runs, pointer jumping, lifting) gives the walk's ranges
    import bisect
    rng = np.random.default_rng(33)
    for trial in range(400):
        B = int(rng.integers(1, 300))
        kind = trial % 4
        if kind == 0:
            L = rng.integers(0, 5000, size=B)
        elif kind == 1:
            L = rng.integers(0, 200, size=B)
        elif kind == 2:
            L = np.full(B, int(rng.integers(0, 9000)))
        else:
            L = rng.integers(256, 1025, size=B)
            L[rng.integers(0, B)] = 32768
        if rng.random() < 0.2:
            L[rng.random(B) < 0.3] = 0
        sc = int(rng.choice([1, 3, 8, 15]))
        P = int(rng.choice([1, 2, 3, 7, 64, 128, 256, 1024]))
        npg = [(int(x) + 63) // 64 for x in L]
        S = [0]
        for n in npg:
            S.append(S[-1] + sc + n)
        W = S[-1]
        lo = max(1, -(-W // P))
        for c in range(sc + 1):                          # the walk, as in cost_line_schedule
            bd, v, V, ok = lo + c, 0, [], True
            while v < W:
                if len(V) == P or bd <= sc:
                    ok = False
                    break
                V.append(v)
                E = v + bd
                if E >= W:
                    v = W
                else:
                    e = bisect.bisect_right(S, E) - 1
                    v = S[e] if E - S[e] <= sc else E - sc
            if ok:
                break
        bd2, V2 = parallel_range_starts(L, sc, P)
        assert (bd2, V2) == (bd, V + [W]), (trial, B, sc, P)
