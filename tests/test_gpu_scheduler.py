"""The tile scheduler on the device (mla_get_metadata_device) against the host one: integer
work, so the metadata must be identical bit for bit, and a decode with either gives
bitwise-identical outputs."""
import numpy as np
import pytest
import torch

from workloads import WORKLOAD_SPECS, make_workload, named_workload

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")


def _both(L, M, h_kv=1, fmt="bf16", parts=0):
    import paged_mla_decode_amd as mla
    Lt = torch.tensor(np.asarray(L, dtype=np.int32))
    mh, sh = mla.mla_get_metadata_host(Lt, M, h_kv, kv_format=fmt, num_parts=parts)
    md, sd = mla.mla_get_metadata_device(Lt.to(DEV), M, h_kv, kv_format=fmt, num_parts=parts)
    torch.cuda.synchronize()
    return mh, sh, md.cpu(), sd.cpu()


def _same(L, M, h_kv=1, fmt="bf16", parts=0, label=""):
    mh, sh, md, sd = _both(L, M, h_kv, fmt, parts)
    assert torch.equal(mh, md), f"{label}: tile_metadata differs"
    assert torch.equal(sh, sd), f"{label}: num_splits differs"


@pytest.mark.parametrize("name", list(WORKLOAD_SPECS))
def test_device_metadata_equals_host_on_the_workloads(name):
    spec = WORKLOAD_SPECS[name]
    w = named_workload(name)
    print(f"[sched] {name}", flush=True)
    _same(w.cache_seqlens.numpy(), w.heads_per_kv, 1, w.kv_format, 0, name)


def test_device_metadata_equals_host_on_random_lengths():
    rng = np.random.default_rng(2024)
    for trial in range(300):
        B = int(rng.integers(1, 1024))
        kind = trial % 5
        if kind == 0:
            L = rng.integers(0, 5000, size=B)
        elif kind == 1:
            L = rng.integers(0, 300, size=B)
        elif kind == 2:
            L = np.full(B, int(rng.integers(0, 20000)))
        elif kind == 3:
            L = rng.integers(256, 1025, size=B)
            L[rng.integers(0, B)] = 32768
        else:
            L = rng.integers(0, 200000, size=B)
        if rng.random() < 0.2:
            L[rng.random(B) < 0.3] = 0
        M = int(rng.choice([8, 16, 32, 64, 128, 256]))
        fmt = "fp8" if rng.random() < 0.3 else "bf16"
        parts = int(rng.choice([0, 1, 2, 3, 7, 64, 255, 1024]))
        _same(L, M, 1, fmt, parts, f"trial {trial}: B={B} M={M} parts={parts}")


@pytest.mark.parametrize("L,parts", [([0], 1), ([0] * 9, 4), ([1], 1024), ([5, 0, 7], 1024), ([64] * 1023, 1),
                                     ([32768], 1024), ([1, 2, 3], 0)])
def test_device_metadata_edge_cases(L, parts):
    _same(L, 128, 1, "bf16", parts, f"L={L[:5]} parts={parts}")
    _same(L, 16, 1, "bf16", parts, f"L={L[:5]} parts={parts}")


@pytest.mark.parametrize("name", ["compute_heavy", "ragged"])
def test_decode_with_device_metadata_is_bitwise_equal(name):
    import paged_mla_decode_amd as mla
    w = named_workload(name)
    q, kv, bt, L = w.q.to(DEV), w.kvcache.to(DEV), w.block_table.to(DEV), w.cache_seqlens.to(DEV)
    mh, sh = mla.mla_get_metadata(w.cache_seqlens, w.heads_per_kv, 1, device=DEV)
    md, sd = mla.mla_get_metadata_device(L, w.heads_per_kv, 1)
    # the same combine shape for both (the piece-count hint is a host-side fact)
    hint = int(getattr(sh, "_mla_max_splits", 0))
    o1, l1 = mla.MlaDecoder(q, kv, bt, L, 512, mh, sh, w.causal, max_splits=hint).run()
    o2, l2 = mla.MlaDecoder(q, kv, bt, L, 512, md, sd, w.causal, max_splits=hint).run()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("h_kv", [2, 4])
def test_device_metadata_equals_host_with_several_kv_heads(h_kv):
    # with several KV heads the default range count shrinks (the grid holds every KV head of a
    # range) and the runs of the device scheduler get longer
    rng = np.random.default_rng(77 + h_kv)
    for trial in range(40):
        B = int(rng.integers(1, 400))
        L = rng.integers(0, 6000, size=B) if trial % 2 == 0 else np.full(B, int(rng.integers(1, 9000)))
        M = int(rng.choice([16, 64, 128, 256]))
        fmt = "fp8" if trial % 3 == 0 else "bf16"
        _same(L, M, h_kv, fmt, 0, f"h_kv={h_kv} trial {trial}: B={B} M={M} {fmt}")


@pytest.mark.parametrize("fmt,h_q", [("bf16", 256), ("fp8", 32)])
def test_decode_with_device_metadata_two_kv_heads(fmt, h_q):
    # two KV heads (128 and 16 rows per head): the decode with device metadata gives the bits of
    # the decode with host metadata, and matches the oracle
    import oracle
    import paged_mla_decode_amd as mla
    w = make_workload(name="dev_hkv2", batch=6, s_q=1, h_q=h_q, h_kv=2, seqlens=[3000, 64, 1, 700, 5000, 129],
                      kv_format=fmt, seed=17)
    q, kv, bt, L = w.q.to(DEV), w.kvcache.to(DEV), w.block_table.to(DEV), w.cache_seqlens.to(DEV)
    mh, sh = mla.mla_get_metadata(w.cache_seqlens, w.heads_per_kv, 2, kv_format=fmt, device=DEV)
    md, sd = mla.mla_get_metadata_device(L, w.heads_per_kv, 2, kv_format=fmt)
    hint = int(getattr(sh, "_mla_max_splits", 0))
    o1, l1 = mla.MlaDecoder(q, kv, bt, L, 512, mh, sh, w.causal, max_splits=hint).run()
    o2, l2 = mla.MlaDecoder(q, kv, bt, L, 512, md, sd, w.causal, max_splits=hint).run()
    torch.cuda.synchronize()
    print(f"[sched] dev_hkv2 {fmt} h_q={h_q}", flush=True)
    assert torch.equal(md.cpu(), mh.cpu()) and torch.equal(sd.cpu(), sh.cpu())
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    O_ref, L_ref = oracle.mla_decode_workload(w)
    O = o2.float().cpu().numpy().astype(np.float64)
    LS = l2.cpu().numpy().astype(np.float64)
    tol = 1e-2 if fmt == "bf16" else 3e-2
    assert np.all(np.isfinite(O)) and float(np.max(np.abs(O - O_ref))) <= tol
    assert float(np.max(np.abs(LS - L_ref))) <= 1e-3


def test_device_metadata_for_lengths_past_its_limit_is_empty():
    # more than 2^20 pages in one sequence: every range empty and no pieces (the decode then
    # reports every sequence as NaN) -- the host scheduler has no such limit
    import paged_mla_decode_amd as mla
    L = torch.tensor([100, (1 << 26) + 64, 5], dtype=torch.int32, device=DEV)
    md, sd = mla.mla_get_metadata_device(L, 128, 1, num_parts=8)
    torch.cuda.synchronize()
    md, sd = md.cpu(), sd.cpu()
    assert torch.all(md[:, 0] == -1) and torch.all(md[:, 6] == 3) and torch.all(sd == 0)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_unknown_piece_count_hint(fmt):
    """max_splits = 0 (the piece count is not known on the host, as with device-built metadata):
    tiles of at most 64 rows take the combine with helper workgroups, so a sequence of many
    pieces is merged in one round of loads; sequences of at most 8 pieces give the same bits as
    with the hint, and every sequence matches the oracle."""
    import oracle
    import paged_mla_decode_amd as mla
    w = make_workload(name="hint0", batch=5, s_q=1, h_q=16, seqlens=[6000, 300, 40, 900, 2500], kv_format=fmt,
                      seed=91)
    q, kv, bt, L = w.q.to(DEV), w.kvcache.to(DEV), w.block_table.to(DEV), w.cache_seqlens.to(DEV)
    mh, sh = mla.mla_get_metadata(w.cache_seqlens, w.heads_per_kv, 1, kv_format=fmt, num_parts=256)
    n = np.diff(sh.cpu().numpy())
    assert n.max() > 8 and (n <= 8).any(), n
    hint = int(getattr(sh, "_mla_max_splits", 0))
    o1, l1 = mla.MlaDecoder(q, kv, bt, L, 512, mh, sh, w.causal, max_splits=hint).run()
    o0, l0 = mla.MlaDecoder(q, kv, bt, L, 512, mh, sh, w.causal, max_splits=0).run()
    torch.cuda.synchronize()
    few = [b for b in range(w.batch) if n[b] <= 8]
    assert torch.equal(o0[few], o1[few]) and torch.equal(l0[few], l1[few])
    O_ref, L_ref = oracle.mla_decode_workload(w)
    O = o0.float().cpu().numpy().astype(np.float64)
    LS = l0.cpu().numpy().astype(np.float64)
    tol = 1e-2 if fmt == "bf16" else 3e-2
    assert np.all(np.isfinite(O)) and float(np.max(np.abs(O - O_ref))) <= tol
    assert float(np.max(np.abs(LS - L_ref))) <= 1e-3
