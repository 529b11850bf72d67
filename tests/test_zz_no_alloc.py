"""The entry point that allocates nothing (mla_decode_kvcache_noalloc): its static
scratch replaces the caller's workspace. Called through the C ABI, its outputs must
equal mla_decode_kvcache's bit for bit (the same kernels) and match the oracle, on
consecutive calls of different sizes that share the one scratch array."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from workloads import make_workload

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")


def _decode(w, no_alloc):
    import paged_mla_decode_amd as mla
    from paged_mla_decode_amd import _lib
    meta, splits = mla.mla_get_metadata(w.cache_seqlens, w.heads_per_kv, w.h_kv, kv_format=w.kv_format,
                                        max_blocks_per_seq=int(w.block_table.shape[1]), device=DEV)
    out = torch.full((w.batch, w.s_q, w.h_q, w.dv), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((w.batch, w.h_q, w.s_q), float("nan"), dtype=torch.float32, device=DEV)
    dec = mla.MlaDecoder(w.q.to(DEV), w.kvcache.to(DEV), w.block_table.to(DEV), w.cache_seqlens.to(DEV), w.dv,
                         meta, splits, w.causal, w.softmax_scale, out=out, lse=lse, no_alloc=no_alloc)
    lib = _lib.load()
    entry = lib.mla_decode_kvcache_noalloc if no_alloc else lib.mla_decode_kvcache
    if no_alloc:
        assert dec.args.workspace is None and dec.args.workspace_bytes == 0
    st = entry(ctypes.byref(dec.args), ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream))
    _lib.check(st)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(w, label):
    O_s, L_s = _decode(w, no_alloc=True)
    O_w, L_w = _decode(w, no_alloc=False)
    assert np.array_equal(O_s, O_w) and np.array_equal(L_s, L_w), f"{label}: scratch and workspace calls differ"
    O_ref, L_ref = oracle.mla_decode_workload(w)
    empty = np.isneginf(L_ref)
    assert np.array_equal(np.isneginf(L_s), empty) and np.all(np.isfinite(O_s))
    tol = 1e-2 if w.kv_format == "bf16" else 3e-2
    dO = float(np.max(np.abs(O_s - O_ref)))
    dL = float(np.max(np.abs(L_s[~empty] - L_ref[~empty])))
    print(f"[noalloc] {label}: max|dO|={dO:.3e} max|dLSE|={dL:.3e}", flush=True)
    assert dO <= tol and dL <= 1e-3


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_noalloc_matches_workspace_entry_on_consecutive_calls(fmt):
    # a large call (128-row tiles, sequences cut into several pieces), then a smaller one
    # (16 rows, fp32 partials) that reuses the scratch the first one left behind
    big = make_workload(name="na_big", batch=24, s_q=2, h_q=128, seqlens=list(range(100, 24 * 150 + 100, 150)),
                        causal=True, kv_format=fmt, seed=71)
    small = make_workload(name="na_small", batch=3, s_q=1, h_q=16, seqlens=[5, 700, 64], kv_format=fmt, seed=72)
    _check(big, f"{fmt} first call, batch 24 x 256 rows")
    _check(small, f"{fmt} second call, batch 3 x 16 rows")
