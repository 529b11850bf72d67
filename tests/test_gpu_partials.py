"""The 128-row kernels' fp16 partials (each 64-dim block of a piece's O scaled by a power of two)
in their worst case: every 64-dim block of V holds one value about 10^6 times larger than the
others (positive values near 2e-3 beside +-1000), and each sequence is cut into many pieces.

The bound is the arithmetic's, per element: P enters the MFMA in bf16 (relative error 2^-9 per
weight, so the error of O[d] scales with sum_t p_t |V[t, d]| / l, the attention average of |V|,
computed by the oracle itself with |V| as a separate V cache) and O leaves in bf16 (2^-9 |O|):
|dO| <= 2^-7 avg|V| + 2^-8 |O| + 1e-7. If the block scale let the small values of a block with a
large one round away (or flush to zero), their error would be about |O| itself, far above this.
Checked for one piece per sequence (no partials) and for many pieces."""
import numpy as np
import pytest
import torch

import oracle
from workloads import make_workload

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")


def _mixed_magnitude_workload():
    w = make_workload(name="mixed", batch=2, s_q=1, h_q=128, seqlens=[4096, 3000], seed=501)
    gen = torch.Generator().manual_seed(502)
    kv = w.kvcache.float()
    big = kv[..., :512].view(*kv.shape[:-1], 8, 64)
    big.abs_().mul_(1e-3).add_(1e-3)                                   # the many small values, ~2e-3
    sign = torch.randint(0, 2, big[..., 0].shape, generator=gen).float() * 2 - 1
    big[..., 0] = sign * 1000.0                                        # one large value per block
    w.kvcache = kv.to(torch.bfloat16)
    q = w.q.float()
    q[..., :512].view(*q.shape[:-1], 8, 64)[..., 0] = 0.0               # logits do not see the large dims
    w.q = q.to(torch.bfloat16)
    return w


def _run(w, num_parts):
    import paged_mla_decode_amd as mla
    meta, splits = mla.mla_get_metadata(w.cache_seqlens, w.heads_per_kv, 1, num_parts=num_parts, device=DEV)
    o, lse = mla.mla_decode_kvcache(w.q.to(DEV), w.kvcache.to(DEV), w.block_table.to(DEV), w.cache_seqlens.to(DEV),
                                    512, meta, splits, softmax_scale=w.softmax_scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), splits.cpu()


def test_fp16_partials_mixed_magnitudes_many_pieces():
    w = _mixed_magnitude_workload()
    O_ref, LSE_ref = oracle.mla_decode_workload(w)
    a = w.as_numpy()
    absv = w.kvcache[..., :512].abs().contiguous().view(torch.int16).numpy().view(np.uint16)
    avg_abs, _ = oracle.mla_decode(a["q_bits"], a["kvcache"], "bf16", a["block_table"], a["cache_seqlens"],
                                   softmax_scale=w.softmax_scale, vcache=absv)
    O1, L1, s1 = _run(w, 1)                  # one range: one piece per sequence, no partials
    On, Ln, sn = _run(w, 96)
    pieces = (sn[1:] - sn[:-1]).tolist()
    print(f"[case] mixed magnitudes: pieces per sequence {pieces}", flush=True)
    assert min(pieces) >= 16, pieces
    assert (s1[1:] - s1[:-1]).tolist() == [1, 1]
    tol = 2.0 ** -7 * avg_abs + 2.0 ** -8 * np.abs(O_ref) + 1e-7
    small = np.ones(512, dtype=bool)
    small[::64] = False
    for O, L, label in [(O1, L1, "one piece"), (On, Ln, "many pieces")]:
        assert np.all(np.isfinite(O)) and np.all(np.isfinite(L)), label
        err = np.abs(O - O_ref)
        rel_small = err[..., small] / np.abs(O_ref[..., small])
        print(f"[parity] {label}: max |dO| / bound = {float(np.max(err / tol)):.3f}, small values: max rel "
              f"{float(np.max(rel_small)):.2e}, median rel {float(np.median(rel_small)):.2e}; max|dLSE| = "
              f"{float(np.max(np.abs(L - LSE_ref))):.3e}", flush=True)
        assert np.all(err <= tol), f"{label}: {int(np.sum(err > tol))} elements outside the bound"
        assert np.max(np.abs(L - LSE_ref)) <= 1e-3, label
        assert np.max(rel_small) <= 2.0 ** -6, label
