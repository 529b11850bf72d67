"""Seeded input generators for paged MLA decode workloads.

Shapes and value distributions follow the workloads the FlashMLA pages
describe: queries [batch, s_q, h_q, 576] in BF16, one latent KV head of 576
dims (512 latent + 64 RoPE) stored in 64-token pages that a block table
addresses, per-sequence lengths in int32 ("flash_api.cpp 核心逻辑" on the
mmssai.com FlashMLA article; "Dynamische Sequenzoptimierung" on the
deepseekonline.chat day-1 post), and the FP8 record of 656 bytes per token
("FP8 KV缓存" on the wmrh.cn FlashMLA深度解析 page).

Recipe (the same for every workload):
  * integer structure (lengths, page permutation, the ragged sequence's
    index) from numpy.random.Generator(PCG64(seed));
  * values from torch.Generator().manual_seed(seed): N(0, 1) float32 rounded
    to bfloat16, drawn in the order q, then the page pool;
  * page pool of sum(ceil(L_b / 64)) pages (or a stated size), physical ids
    a seeded permutation of the pool assigned consecutively to sequences in
    batch order; unused block-table entries are 0;
  * every token slot of every page, tails included, holds N(0, 1) values.

FP8 records are produced here by an encoder the decode path never runs:
scale_c = amax_c / 448 per 128-element latent chunk (1.0 when the chunk is
all zero), codes = the round-to-nearest-even cast to float8_e4m3fn of the
chunk divided by its scale (clamped to +-448 first), RoPE dims in bfloat16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Sequence

import numpy as np
import torch

PAGE = 64
D_QK = 576
D_V = 512
D_ROPE = 64
FP8_RECORD = 656
FP8_NOPE_BYTES = 512
FP8_SCALE_OFF = 512
FP8_ROPE_OFF = 528
E4M3_MAX = 448.0


@dataclass
class Workload:
    name: str
    q: torch.Tensor              # bf16 [B, S, H, 576]
    kvcache: torch.Tensor        # bf16 [P, 64, Hk, 576] or uint8 [P, 64, Hk, 656]
    kv_format: str               # "bf16" | "fp8"
    block_table: torch.Tensor    # int32 [B, max_blocks]
    cache_seqlens: torch.Tensor  # int32 [B]
    causal: bool
    softmax_scale: float
    dv: int = D_V
    seed: int = 0
    meta: Dict[str, object] = field(default_factory=dict)
    indices: Optional[torch.Tensor] = None   # int32 [B, S, topk] for token-level sparse decode (-1: padding)
    vcache: Optional[torch.Tensor] = None    # bf16 [P, 64, Hk, dv]: V rows apart from the keys

    @property
    def topk(self) -> int:
        return 0 if self.indices is None else int(self.indices.shape[2])

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def s_q(self) -> int:
        return int(self.q.shape[1])

    @property
    def h_q(self) -> int:
        return int(self.q.shape[2])

    @property
    def h_kv(self) -> int:
        return int(self.kvcache.shape[2])

    @property
    def num_pages(self) -> int:
        return int(self.kvcache.shape[0])

    @property
    def heads_per_kv(self) -> int:
        """Rows per KV head handed to the scheduler: s_q * h_q // h_kv."""
        return self.s_q * self.h_q // self.h_kv

    def as_numpy(self) -> Dict[str, np.ndarray]:
        """Raw views for numpy consumers: bf16 tensors as their uint16 bit patterns."""
        kv = self.kvcache
        kv_np = kv.view(torch.int16).numpy().view(np.uint16) if kv.dtype == torch.bfloat16 else kv.numpy()
        d = dict(
            q_bits=self.q.view(torch.int16).numpy().view(np.uint16),
            kvcache=kv_np,
            block_table=self.block_table.numpy(),
            cache_seqlens=self.cache_seqlens.numpy(),
        )
        if self.vcache is not None:
            d["vcache"] = self.vcache.view(torch.int16).numpy().view(np.uint16)
        return d


def _randn_bf16(gen: torch.Generator, shape, chunk_elems: int = 1 << 26) -> torch.Tensor:
    """N(0,1) float32 draws rounded to bf16, produced chunk by chunk."""
    total = int(np.prod(shape))
    out = torch.empty(total, dtype=torch.bfloat16)
    pos = 0
    while pos < total:
        n = min(chunk_elems, total - pos)
        out[pos:pos + n] = torch.randn(n, generator=gen, dtype=torch.float32).to(torch.bfloat16)
        pos += n
    return out.view(*shape)


def quantize_fp8_records(latent: torch.Tensor, rope_bf16: torch.Tensor) -> torch.Tensor:
    """Encode float32 latent [..., 512] and bf16 RoPE [..., 64] into 656-byte records.

    Byte layout per token: [0, 512) e4m3fn codes, [512, 528) four little-endian
    float32 scales (scale c covers latent dims [128c, 128c + 128)), [528, 656)
    64 little-endian bf16 RoPE values.
    """
    lead = latent.shape[:-1]
    x = latent.reshape(-1, 4, 128).to(torch.float32)
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (x / scale.unsqueeze(-1)).clamp(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(-1, 512)
    rec = torch.empty(codes.shape[0], FP8_RECORD, dtype=torch.uint8)
    rec[:, :FP8_NOPE_BYTES] = codes
    rec[:, FP8_SCALE_OFF:FP8_ROPE_OFF] = scale.contiguous().view(torch.uint8).reshape(-1, 16)
    rec[:, FP8_ROPE_OFF:] = rope_bf16.reshape(-1, D_ROPE).contiguous().view(torch.uint8).reshape(-1, 128)
    return rec.reshape(*lead, FP8_RECORD)


def _fp8_pool(gen: torch.Generator, num_pages: int, h_kv: int, chunk_pages: int = 1024) -> torch.Tensor:
    out = torch.empty(num_pages, PAGE, h_kv, FP8_RECORD, dtype=torch.uint8)
    for p0 in range(0, num_pages, chunk_pages):
        p1 = min(num_pages, p0 + chunk_pages)
        n = p1 - p0
        latent = torch.randn(n, PAGE, h_kv, D_V, generator=gen, dtype=torch.float32)
        rope = torch.randn(n, PAGE, h_kv, D_ROPE, generator=gen, dtype=torch.float32).to(torch.bfloat16)
        out[p0:p1] = quantize_fp8_records(latent, rope)
    return out


def make_workload(
    *,
    name: str,
    batch: int,
    s_q: int,
    h_q: int,
    h_kv: int = 1,
    seqlens: Sequence[int],
    kv_format: str = "bf16",
    causal: bool = False,
    seed: int = 0,
    pool_pages: Optional[int] = None,
    max_blocks: Optional[int] = None,
    softmax_scale: Optional[float] = None,
    rng: Optional[np.random.Generator] = None,
    vcache: bool = False,
) -> Workload:
    """Build one workload from explicit lengths.

    `pool_pages` (default: the pages the lengths need) sizes the physical
    pool; extra pages stay unreferenced. `max_blocks` widens the block table
    beyond the longest sequence. `vcache`: also draw a separate bf16 V cache
    [pool, 64, h_kv, 512] (after q and the keys, from the same generator).
    """
    if kv_format not in ("bf16", "fp8"):
        raise ValueError(f"kv_format must be 'bf16' or 'fp8', got {kv_format!r}")
    if h_q % h_kv:
        raise ValueError("h_q must be a multiple of h_kv")
    L = np.asarray(list(seqlens), dtype=np.int64)
    if L.shape != (batch,):
        raise ValueError("need one length per sequence")
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    npages = (L + PAGE - 1) // PAGE
    need = int(npages.sum())
    pool = need if pool_pages is None else int(pool_pages)
    if pool < need:
        raise ValueError(f"pool of {pool} pages is smaller than the {need} the lengths need")
    pool = max(pool, 1)
    nb = int(npages.max()) if batch else 0
    nb = max(nb, 1) if max_blocks is None else max(int(max_blocks), nb, 1)
    perm = rng.permutation(pool)
    bt = np.zeros((batch, nb), dtype=np.int32)
    pos = 0
    for b in range(batch):
        k = int(npages[b])
        bt[b, :k] = perm[pos:pos + k]
        pos += k

    gen = torch.Generator().manual_seed(seed)
    q = _randn_bf16(gen, (batch, s_q, h_q, D_QK))
    if kv_format == "bf16":
        kv = _randn_bf16(gen, (pool, PAGE, h_kv, D_QK))
    else:
        kv = _fp8_pool(gen, pool, h_kv)
    vc = _randn_bf16(gen, (pool, PAGE, h_kv, D_V)) if vcache else None
    scale = 1.0 / math.sqrt(D_QK) if softmax_scale is None else float(softmax_scale)
    return Workload(
        name=name, q=q, kvcache=kv, kv_format=kv_format,
        block_table=torch.from_numpy(bt), cache_seqlens=torch.from_numpy(L.astype(np.int32)),
        causal=bool(causal), softmax_scale=scale, seed=seed, vcache=vc,
    )


def draw_indices(L: Sequence[int], s_q: int, topk: int, causal: bool, rng: np.random.Generator,
                 duplicates: float = 0.0, padding: float = 0.0) -> torch.Tensor:
    """Seeded token selections for sparse decode: int32 [B, s_q, topk].

    Row (b, s) draws topk distinct positions uniformly, in random order, from the tokens the
    query may see ([0, L_b), or [0, L_b - s_q + s] when causal); when there are fewer than
    topk the row lists all of them and pads with -1. `duplicates` is the share of entries
    then overwritten by another entry of the same row, `padding` the share set to -1."""
    B = len(L)
    out = np.full((B, s_q, topk), -1, dtype=np.int64)
    for b in range(B):
        for s in range(s_q):
            n = int(L[b]) - (s_q - 1 - s if causal else 0)
            n = max(n, 0)
            k = min(n, topk)
            if k:
                out[b, s, :k] = rng.choice(n, size=k, replace=False)
            if duplicates and k > 1:
                m = rng.random(topk) < duplicates
                m[:1] = False
                src = rng.integers(0, k, size=topk)
                out[b, s, m & (np.arange(topk) < k)] = out[b, s, src[m & (np.arange(topk) < k)]]
            if padding:
                out[b, s, rng.random(topk) < padding] = -1
            out[b, s] = out[b, s, rng.permutation(topk)]
    return torch.from_numpy(out.astype(np.int32))


def make_sparse_workload(*, topk: int, duplicates: float = 0.0, padding: float = 0.0, **kwargs) -> Workload:
    """make_workload plus indices drawn by draw_indices from the same seed (after the values)."""
    w = make_workload(**kwargs)
    rng = np.random.Generator(np.random.PCG64(int(kwargs.get("seed", 0)) + 7919))
    w.indices = draw_indices(w.cache_seqlens.tolist(), w.s_q, topk, w.causal, rng, duplicates, padding)
    return w


# The six workloads: the five stated decode configurations, the fourth with
# its ragged and its uniform run. Lengths are drawn from the seeded rng.
WORKLOAD_SPECS: Dict[str, Dict[str, object]] = {
    "tiny": dict(batch=2, s_q=1, h_q=16, causal=False, kv_format="bf16", seed=1,
                 lengths=("fixed", [100, 257]), pool_pages=16,
                 text="batch=2, s_q=1, h_q=16, L={100,257}, 16-page pool, non-causal"),
    "compute_heavy": dict(batch=64, s_q=1, h_q=128, causal=False, kv_format="bf16", seed=2,
                          lengths=("uniform", 1, 4096),
                          text="batch=64, s_q=1, h_q=128, L~U[1,4096], shuffled pool"),
    "mtp": dict(batch=128, s_q=2, h_q=128, causal=True, kv_format="bf16", seed=3,
                lengths=("uniform", 3072, 5120),
                text="batch=128, s_q=2, h_q=128, causal, L~U[3072,5120]"),
    "ragged": dict(batch=128, s_q=1, h_q=16, causal=False, kv_format="bf16", seed=4,
                   lengths=("ragged", 32768, 256, 1024),
                   text="batch=128, s_q=1, h_q=16, one L=32768, rest U[256,1024]"),
    "uniform_long": dict(batch=128, s_q=1, h_q=16, causal=False, kv_format="bf16", seed=44,
                         lengths=("fixed", [8192] * 128),
                         text="batch=128, s_q=1, h_q=16, all L=8192"),
    "fp8": dict(batch=64, s_q=1, h_q=128, causal=False, kv_format="fp8", seed=5,
                lengths=("fixed", [8192] * 64),
                text="batch=64, s_q=1, h_q=128, all L=8192, FP8 656 B/token"),
    # token-level sparse decode over an FP8 cache: every query token attends to 2048 of its
    # sequence's 16384 cached tokens
    # a separate bf16 V cache beside the keys (the optional V cache of the decode call)
    "vcache": dict(batch=128, s_q=1, h_q=16, causal=False, kv_format="bf16", seed=8,
                   lengths=("uniform", 1024, 8192), vcache=True,
                   text="batch=128, s_q=1, h_q=16, L~U[1024,8192], separate bf16 V cache [pages, 64, 1, 512]"),
    "sparse_fp8": dict(batch=64, s_q=1, h_q=128, causal=False, kv_format="fp8", seed=6,
                       lengths=("fixed", [16384] * 64), topk=2048,
                       text="batch=64, s_q=1, h_q=128, all L=16384, topk=2048 of them per query token, "
                            "FP8 656 B/token"),
}


def _draw_lengths(spec, batch: int, rng: np.random.Generator) -> np.ndarray:
    kind = spec[0]
    if kind == "fixed":
        return np.asarray(spec[1], dtype=np.int64)
    if kind == "uniform":
        lo, hi = spec[1], spec[2]
        return rng.integers(lo, hi + 1, size=batch, dtype=np.int64)
    if kind == "ragged":
        long_len, lo, hi = spec[1], spec[2], spec[3]
        L = rng.integers(lo, hi + 1, size=batch, dtype=np.int64)
        L[int(rng.integers(0, batch))] = long_len
        return L
    raise ValueError(kind)


def named_workload(name: str, **overrides) -> Workload:
    """One of WORKLOAD_SPECS at its full size, reproducibly seeded."""
    spec = dict(WORKLOAD_SPECS[name])
    spec.update(overrides)
    rng = np.random.Generator(np.random.PCG64(int(spec["seed"])))
    L = _draw_lengths(spec["lengths"], int(spec["batch"]), rng)
    w = make_workload(name=name, batch=int(spec["batch"]), s_q=int(spec["s_q"]), h_q=int(spec["h_q"]),
                      h_kv=1, seqlens=L.tolist(), kv_format=str(spec["kv_format"]),
                      causal=bool(spec["causal"]), seed=int(spec["seed"]),
                      pool_pages=spec.get("pool_pages"), rng=rng, vcache=bool(spec.get("vcache", False)))
    if spec.get("topk"):
        irng = np.random.Generator(np.random.PCG64(int(spec["seed"]) + 7919))
        w.indices = draw_indices(w.cache_seqlens.tolist(), w.s_q, int(spec["topk"]), w.causal, irng)
    w.meta["text"] = spec["text"]
    return w


def poison_unused(w: Workload) -> Workload:
    """Copy of `w` whose never-read cache bytes are NaN.

    Adds one extra page filled with NaN (bf16 0x7FC0, or e4m3fn code 0x7F in
    every latent byte, NaN scales and NaN RoPE), points every unused
    block-table entry at it, and overwrites each sequence's last-page tail
    (token slots >= L_b) with the same NaN pattern. Attention results must not
    change.
    """
    kv = w.kvcache
    P = kv.shape[0]
    if w.kv_format == "bf16":
        nan_row = torch.full((kv.shape[-1],), float("nan"), dtype=torch.bfloat16)
    else:
        nan_row = torch.empty(FP8_RECORD, dtype=torch.uint8)
        nan_row[:FP8_NOPE_BYTES] = 0x7F
        nan_row[FP8_SCALE_OFF:FP8_ROPE_OFF] = torch.full((4,), float("nan")).view(torch.uint8)
        nan_row[FP8_ROPE_OFF:] = torch.full((64,), float("nan"), dtype=torch.bfloat16).view(torch.uint8)
    kv2 = torch.empty((P + 1,) + tuple(kv.shape[1:]), dtype=kv.dtype)
    kv2[:P] = kv
    kv2[P] = nan_row
    vc2 = None
    if w.vcache is not None:
        vc2 = torch.empty((P + 1,) + tuple(w.vcache.shape[1:]), dtype=w.vcache.dtype)
        vc2[:P] = w.vcache
        vc2[P] = float("nan")
    bt = w.block_table.clone()
    L = w.cache_seqlens.tolist()
    for b, Lb in enumerate(L):
        n = (Lb + PAGE - 1) // PAGE
        bt[b, n:] = P
        if Lb % PAGE:
            last = int(bt[b, n - 1])
            kv2[last, Lb % PAGE:] = nan_row
            if vc2 is not None:
                vc2[last, Lb % PAGE:] = float("nan")
    return replace(w, kvcache=kv2, block_table=bt, vcache=vc2, name=w.name + "+poison")


def permute_pages(w: Workload, seed: int) -> Workload:
    """Copy of `w` with the physical pages shuffled and the block table renamed to match."""
    rng = np.random.Generator(np.random.PCG64(seed))
    P = w.kvcache.shape[0]
    perm = torch.from_numpy(rng.permutation(P).astype(np.int64))   # new position of old page i
    kv2 = torch.empty_like(w.kvcache)
    kv2[perm] = w.kvcache
    vc2 = None
    if w.vcache is not None:
        vc2 = torch.empty_like(w.vcache)
        vc2[perm] = w.vcache
    bt = w.block_table.clone()
    L = w.cache_seqlens.tolist()
    for b, Lb in enumerate(L):
        n = (Lb + PAGE - 1) // PAGE
        bt[b, :n] = perm[w.block_table[b, :n].long()].to(torch.int32)
    return replace(w, kvcache=kv2, block_table=bt, vcache=vc2, name=w.name + "+permuted")


def dense_as_sparse(w: Workload) -> Workload:
    """Copy of `w` whose indices list every cached token of each sequence once, in order
    (topk = the longest sequence, shorter rows padded with -1)."""
    L = w.cache_seqlens.tolist()
    topk = max(max(L), 1)
    idx = torch.full((w.batch, w.s_q, topk), -1, dtype=torch.int32)
    for b, Lb in enumerate(L):
        idx[b, :, :Lb] = torch.arange(Lb, dtype=torch.int32)
    return replace(w, indices=idx, name=w.name + "+as-sparse")


@dataclass
class PrefillWorkload:
    """Sparse prefill inputs: q bf16 [s_q, h_q, 576], kv bf16 [s_kv, h_kv, 576] (contiguous rows),
    indices int32 [s_q, h_kv, topk] (rows of kv; -1: padding)."""
    name: str
    q: torch.Tensor
    kv: torch.Tensor
    indices: torch.Tensor
    softmax_scale: float
    dv: int = D_V
    seed: int = 0
    meta: Dict[str, object] = field(default_factory=dict)

    @property
    def s_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def h_q(self) -> int:
        return int(self.q.shape[1])

    @property
    def s_kv(self) -> int:
        return int(self.kv.shape[0])

    @property
    def h_kv(self) -> int:
        return int(self.kv.shape[1])

    @property
    def topk(self) -> int:
        return int(self.indices.shape[2])

    def as_numpy(self) -> Dict[str, np.ndarray]:
        return dict(q_bits=self.q.view(torch.int16).numpy().view(np.uint16),
                    kv_bits=self.kv.view(torch.int16).numpy().view(np.uint16),
                    indices=self.indices.numpy())


def make_prefill_workload(*, name: str, s_q: int, h_q: int, s_kv: int, topk: int, h_kv: int = 1, seed: int = 0,
                          duplicates: float = 0.0, padding: float = 0.0,
                          softmax_scale: Optional[float] = None) -> PrefillWorkload:
    """Seeded sparse-prefill inputs: values from torch.Generator(seed) (q, then kv: N(0, 1) rounded to
    bf16); each (s, kvh) lists topk distinct rows of kv drawn uniformly (numpy PCG64(seed)), in random
    order (all rows and -1 padding when s_kv < topk); duplicates / padding as in draw_indices."""
    gen = torch.Generator().manual_seed(seed)
    q = _randn_bf16(gen, (s_q, h_q, D_QK))
    kv = _randn_bf16(gen, (s_kv, h_kv, D_QK))
    rng = np.random.Generator(np.random.PCG64(seed))
    idx = draw_indices([s_kv] * s_q, h_kv, topk, False, rng, duplicates, padding)     # [s_q, h_kv, topk]
    scale = 1.0 / math.sqrt(D_QK) if softmax_scale is None else float(softmax_scale)
    return PrefillWorkload(name=name, q=q, kv=kv, indices=idx, softmax_scale=scale, seed=seed)


PREFILL_SPECS: Dict[str, Dict[str, object]] = {
    # every one of 4096 query tokens attends to 2048 of 8192 rows (h_q = 128 heads, one latent KV head)
    "sparse_prefill": dict(s_q=4096, h_q=128, s_kv=8192, topk=2048, h_kv=1, seed=7,
                           text="s_q=4096, h_q=128, s_kv=8192, h_kv=1, topk=2048, bf16"),
}


def named_prefill(name: str) -> PrefillWorkload:
    spec = dict(PREFILL_SPECS[name])
    text = spec.pop("text")
    w = make_prefill_workload(name=name, **spec)
    w.meta["text"] = text
    return w
