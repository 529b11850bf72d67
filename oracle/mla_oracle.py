"""Plain fp64 reference for MLA decode over a paged KV cache.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
benchmark's cpu_baseline leg, never by the product path. It shares no code
with the HIP library.

What is computed (the plain definition; the split-KV kernel and its LSE merge
are an exact rearrangement of it, up to rounding):

  For each sequence b with L_b cached tokens, token t lives in physical page
  block_table[b, t // 64] at slot t % 64 (64-token pages: "功能 2" on the
  kdjingpai.com FlashMLA post; block_table [batch, max_num_blocks_per_seq] and
  kcache [num_blocks, page_block_size, num_heads_k, head_size] in
  "代码解读：flash_api.cpp 核心逻辑" on the mmssai.com article).
  Query head h reads KV head h // G with G = h_q / h_kv (the query view
  [b, s, h_k, ngroups, d] in "Dynamische Sequenzoptimierung" on the
  deepseekonline.chat day-1 post).
  Keys are the 576-dim cached rows (run_mha_fwd_splitkv_mla<bf16, 576> on the
  mmssai.com article); values are their first dv = 512 dims (d_v=512 in the
  sparse-prefill example on the wmrh.cn page).
      z_t   = scale * <q[b,s,h,:], K_t>             over allowed t
      LSE   = ln sum_t exp(z_t)                      (natural log)
      O     = sum_t exp(z_t - LSE) * V_t
  The call returns both the attention output and the natural-log softmax
  normaliser (mmssai.com article, section "代码解读：flash_api.cpp 核心逻辑";
  the (o_i, lse_i) pair in "功能 1" on kdjingpai.com), here as
  o [b, s_q, h_q, dv] and lse [b, h_q, s_q].

Readings taken where the pages are silent (each listed in the design notes):
  * causal (passed as causal=True in every usage example) is bottom-right
    aligned: query token s of S may read keys t <= L_b - S + s; with S == 1
    causal changes nothing;
  * a query row with no allowed key has O = 0 and LSE = -inf (empty sum) --
    parity unpinned: no page fixes it, it is a convention;
  * the lse layout [b, h_q, s_q] is an interface choice -- parity unpinned;
  * FP8 record (the "FP8 KV缓存" table on the wmrh.cn page): bytes [0,512)
    float8_e4m3 codes (OCP E4M3FN), [512,528) four little-endian float32
    scales, scale c multiplying latent dims [128c, 128c+128), [528,656) 64
    little-endian bf16 RoPE dims; V under FP8 is the dequantised latent.

Arithmetic is float64 throughout; bf16 inputs convert exactly. The softmax is
evaluated as exp(z - LSE) with LSE = max + ln sum exp(z - max), which is the
definition rearranged exactly (no approximation). Matrix products use numpy's
matmul as the library primitive.
"""
from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np

PAGE = 64
D_QK = 576
D_V = 512
D_ROPE = 64
FP8_RECORD = 656


# ---------------------------------------------------------------------------
# Element decoders
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN code -> float64.

    sign = bit 7, exponent = bits 6..3 (bias 7), mantissa = bits 2..0.
    exponent 0: subnormal (m / 8) * 2^-6; exponent 1..15: (1 + m / 8) * 2^(e - 7);
    S.1111.111 is NaN; there is no infinity (the format the wmrh.cn page names
    "float8_e4m3" in its FP8 KV缓存 table).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = sign * mag
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, val)


def decode_fp8_records(rec: np.ndarray) -> np.ndarray:
    """656-byte FP8 records [..., 656] (uint8) -> dequantised rows [..., 576] float64.

    latent[j] = e4m3fn(rec[j]) * scale[j // 128]  for j < 512
    rope[i]   = bf16(rec[528 + 2i : 530 + 2i])     for i < 64
    """
    r = np.ascontiguousarray(np.asarray(rec, dtype=np.uint8))
    if r.shape[-1] != FP8_RECORD:
        raise ValueError(f"FP8 record must be {FP8_RECORD} bytes, got {r.shape[-1]}")
    lead = r.shape[:-1]
    codes = r[..., :512]
    scales = r[..., 512:528].copy().view("<f4").astype(np.float64)           # [..., 4]
    rope_bits = r[..., 528:656].copy().view("<u2")                            # [..., 64]
    latent = e4m3fn_to_f64(codes).reshape(lead + (4, 128)) * scales[..., :, None]
    out = np.empty(lead + (D_QK,), dtype=np.float64)
    out[..., :512] = latent.reshape(lead + (512,))
    out[..., 512:] = bf16_bits_to_f64(rope_bits)
    return out


def decode_kv_rows(rows: np.ndarray, kv_format: str) -> np.ndarray:
    """Raw cached rows (bf16 bits [..., 576] or FP8 records [..., 656]) -> float64 [..., 576]."""
    if kv_format == "bf16":
        r = np.asarray(rows)
        if r.shape[-1] != D_QK:
            raise ValueError(f"bf16 rows must have {D_QK} dims")
        return bf16_bits_to_f64(r)
    if kv_format == "fp8":
        return decode_fp8_records(rows)
    raise ValueError(f"unknown kv_format {kv_format!r}")


# ---------------------------------------------------------------------------
# Paged gather, attention, and the split merge
# ---------------------------------------------------------------------------

def gather_sequence(kvcache: np.ndarray, kv_format: str, block_table_row: np.ndarray, L: int) -> np.ndarray:
    """Keys of one sequence in token order: float64 [L, h_kv, 576].

    Token t comes from page block_table_row[t // 64], slot t % 64.
    """
    L = int(L)
    nb = int(block_table_row.shape[0])
    if L < 0 or L > nb * PAGE:
        raise ValueError(f"sequence length {L} outside [0, {nb * PAGE}] for {nb} block-table entries")
    t = np.arange(L)
    pages = np.asarray(block_table_row)[t // PAGE].astype(np.int64)
    if L and (pages.min() < 0 or pages.max() >= kvcache.shape[0]):
        raise ValueError("block_table entry outside the page pool")
    rows = kvcache[pages, t % PAGE]                                          # [L, h_kv, raw]
    return decode_kv_rows(rows, kv_format)


def gather_values(vcache: np.ndarray, block_table_row: np.ndarray, L: int) -> np.ndarray:
    """Values of one sequence from a separate V cache, in token order: float64 [L, h_kv, dv].

    The optional vcache_ argument of mha_fwd_kvcache_mla (num_blocks x page_block_size x
    num_heads_k x head_size_v: mmssai.com, section "代码解读：flash_api.cpp 核心逻辑"). Reading:
    bf16 rows, addressed like the keys (token t at page block_table_row[t // 64], slot t % 64).
    """
    L = int(L)
    t = np.arange(L)
    page_of = np.asarray(block_table_row).astype(np.int64)[t // PAGE]
    if L and (page_of.min() < 0 or page_of.max() >= vcache.shape[0]):
        raise ValueError("block_table entry outside the V cache")
    return bf16_bits_to_f64(np.asarray(vcache)[page_of, t % PAGE])


def attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of query rows Q [n, d] over keys K [t, d], values V [t, dv].

    Returns (O [n, dv], LSE [n]); with t == 0, O = 0 and LSE = -inf.
    """
    Q = np.asarray(Q, dtype=np.float64)
    n = Q.shape[0]
    if K.shape[0] == 0:
        return np.zeros((n, V.shape[1])), np.full(n, -np.inf)
    z = scale * (Q @ K.T)                                                    # [n, t]
    mx = z.max(axis=1)
    lse = mx + np.log(np.exp(z - mx[:, None]).sum(axis=1))
    p = np.exp(z - lse[:, None])
    return p @ V, lse


def combine_partials(O_parts: Iterable[np.ndarray], lse_parts: Iterable[np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """Merge attention over disjoint key sets (the split-KV combine).

    LSE = ln sum_i exp(LSE_i);  O = sum_i exp(LSE_i - LSE) * O_i.
    Parts with LSE_i = -inf carry no weight; if every part is empty the
    result is O = 0, LSE = -inf.
    """
    O_parts = [np.asarray(o, dtype=np.float64) for o in O_parts]
    L = np.stack([np.asarray(l, dtype=np.float64) for l in lse_parts])      # [k, n]
    mx = L.max(axis=0)
    finite = np.isfinite(mx)
    safe = np.where(finite, mx, 0.0)
    w_un = np.exp(L - safe)                                                  # exp(-inf) = 0
    tot = w_un.sum(axis=0)
    lse = np.where(finite, safe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    O = np.zeros_like(O_parts[0])
    for i, o in enumerate(O_parts):
        w = np.where(finite, np.exp(L[i] - np.where(finite, lse, 0.0)), 0.0)
        O = O + w[:, None] * o
    return O, lse


def mla_decode(
    q_bits: np.ndarray,
    kvcache: np.ndarray,
    kv_format: str,
    block_table: np.ndarray,
    cache_seqlens: np.ndarray,
    *,
    dv: int = D_V,
    causal: bool = False,
    softmax_scale: Optional[float] = None,
    batches: Optional[Iterable[int]] = None,
    vcache: Optional[np.ndarray] = None,
) -> Tuple[np.ndarray, np.ndarray]:
    """Reference MLA decode.

    q_bits        uint16 [B, S, H, 576]  (bf16 bit patterns)
    kvcache       uint16 [P, 64, Hk, 576] (bf16 bits) or uint8 [P, 64, Hk, 656] (FP8 records)
    block_table   int    [B, NB]
    cache_seqlens int    [B]
    vcache        optional uint16 [P, 64, Hk, dv] (bf16 bits): V rows from here (gather_values)
                  instead of the first dv dims of the keys
    Returns O float64 [B, S, H, dv] and LSE float64 [B, H, S]. With `batches`,
    only those sequences are computed and the others are NaN.
    """
    q = np.asarray(q_bits)
    if q.ndim != 4 or q.shape[-1] != D_QK:
        raise ValueError("q must be [batch, s_q, h_q, 576]")
    B, S, H, _ = q.shape
    kv = np.asarray(kvcache)
    Hk = kv.shape[2]
    if H % Hk:
        raise ValueError("h_q must be a multiple of h_kv")
    if not (0 < dv <= D_QK):
        raise ValueError("dv must lie in (0, 576]")
    G = H // Hk
    scale = (1.0 / np.sqrt(D_QK)) if softmax_scale is None else float(softmax_scale)
    seqlens = np.asarray(cache_seqlens).astype(np.int64)
    bt = np.asarray(block_table)
    O = np.full((B, S, H, dv), np.nan)
    LSE = np.full((B, H, S), np.nan)
    todo = range(B) if batches is None else [int(b) for b in batches]
    if vcache is not None:
        vc = np.asarray(vcache)
        if vc.ndim != 4 or vc.shape[1] != PAGE or vc.shape[2] != Hk or vc.shape[3] != dv:
            raise ValueError("vcache must be [pages, 64, h_kv, dv]")
    for b in todo:
        L = int(seqlens[b])
        K = gather_sequence(kv, kv_format, bt[b], L)                        # [L, Hk, 576]
        Vsep = None if vcache is None else gather_values(vc, bt[b], L)      # [L, Hk, dv]
        for kvh in range(Hk):
            Kh = K[:, kvh, :]
            Vh = Kh[:, :dv]
            if Vsep is not None:
                Vh = Vsep[:, kvh, :]
            for s in range(S):
                last = (L - S + s) if causal else (L - 1)
                n_allowed = max(0, min(L, last + 1))
                Qs = bf16_bits_to_f64(q[b, s, kvh * G:(kvh + 1) * G, :])    # [G, 576]
                o, lse = attend(Qs, Kh[:n_allowed], Vh[:n_allowed], scale)
                O[b, s, kvh * G:(kvh + 1) * G, :] = o
                LSE[b, kvh * G:(kvh + 1) * G, s] = lse
    return O, LSE


def mla_decode_sparse(
    q_bits: np.ndarray,
    kvcache: np.ndarray,
    kv_format: str,
    block_table: np.ndarray,
    cache_seqlens: np.ndarray,
    indices: np.ndarray,
    *,
    dv: int = D_V,
    causal: bool = False,
    softmax_scale: Optional[float] = None,
    batches: Optional[Iterable[int]] = None,
) -> Tuple[np.ndarray, np.ndarray]:
    """Token-level sparse decode: query token s of sequence b attends only to the cached
    tokens that indices[b, s, :] names.

    The pages give the call (flash_mla_with_kvcache with is_fp8_kvcache and indices, and
    get_mla_metadata with topk: section "解码阶段使用示例" of the wmrh.cn FlashMLA深度解析 page)
    and name it token-level sparse attention over an FP8 KV cache (section "实际性能表现与优化效果");
    they do not define the indices. Readings taken here:
      * indices int [B, S, topk]: entry j is a token position t of sequence b's cache
        (0 <= t < L_b), found through the block table like any cached token; -1 is padding
        and selects nothing; any other value is an error (ValueError);
      * the selected keys are the listed entries: a position listed twice counts twice
        (the softmax runs over the topk list, not over a set);
      * with causal, keys past L_b - S + s are dropped as in dense decode;
      * no selected key: O = 0, LSE = -inf.
    Returns O float64 [B, S, H, dv] and LSE float64 [B, H, S] (the sequences not in
    `batches` are NaN)."""
    q = np.asarray(q_bits)
    B, S, H, _ = q.shape
    kv = np.asarray(kvcache)
    Hk = kv.shape[2]
    if H % Hk:
        raise ValueError("h_q must be a multiple of h_kv")
    G = H // Hk
    idx = np.asarray(indices).astype(np.int64)
    if idx.ndim != 3 or idx.shape[:2] != (B, S):
        raise ValueError("indices must be [batch, s_q, topk]")
    scale = (1.0 / np.sqrt(D_QK)) if softmax_scale is None else float(softmax_scale)
    seqlens = np.asarray(cache_seqlens).astype(np.int64)
    bt = np.asarray(block_table)
    O = np.full((B, S, H, dv), np.nan)
    LSE = np.full((B, H, S), np.nan)
    todo = range(B) if batches is None else [int(b) for b in batches]
    for b in todo:
        L = int(seqlens[b])
        if L < 0 or L > bt.shape[1] * PAGE:
            raise ValueError(f"sequence length {L} outside [0, {bt.shape[1] * PAGE}]")
        for s in range(S):
            row = idx[b, s]
            sel = row[row != -1]
            if sel.size and (sel.min() < 0 or sel.max() >= L):
                raise ValueError(f"indices[{b}, {s}] names a position outside [0, {L}) (or below -1)")
            if causal:
                sel = sel[sel <= L - S + s]
            pages = bt[b, sel // PAGE].astype(np.int64)
            if sel.size and (pages.min() < 0 or pages.max() >= kv.shape[0]):
                raise ValueError("block_table entry outside the page pool")
            K = decode_kv_rows(kv[pages, sel % PAGE], kv_format)                # [n, Hk, 576]
            for kvh in range(Hk):
                Kh = K[:, kvh, :]
                heads = slice(kvh * G, (kvh + 1) * G)                          # the G heads of KV head kvh
                Qs = bf16_bits_to_f64(q[b, s, heads, :])
                o, lse = attend(Qs, Kh, Kh[:, :dv], scale)
                O[b, s, heads, :] = o
                LSE[b, heads, s] = lse
    return O, LSE


def mla_sparse_prefill(
    q_bits: np.ndarray,
    kv_bits: np.ndarray,
    indices: np.ndarray,
    softmax_scale: float,
    *,
    dv: int = D_V,
    tokens: Optional[Iterable[int]] = None,
) -> Tuple[np.ndarray, np.ndarray]:
    """Sparse prefill: query token s attends, for each KV head, to the keys that
    indices[s, kvh, :] names (flash_mla_sparse_fwd(q [s_q, h_q, d_qk], kv [s_kv, h_kv, d_qk],
    indices [s_q, h_kv, topk], sm_scale, d_v=512): section "稀疏预填充使用" of the wmrh.cn
    FlashMLA深度解析 page). The page gives only the arguments. Readings taken here: kv rows are
    bf16 and contiguous (no pages); an entry is a row of kv in [0, s_kv), -1 is padding, any
    other value is an error (ValueError); listed entries count as listed; query head h reads KV
    head h // (h_q / h_kv); V is the first dv dims of each row; no key: O = 0, LSE = -inf; the
    call returns O [s_q, h_q, dv] and the natural-log LSE [s_q, h_q].
    Returns float64 arrays; with `tokens`, only those query tokens, in that order
    (O [len(tokens), h_q, dv], LSE [len(tokens), h_q])."""
    q = np.asarray(q_bits)
    kv = np.asarray(kv_bits)
    if q.ndim != 3 or q.shape[-1] != D_QK or kv.ndim != 3 or kv.shape[-1] != D_QK:
        raise ValueError("q must be [s_q, h_q, 576] and kv [s_kv, h_kv, 576]")
    Sq, H, _ = q.shape
    Skv, Hk, _ = kv.shape
    if H % Hk:
        raise ValueError("h_q must be a multiple of h_kv")
    G = H // Hk
    idx = np.asarray(indices)
    if idx.ndim != 3 or idx.shape[:2] != (Sq, Hk):
        raise ValueError("indices must be [s_q, h_kv, topk]")
    todo = list(range(Sq)) if tokens is None else [int(t) for t in tokens]
    O = np.full((len(todo), H, dv), np.nan)
    LSE = np.full((len(todo), H), np.nan)
    for i, s in enumerate(todo):
        for kvh in range(Hk):
            row = idx[s, kvh].astype(np.int64)
            keep = row != -1                                                    # -1: padding
            sel = row[keep]
            if sel.size and (sel.min() < 0 or sel.max() >= Skv):
                raise ValueError(f"indices[{s}, {kvh}] names a row outside [0, {Skv}) (or below -1)")
            K = bf16_bits_to_f64(kv[sel, kvh, :])                               # [n, 576]
            heads = slice(kvh * G, (kvh + 1) * G)
            o, lse = attend(bf16_bits_to_f64(q[s, heads, :]), K, K[:, :dv], float(softmax_scale))
            O[i, heads, :] = o
            LSE[i, heads] = lse
    return O, LSE


def mla_decode_workload(w, batches: Optional[Iterable[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """mla_decode (mla_decode_sparse when it carries indices) on an object with the fields of
    workloads.Workload."""
    a = w.as_numpy()
    if getattr(w, "indices", None) is not None:
        return mla_decode_sparse(a["q_bits"], a["kvcache"], w.kv_format, a["block_table"], a["cache_seqlens"],
                                 w.indices.numpy(), dv=w.dv, causal=w.causal, softmax_scale=w.softmax_scale,
                                 batches=batches)
    return mla_decode(a["q_bits"], a["kvcache"], w.kv_format, a["block_table"], a["cache_seqlens"],
                      dv=w.dv, causal=w.causal, softmax_scale=w.softmax_scale, batches=batches,
                      vcache=a.get("vcache"))
