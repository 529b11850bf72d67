"""Paged MLA decode for MI355X (gfx950): thin Python binding over libmla.so.

Two calls, named after the C ABI in include/mla.h:

    tile_metadata, num_splits = mla_get_metadata(cache_seqlens, s_q * h_q // h_kv, h_kv)
    o, lse = mla_decode_kvcache(q, kvcache, block_table, cache_seqlens, dv,
                                tile_metadata, num_splits, causal=True)

(the call pattern of FlashMLA's get_mla_metadata / flash_mla_with_kvcache:
"功能 1" on the kdjingpai.com post). PyTorch supplies device memory and the
current stream; every step of the computation runs in the HIP library. If the
library is not built, importing the calls raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import D_QK, D_V, FP8_RECORD_BYTES, META_INTS, PAGE_TOKENS, MlaDecodeArgs, MlaError, MlaSparsePrefillArgs

__all__ = [
    "mla_get_metadata", "mla_get_metadata_device", "mla_get_metadata_sparse", "mla_decode_kvcache",
    "mla_workspace_bytes", "mla_num_parts", "MlaDecoder", "MlaSparsePrefill", "flash_mla_sparse_fwd",
    "MlaError", "kv_format_of", "library_path",
]

_FORMATS = {"bf16": _lib.MLA_KV_BF16, "fp8": _lib.MLA_KV_FP8_E4M3}


def library_path() -> str:
    return _lib.LIB_PATH


def _fmt_code(kv_format) -> int:
    if isinstance(kv_format, int):
        return kv_format
    try:
        return _FORMATS[kv_format]
    except KeyError:
        raise ValueError(f"kv_format must be 'bf16' or 'fp8', got {kv_format!r}") from None


def kv_format_of(kvcache: torch.Tensor) -> str:
    if kvcache.dtype == torch.bfloat16 and kvcache.shape[-1] == D_QK:
        return "bf16"
    if kvcache.dtype == torch.uint8 and kvcache.shape[-1] == FP8_RECORD_BYTES:
        return "fp8"
    raise ValueError(f"kvcache must be bf16 [..., {D_QK}] or uint8 FP8 records [..., {FP8_RECORD_BYTES}], "
                     f"got {kvcache.dtype} {tuple(kvcache.shape)}")


def mla_num_parts(batch: int, heads_per_kv: int, h_kv: int = 1, kv_format="bf16", num_cus: int = 0) -> int:
    lib = _lib.load()
    n = lib.mla_num_parts(int(batch), int(heads_per_kv), int(h_kv), _fmt_code(kv_format), int(num_cus))
    if n < 0:
        raise ValueError(_lib.last_error())
    return n


def mla_workspace_bytes(batch: int, num_parts: int, heads_per_kv: int, h_kv: int = 1) -> int:
    return int(_lib.load().mla_workspace_bytes(int(batch), int(num_parts), int(heads_per_kv), int(h_kv)))


def _i32p(t: torch.Tensor):
    return ctypes.cast(ctypes.c_void_p(t.data_ptr()), ctypes.POINTER(ctypes.c_int32))


def mla_get_metadata_host(cache_seqlens_host: torch.Tensor, heads_per_kv: int, h_kv: int = 1, *,
                          kv_format="bf16", max_blocks_per_seq: int = 0, num_parts: int = 0, num_cus: int = 0,
                          pin: bool = False, out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Host tile scheduler: int32 CPU tensors (tile_metadata [P, 8], num_splits [B + 1]).

    `max_blocks_per_seq` (the block table's width; 0 = unchecked): a length above 64 times it
    raises ValueError. `out` (optional): a contiguous int32 CPU tensor of P * 8 + B + 1 elements
    (pinned, say) that receives [tile_metadata | num_splits]; the returned tensors are views of
    it. The caller must not overwrite a buffer whose previous contents are still being copied to
    the device."""
    lib = _lib.load()
    L = cache_seqlens_host
    if L.device.type != "cpu":
        L = L.cpu()
    L = L.to(torch.int32).contiguous()
    if L.dim() != 1:
        raise ValueError("cache_seqlens must be 1-D [batch]")
    B = int(L.shape[0])
    fmt = _fmt_code(kv_format)
    parts = int(num_parts)
    if parts == 0:
        parts = lib.mla_num_parts(B, int(heads_per_kv), int(h_kv), fmt, int(num_cus))
        if parts < 0:
            raise ValueError(_lib.last_error())
    # one buffer [tile_metadata (parts x 8) | num_splits (B + 1)]: a single upload
    n = parts * META_INTS + B + 1
    if out is not None:
        if (out.device.type != "cpu" or out.dtype != torch.int32 or not out.is_contiguous()
                or out.dim() != 1 or int(out.shape[0]) != n):
            raise ValueError(f"out must be a contiguous 1-D int32 CPU tensor of {n} elements")
        flat = out
    else:
        flat = torch.empty((n,), dtype=torch.int32, pin_memory=pin)
    meta = flat[:parts * META_INTS].view(parts, META_INTS)
    splits = flat[parts * META_INTS:]
    got = ctypes.c_int(0)
    _lib.check(lib.mla_get_metadata(_i32p(L), B, int(heads_per_kv), int(h_kv), fmt, int(max_blocks_per_seq),
                                    int(num_cus), parts, _i32p(meta), _i32p(splits), ctypes.byref(got)))
    return meta, splits


def split_metadata(flat: torch.Tensor, batch: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Views (tile_metadata [P, 8], num_splits [batch + 1]) of one packed int32 buffer
    laid out as mla_get_metadata_host leaves it (metadata rows, then num_splits)."""
    n = int(flat.shape[0]) - (batch + 1)
    if n <= 0 or n % META_INTS:
        raise ValueError("packed metadata buffer has the wrong length for this batch")
    return flat[:n].view(n // META_INTS, META_INTS), flat[n:]


def packed_metadata(meta: torch.Tensor) -> torch.Tensor:
    """The packed buffer behind a (tile_metadata, num_splits) pair from mla_get_metadata_host."""
    base = meta._base if meta._base is not None else meta
    return base


def mla_get_metadata(cache_seqlens: torch.Tensor, heads_per_kv: int, h_kv: int = 1, *, kv_format="bf16",
                     max_blocks_per_seq: int = 0, num_parts: int = 0, num_cus: int = 0,
                     device: Optional[torch.device] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Tile-scheduler metadata for one decode step, on `device` (default: the device of
    cache_seqlens, or the current CUDA device for a CPU tensor). Reuse it for every layer.
    A device-resident cache_seqlens is read back to the host (a synchronising copy).
    `max_blocks_per_seq`: the block table's width, to reject lengths it cannot hold (0: the
    decode reports such a sequence as NaN instead)."""
    if device is None:
        device = cache_seqlens.device if cache_seqlens.device.type != "cpu" else torch.device("cuda")
    pin = torch.device(device).type == "cuda"
    meta, splits = mla_get_metadata_host(cache_seqlens, heads_per_kv, h_kv, kv_format=kv_format,
                                         max_blocks_per_seq=max_blocks_per_seq, num_parts=num_parts,
                                         num_cus=num_cus, pin=pin)
    flat_d = packed_metadata(meta).to(device, non_blocking=True)
    meta_d, splits_d = split_metadata(flat_d, int(splits.shape[0]) - 1)
    # host-side fact carried along for the decode call's combine-shape hint
    splits_d._mla_max_splits = max_splits_of(splits)
    return meta_d, splits_d


def mla_get_metadata_device(cache_seqlens: torch.Tensor, heads_per_kv: int, h_kv: int = 1, *, kv_format="bf16",
                            num_parts: int = 0, num_cus: int = 0, out: Optional[torch.Tensor] = None,
                            stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The tile scheduler on the device: (tile_metadata [P, 8], num_splits [B + 1]) computed by one
    kernel from device-resident int32 cache_seqlens, queued on `stream` (default: the current one);
    nothing is copied to the host. Equal, bit for bit, to mla_get_metadata for the same lengths.
    `out`: optional contiguous int32 device tensor of P * 8 + B + 1 elements that receives
    [tile_metadata | num_splits] (the returned tensors are views of it)."""
    L = cache_seqlens
    if L.device.type != "cuda" or L.dtype != torch.int32 or L.dim() != 1 or not L.is_contiguous():
        raise ValueError("cache_seqlens must be a contiguous 1-D int32 device tensor")
    lib = _lib.load()
    B = int(L.shape[0])
    fmt = _fmt_code(kv_format)
    parts = int(num_parts)
    if parts == 0:
        parts = lib.mla_num_parts(B, int(heads_per_kv), int(h_kv), fmt, int(num_cus))
        if parts < 0:
            raise ValueError(_lib.last_error())
    n = parts * META_INTS + B + 1
    if out is None:
        out = torch.empty((n,), dtype=torch.int32, device=L.device)
    elif (out.device != L.device or out.dtype != torch.int32 or not out.is_contiguous() or out.dim() != 1
          or int(out.shape[0]) != n):
        raise ValueError(f"out must be a contiguous 1-D int32 tensor of {n} elements on {L.device}")
    meta, splits = split_metadata(out, B)
    s = torch.cuda.current_stream(L.device) if stream is None else stream
    got = ctypes.c_int(0)
    _lib.check(lib.mla_get_metadata_device(ctypes.c_void_p(L.data_ptr()), B, int(heads_per_kv), int(h_kv), fmt,
                                           int(num_cus), parts, ctypes.c_void_p(meta.data_ptr()),
                                           ctypes.c_void_p(splits.data_ptr()), ctypes.byref(got),
                                           ctypes.c_void_p(s.cuda_stream)))
    return meta, splits


def mla_get_metadata_sparse(batch: int, s_q: int, topk: int, h_q: int, h_kv: int = 1, *, kv_format="bf16",
                            num_parts: int = 0, num_cus: int = 0, device: Optional[torch.device] = None,
                            host: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """Tile-scheduler metadata for token-level sparse decode (every (sequence, query token)
    pair scheduled as a sequence of topk entries): (tile_metadata [P, 8], num_splits
    [batch * s_q + 1]) on `device` (default: the current CUDA device), or int32 CPU tensors
    with host=True."""
    lib = _lib.load()
    fmt = _fmt_code(kv_format)
    parts = int(num_parts)
    vb = int(batch) * int(s_q)
    if parts == 0:
        parts = lib.mla_num_parts(vb, max(int(h_q) // max(int(h_kv), 1), 1), int(h_kv), fmt, int(num_cus))
        if parts < 0:
            raise ValueError(_lib.last_error())
    flat = torch.empty((parts * META_INTS + vb + 1,), dtype=torch.int32, pin_memory=not host)
    meta, splits = split_metadata(flat, vb)
    got = ctypes.c_int(0)
    _lib.check(lib.mla_get_metadata_sparse(int(batch), int(s_q), int(topk), int(h_q), int(h_kv), fmt, int(num_cus),
                                           parts, _i32p(meta), _i32p(splits), ctypes.byref(got)))
    if host:
        return meta, splits
    flat_d = flat.to(torch.device("cuda") if device is None else device, non_blocking=True)
    meta_d, splits_d = split_metadata(flat_d, vb)
    splits_d._mla_max_splits = max_splits_of(splits)
    return meta_d, splits_d


def max_splits_of(num_splits_host: torch.Tensor) -> int:
    """Largest number of pieces of any sequence, from host num_splits [batch + 1]."""
    d = num_splits_host[1:] - num_splits_host[:-1]
    return int(d.max()) if d.numel() else 0


def _check_tensor(name, t, dtype, ndim, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


class MlaDecoder:
    """A decode call with its argument block marshalled once.

    Holds references to every tensor it points at; `run()` launches on the
    current (or given) stream. Use it when the same buffers are decoded
    repeatedly (one per layer of a decode step, or a benchmark loop)."""

    def __init__(self, q, kvcache, block_table, cache_seqlens, dv, tile_metadata, num_splits, causal=False,
                 softmax_scale=None, *, out=None, lse=None, workspace=None, events=None, max_splits=None,
                 no_alloc=False, indices=None, vcache=None):
        dev = q.device
        if dev.type != "cuda":
            raise ValueError("q must be a CUDA (HIP) tensor")
        fmt = kv_format_of(kvcache)
        _check_tensor("q", q, torch.bfloat16, 4, dev)
        _check_tensor("kvcache", kvcache, kvcache.dtype, 4, dev)
        _check_tensor("block_table", block_table, torch.int32, 2, dev)
        _check_tensor("cache_seqlens", cache_seqlens, torch.int32, 1, dev)
        _check_tensor("tile_metadata", tile_metadata, torch.int32, 2, dev)
        _check_tensor("num_splits", num_splits, torch.int32, 1, dev)
        if q.stride(-1) != 1 or kvcache.stride(-1) != 1 or block_table.stride(-1) != 1:
            raise ValueError("q, kvcache and block_table need a contiguous last dimension")
        if not (cache_seqlens.is_contiguous() and tile_metadata.is_contiguous() and num_splits.is_contiguous()):
            raise ValueError("cache_seqlens, tile_metadata and num_splits must be contiguous")
        if tile_metadata.shape[1] != META_INTS:
            raise ValueError(f"tile_metadata must be [num_parts, {META_INTS}]")
        B, S, H, D = q.shape
        Hk = int(kvcache.shape[2])
        if kvcache.shape[1] != PAGE_TOKENS:
            raise ValueError(f"kvcache pages must hold {PAGE_TOKENS} tokens")
        nseq = B * S if indices is not None else B
        if num_splits.shape[0] != nseq + 1 or cache_seqlens.shape[0] != B or block_table.shape[0] != B:
            raise ValueError("cache_seqlens [batch], block_table [batch, n] and num_splits [batch + 1] (sparse: "
                             "[batch * s_q + 1]) must agree with q")
        if indices is not None:
            _check_tensor("indices", indices, torch.int32, 3, dev)
            if tuple(indices.shape[:2]) != (B, S) or indices.shape[2] < 1 or indices.stride(-1) != 1:
                raise ValueError("indices must be int32 [batch, s_q, topk] with a contiguous last dimension")
        if vcache is not None:
            _check_tensor("vcache", vcache, torch.bfloat16, 4, dev)
            if (tuple(vcache.shape) != (int(kvcache.shape[0]), PAGE_TOKENS, Hk, int(dv))
                    or vcache.stride(-1) != 1):
                raise ValueError("vcache must be bf16 [num_pages, 64, h_kv, dv] with a contiguous last dimension")
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(D)
        rows = S * H // max(Hk, 1)
        parts = int(tile_metadata.shape[0])
        if out is None:
            out = torch.empty((B, S, H, int(dv)), dtype=torch.bfloat16, device=dev)
        if lse is None:
            lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
        _check_tensor("out", out, torch.bfloat16, 4, dev)
        _check_tensor("lse", lse, torch.float32, 3, dev)
        if not (out.is_contiguous() and lse.is_contiguous()):
            raise ValueError("out and lse must be contiguous")
        if tuple(out.shape) != (B, S, H, int(dv)) or tuple(lse.shape) != (B, H, S):
            raise ValueError("out must be [batch, s_q, h_q, dv] and lse [batch, h_q, s_q]")
        if H % max(Hk, 1) != 0:
            need = 0
        elif indices is not None:
            need = int(_lib.load().mla_workspace_bytes_sparse(B, S, parts, H, Hk))
        else:
            need = mla_workspace_bytes(B, parts, rows, Hk)
        if workspace is None and not no_alloc:
            workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
        self.tensors = (q, kvcache, block_table, cache_seqlens, tile_metadata, num_splits, out, lse, workspace,
                        indices, vcache)
        self.out, self.lse, self.workspace = out, lse, workspace
        a = MlaDecodeArgs()
        a.q = q.data_ptr()
        a.q_stride[:] = [q.stride(0), q.stride(1), q.stride(2)]
        a.kvcache = kvcache.data_ptr()
        a.kv_stride[:] = [kvcache.stride(0), kvcache.stride(1), kvcache.stride(2)]
        a.kv_format = _FORMATS[fmt]
        a.num_pages = int(kvcache.shape[0])
        a.block_table = block_table.data_ptr()
        a.bt_stride = block_table.stride(0)
        a.max_blocks_per_seq = int(block_table.shape[1])
        a.cache_seqlens = cache_seqlens.data_ptr()
        a.tile_metadata = tile_metadata.data_ptr()
        a.num_parts = parts
        a.num_splits = num_splits.data_ptr()
        a.batch, a.s_q, a.h_q, a.h_kv = B, S, H, Hk
        a.d_qk, a.dv = int(D), int(dv)
        a.causal = 1 if causal else 0
        a.softmax_scale = float(softmax_scale)
        a.o = out.data_ptr()
        a.lse = lse.data_ptr()
        a.workspace = workspace.data_ptr() if workspace is not None else None
        a.workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        if max_splits is None:
            max_splits = getattr(num_splits, "_mla_max_splits", 0)
        a.max_splits = int(max_splits)
        if indices is not None:
            a.indices = indices.data_ptr()
            a.idx_stride[:] = [indices.stride(0), indices.stride(1)]
            a.topk = int(indices.shape[2])
        if vcache is not None:
            a.vcache = vcache.data_ptr()
            a.vc_stride[:] = [vcache.stride(0), vcache.stride(1), vcache.stride(2)]
        self.args = a
        if events is not None:
            self.set_events(events)
        self._args_ref = ctypes.byref(a)
        self._lib = _lib.load()
        # no_alloc: the library's static scratch replaces the workspace (mla_decode_kvcache_noalloc)
        self._entry = self._lib.mla_decode_kvcache_noalloc if no_alloc else self._lib.mla_decode_kvcache
        self.device = dev

    def set_events(self, events: Sequence) -> None:
        """Timing hooks: three raw hipEvent_t handles (ints) or None."""
        for i in range(3):
            e = events[i] if i < len(events) else None
            self.args.events[i] = None if e is None else int(e)

    def run(self, stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor]:
        s = torch.cuda.current_stream(self.device) if stream is None else stream
        _lib.check(self._entry(self._args_ref, ctypes.c_void_p(s.cuda_stream)))
        return self.out, self.lse


def mla_decode_kvcache(q: torch.Tensor, kvcache: torch.Tensor, block_table: torch.Tensor, cache_seqlens: torch.Tensor,
                       dv: int, tile_metadata: torch.Tensor, num_splits: torch.Tensor, causal: bool = False,
                       softmax_scale: Optional[float] = None, *, out=None, lse=None, workspace=None,
                       indices: Optional[torch.Tensor] = None,
                       vcache: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """o [batch, s_q, h_q, dv] bf16 and lse [batch, h_q, s_q] fp32 for one layer.

    q bf16 [batch, s_q, h_q, 576]; kvcache bf16 [pages, 64, h_kv, 576] or uint8
    FP8 records [pages, 64, h_kv, 656]; block_table int32 [batch, max_blocks];
    cache_seqlens int32 [batch]; tile_metadata / num_splits from mla_get_metadata
    for these lengths. causal: query token s of s_q reads keys t <= L - s_q + s.
    softmax_scale defaults to 1/sqrt(576). indices (optional, int32 [batch, s_q, topk]):
    token-level sparse decode -- query token s of sequence b attends only to the listed cached
    positions of b (-1: padding); its metadata comes from mla_get_metadata_sparse. vcache
    (optional, bf16 [pages, 64, h_kv, dv]): V rows from here, at the keys' pages and slots,
    instead of the first dv dims of the keys (bf16 keys, dense decode)."""
    dec = MlaDecoder(q, kvcache, block_table, cache_seqlens, dv, tile_metadata, num_splits, causal, softmax_scale,
                     out=out, lse=lse, workspace=workspace, indices=indices, vcache=vcache)
    return dec.run()


class MlaSparsePrefill:
    """A sparse prefill call (mla_sparse_prefill_fwd) with its argument block marshalled once.

    q bf16 [s_q, h_q, 576]; kv bf16 [s_kv, h_kv, 576]; indices int32 [s_q, h_kv, topk] (rows
    of kv, -1: padding). tile_metadata / num_splits default to mla_get_metadata_sparse(s_q, 1,
    topk, h_q, h_kv) on q's device. `run()` launches on the current (or given) stream and
    returns (o [s_q, h_q, dv] bf16, lse [s_q, h_q] fp32, natural log)."""

    def __init__(self, q, kv, indices, sm_scale=None, d_v=D_V, *, tile_metadata=None, num_splits=None, out=None,
                 lse=None, workspace=None, events=None, max_splits=None, num_parts: int = 0):
        dev = q.device
        if dev.type != "cuda":
            raise ValueError("q must be a CUDA (HIP) tensor")
        _check_tensor("q", q, torch.bfloat16, 3, dev)
        _check_tensor("kv", kv, torch.bfloat16, 3, dev)
        _check_tensor("indices", indices, torch.int32, 3, dev)
        if q.stride(-1) != 1 or kv.stride(-1) != 1 or indices.stride(-1) != 1:
            raise ValueError("q, kv and indices need a contiguous last dimension")
        Sq, H, D = q.shape
        Skv, Hk = int(kv.shape[0]), int(kv.shape[1])
        if tuple(indices.shape[:2]) != (Sq, Hk) or indices.shape[2] < 1:
            raise ValueError("indices must be int32 [s_q, h_kv, topk]")
        topk = int(indices.shape[2])
        if tile_metadata is None or num_splits is None:
            tile_metadata, num_splits = mla_get_metadata_sparse(Sq, 1, topk, H, Hk, num_parts=num_parts, device=dev)
        _check_tensor("tile_metadata", tile_metadata, torch.int32, 2, dev)
        _check_tensor("num_splits", num_splits, torch.int32, 1, dev)
        if not (tile_metadata.is_contiguous() and num_splits.is_contiguous()) or tile_metadata.shape[1] != META_INTS:
            raise ValueError(f"tile_metadata must be contiguous [num_parts, {META_INTS}] and num_splits contiguous")
        if num_splits.shape[0] != Sq + 1:
            raise ValueError("num_splits must be [s_q + 1]")
        if sm_scale is None:
            sm_scale = 1.0 / math.sqrt(D)
        parts = int(tile_metadata.shape[0])
        if out is None:
            out = torch.empty((Sq, H, int(d_v)), dtype=torch.bfloat16, device=dev)
        if lse is None:
            lse = torch.empty((Sq, H), dtype=torch.float32, device=dev)
        _check_tensor("out", out, torch.bfloat16, 3, dev)
        _check_tensor("lse", lse, torch.float32, 2, dev)
        if not (out.is_contiguous() and lse.is_contiguous()):
            raise ValueError("out and lse must be contiguous")
        if tuple(out.shape) != (Sq, H, int(d_v)) or tuple(lse.shape) != (Sq, H):
            raise ValueError("out must be [s_q, h_q, d_v] and lse [s_q, h_q]")
        lib = _lib.load()
        need = int(lib.mla_workspace_bytes_sparse(Sq, 1, parts, H, Hk)) if H % max(Hk, 1) == 0 else 0
        if workspace is None:
            workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
        self.tensors = (q, kv, indices, tile_metadata, num_splits, out, lse, workspace)
        self.out, self.lse, self.workspace = out, lse, workspace
        a = MlaSparsePrefillArgs()
        a.q = q.data_ptr()
        a.q_stride[:] = [q.stride(0), q.stride(1)]
        a.kv = kv.data_ptr()
        a.kv_stride[:] = [kv.stride(0), kv.stride(1)]
        a.indices = indices.data_ptr()
        a.idx_stride[:] = [indices.stride(0), indices.stride(1)]
        a.s_q, a.s_kv, a.h_q, a.h_kv, a.topk = int(Sq), Skv, int(H), Hk, topk
        a.d_qk, a.dv = int(D), int(d_v)
        a.softmax_scale = float(sm_scale)
        a.tile_metadata = tile_metadata.data_ptr()
        a.num_parts = parts
        a.num_splits = num_splits.data_ptr()
        a.o = out.data_ptr()
        a.lse = lse.data_ptr()
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
        if max_splits is None:
            max_splits = getattr(num_splits, "_mla_max_splits", 0)
        a.max_splits = int(max_splits)
        self.args = a
        if events is not None:
            self.set_events(events)
        self._args_ref = ctypes.byref(a)
        self._lib = lib
        self.device = dev

    def set_events(self, events: Sequence) -> None:
        """Timing hooks: three raw hipEvent_t handles (ints) or None."""
        for i in range(3):
            e = events[i] if i < len(events) else None
            self.args.events[i] = None if e is None else int(e)

    def run(self, stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor]:
        s = torch.cuda.current_stream(self.device) if stream is None else stream
        _lib.check(self._lib.mla_sparse_prefill_fwd(self._args_ref, ctypes.c_void_p(s.cuda_stream)))
        return self.out, self.lse


def flash_mla_sparse_fwd(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor, sm_scale: Optional[float] = None,
                         d_v: int = D_V, **kw) -> Tuple[torch.Tensor, torch.Tensor]:
    """Sparse prefill: (o [s_q, h_q, d_v] bf16, lse [s_q, h_q] fp32). Query token s, head h
    attends to the rows indices[s, h // (h_q // h_kv), :] of kv's KV head h // (h_q // h_kv)
    (-1: padding). Keyword arguments go to MlaSparsePrefill (metadata, out, lse, workspace)."""
    return MlaSparsePrefill(q, kv, indices, sm_scale, d_v, **kw).run()
