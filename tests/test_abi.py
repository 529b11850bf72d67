"""The C ABI on the CPU: the library loads, exports what include/mla.h declares,
and rejects bad arguments before anything is launched (no GPU call is reached)."""
import ctypes
import os
import re

import pytest

from paged_mla_decode_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "mla.h"), encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    lib = _lib.load()
    declared = _declared_functions()
    assert "mla_get_metadata" in declared and "mla_decode_kvcache" in declared
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in include/mla.h but not exported"
    assert set(_lib.EXPORTED_SYMBOLS) == set(declared)


def test_args_struct_layout_matches():
    lib = _lib.load()
    assert lib.mla_decode_args_size() == ctypes.sizeof(_lib.MlaDecodeArgs)
    assert b"gfx950" in lib.mla_version()


def _meta(L, M=16, hkv=1, fmt=0, cus=256, parts=0, maxb=0):
    lib = _lib.load()
    B = len(L)
    Ls = (ctypes.c_int32 * B)(*L)
    if parts == 0:
        parts = lib.mla_num_parts(B, M, hkv, fmt, cus)
        assert parts >= 1
    meta = (ctypes.c_int32 * (parts * 8))()
    splits = (ctypes.c_int32 * (B + 1))()
    got = ctypes.c_int(0)
    st = lib.mla_get_metadata(Ls, B, M, hkv, fmt, maxb, cus, parts, meta, splits, ctypes.byref(got))
    return st, [list(meta[p * 8:(p + 1) * 8]) for p in range(parts)], list(splits), got.value


def test_get_metadata_rejects_bad_arguments():
    lib = _lib.load()
    st, *_ = _meta([10, -1])
    assert st == _lib.MLA_ERR_INVALID_ARGUMENT and b"negative" in lib.mla_last_error()
    st, *_ = _meta([10], M=0, parts=4)
    assert st == _lib.MLA_ERR_INVALID_ARGUMENT
    st, *_ = _meta([10], fmt=7, parts=4)
    assert st == _lib.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_num_parts(0, 16, 1, 0, 256) == -1
    assert lib.mla_workspace_bytes(0, 4, 16, 1) == 0


def test_python_metadata_rejects_lengths_beyond_the_block_table():
    import torch
    import paged_mla_decode_amd as mla
    L = torch.tensor([100, 200], dtype=torch.int32)
    mla.mla_get_metadata_host(L, 16, 1, num_cus=256, max_blocks_per_seq=4)
    with pytest.raises(ValueError, match="exceeds the block table"):
        mla.mla_get_metadata_host(L, 16, 1, num_cus=256, max_blocks_per_seq=3)


def test_decode_rejects_huge_block_table_width():
    lib = _lib.load()
    a = _valid_args()
    a.max_blocks_per_seq = (1 << 25) + 1
    a.bt_stride = a.max_blocks_per_seq
    assert lib.mla_decode_kvcache(ctypes.byref(a), None) == _lib.MLA_ERR_UNSUPPORTED


def test_workspace_bytes():
    lib = _lib.load()
    B, P, M = 64, 256, 128
    n = lib.mla_workspace_bytes(B, P, M, 1)
    slots = B + P
    assert n >= slots * M * 512 * 2 + slots * M * 8 * 4 + slots * M * 4   # fp16 O, 8 block scales, LSE
    assert n % 256 == 0
    n16 = lib.mla_workspace_bytes(B, P, 16, 1)                               # up to 64 rows: fp32 O
    assert n16 >= slots * 16 * 512 * 4 + slots * 16 * 4 and n16 % 256 == 0


def _valid_args():
    a = _lib.MlaDecodeArgs()
    fake = 1 << 20          # never dereferenced: every case below fails validation first
    a.q = fake
    a.q_stride[:] = [16 * 576, 16 * 576, 576]
    a.kvcache = fake
    a.kv_stride[:] = [64 * 576, 576, 576]
    a.kv_format = 0
    a.num_pages = 4
    a.block_table = fake
    a.bt_stride = 2
    a.max_blocks_per_seq = 2
    a.cache_seqlens = fake
    a.tile_metadata = fake
    a.num_parts = 4
    a.num_splits = fake
    a.batch, a.s_q, a.h_q, a.h_kv = 2, 1, 16, 1
    a.d_qk, a.dv = 576, 512
    a.causal = 0
    a.softmax_scale = 1 / 24
    a.o = fake
    a.lse = fake
    a.workspace = fake
    a.workspace_bytes = _lib.load().mla_workspace_bytes(2, 4, 16, 1)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("d_qk", 512, _lib.MLA_ERR_UNSUPPORTED),
    ("dv", 576, _lib.MLA_ERR_UNSUPPORTED),
    ("h_kv", 3, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("s_q", 0, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("batch", 0, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("kv_format", 5, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("num_pages", 0, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("max_blocks_per_seq", 0, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("bt_stride", 1, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("num_parts", 0, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("workspace_bytes", 16, _lib.MLA_ERR_WORKSPACE_TOO_SMALL),
    ("workspace", None, _lib.MLA_ERR_WORKSPACE_TOO_SMALL),
    ("q", None, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("q", (1 << 20) + 2, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("kvcache", (1 << 20) + 8, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("o", None, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("softmax_scale", float("nan"), _lib.MLA_ERR_INVALID_ARGUMENT),
])
def test_decode_rejects_bad_arguments(field, value, status):
    lib = _lib.load()
    a = _valid_args()
    setattr(a, field, value)
    assert lib.mla_decode_kvcache(ctypes.byref(a), None) == status
    assert lib.mla_last_error() != b""


@pytest.mark.parametrize("which,value", [("q_stride", 7), ("kv_stride", 4)])
def test_decode_rejects_bad_strides(which, value):
    lib = _lib.load()
    a = _valid_args()
    getattr(a, which)[1] = value
    assert lib.mla_decode_kvcache(ctypes.byref(a), None) == _lib.MLA_ERR_INVALID_ARGUMENT


def test_decode_rejects_null_args():
    lib = _lib.load()
    assert lib.mla_decode_kvcache(None, None) == _lib.MLA_ERR_INVALID_ARGUMENT


def test_python_binding_refuses_cpu_tensors():
    import torch
    import paged_mla_decode_amd as mla
    q = torch.zeros(1, 1, 16, 576, dtype=torch.bfloat16)
    kv = torch.zeros(1, 64, 1, 576, dtype=torch.bfloat16)
    bt = torch.zeros(1, 1, dtype=torch.int32)
    L = torch.ones(1, dtype=torch.int32)
    meta, splits = mla.mla_get_metadata_host(L, 16, 1, num_cus=256)
    with pytest.raises(ValueError):
        mla.mla_decode_kvcache(q, kv, bt, L, 512, meta, splits)


def test_packed_metadata_round_trip():
    import torch
    import paged_mla_decode_amd as mla
    L = torch.tensor([0, 5, 700, 64, 3000], dtype=torch.int32)
    meta, splits = mla.mla_get_metadata_host(L, 128, 1, num_cus=256, num_parts=9)
    flat = mla.packed_metadata(meta)
    assert flat.shape == (9 * 8 + 6,)
    m2, s2 = mla.split_metadata(flat, 5)
    assert torch.equal(m2, meta) and torch.equal(s2, splits)
    assert m2.data_ptr() == meta.data_ptr() and s2.data_ptr() == splits.data_ptr()
    with pytest.raises(ValueError):
        mla.split_metadata(flat, 6)


def test_metadata_into_caller_buffer():
    import torch
    import paged_mla_decode_amd as mla
    L = torch.tensor([0, 5, 700, 64, 3000], dtype=torch.int32)
    meta, splits = mla.mla_get_metadata_host(L, 16, 1, num_cus=256, num_parts=7)
    buf = torch.full((7 * 8 + 6,), -123, dtype=torch.int32)
    m2, s2 = mla.mla_get_metadata_host(L, 16, 1, num_cus=256, num_parts=7, out=buf)
    assert torch.equal(m2, meta) and torch.equal(s2, splits)
    assert m2.data_ptr() == buf.data_ptr()
    with pytest.raises(ValueError):
        mla.mla_get_metadata_host(L, 16, 1, num_cus=256, num_parts=7, out=torch.empty(10, dtype=torch.int32))


def test_noalloc_entry_validates_before_launch():
    # the same argument checks as mla_decode_kvcache; the workspace fields are ignored
    lib = _lib.load()
    a = _valid_args()
    a.d_qk = 512
    assert lib.mla_decode_kvcache_noalloc(ctypes.byref(a), None) == _lib.MLA_ERR_UNSUPPORTED
    a = _valid_args()
    a.h_kv = 3
    assert lib.mla_decode_kvcache_noalloc(ctypes.byref(a), None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_decode_kvcache_noalloc(None, None) == _lib.MLA_ERR_INVALID_ARGUMENT


def test_noalloc_entry_rejects_work_beyond_the_scratch():
    lib = _lib.load()
    a = _valid_args()
    a.workspace = None
    a.workspace_bytes = 0
    # 1024 sequences x 1024 ranges of 128 rows: far more partials than the static scratch holds
    a.batch, a.h_q, a.num_parts = 1024, 128, 1024
    a.q_stride[:] = [128 * 576, 128 * 576, 576]
    need = lib.mla_workspace_bytes(1024, 1024, 128, 1)
    assert need > _lib.SCRATCH_BYTES
    assert lib.mla_decode_kvcache_noalloc(ctypes.byref(a), None) == _lib.MLA_ERR_WORKSPACE_TOO_SMALL
    assert b"static scratch holds" in lib.mla_last_error()


def test_device_scheduler_checks_before_launch():
    lib = _lib.load()
    fake = ctypes.c_void_p(1 << 20)     # never dereferenced: every case fails before a launch
    args = lambda B, parts: (fake, B, 16, 1, 0, 256, parts, fake, fake, None, None)
    assert lib.mla_get_metadata_device(None, 4, 16, 1, 0, 256, 4, fake, fake, None, None) == \
        _lib.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_get_metadata_device(*args(1024, 4)) == _lib.MLA_ERR_UNSUPPORTED
    assert b"batch <= 1023" in lib.mla_last_error()
    assert lib.mla_get_metadata_device(*args(8, 1025)) == _lib.MLA_ERR_UNSUPPORTED
    assert lib.mla_get_metadata_device(fake, 4, 16, 1, 9, 256, 4, fake, fake, None, None) == \
        _lib.MLA_ERR_INVALID_ARGUMENT


def test_prefill_args_struct_layout_matches():
    assert _lib.load().mla_sparse_prefill_args_size() == ctypes.sizeof(_lib.MlaSparsePrefillArgs)


def _valid_prefill_args():
    a = _lib.MlaSparsePrefillArgs()
    fake = 1 << 20          # never dereferenced: every case below fails validation first
    a.q = fake
    a.q_stride[:] = [128 * 576, 576]
    a.kv = fake
    a.kv_stride[:] = [576, 576]
    a.indices = fake
    a.idx_stride[:] = [64, 64]
    a.s_q, a.s_kv, a.h_q, a.h_kv, a.topk = 4, 300, 128, 1, 64
    a.d_qk, a.dv = 576, 512
    a.softmax_scale = 1 / 24
    a.tile_metadata = fake
    a.num_parts = 4
    a.num_splits = fake
    a.o = fake
    a.lse = fake
    a.workspace = fake
    a.workspace_bytes = _lib.load().mla_workspace_bytes_sparse(4, 1, 4, 128, 1)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("d_qk", 512, _lib.MLA_ERR_UNSUPPORTED),
    ("dv", 576, _lib.MLA_ERR_UNSUPPORTED),
    ("h_kv", 3, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("s_q", 0, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("s_kv", 0, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("topk", 0, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("s_kv", 1 << 21, _lib.MLA_ERR_UNSUPPORTED),               # rows past 2^31 bytes
    ("num_parts", 0, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("workspace_bytes", 16, _lib.MLA_ERR_WORKSPACE_TOO_SMALL),
    ("workspace", None, _lib.MLA_ERR_WORKSPACE_TOO_SMALL),
    ("workspace", (1 << 20) + 16, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("indices", None, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("q", (1 << 20) + 2, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("kv", (1 << 20) + 8, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("lse", None, _lib.MLA_ERR_INVALID_ARGUMENT),
    ("softmax_scale", float("inf"), _lib.MLA_ERR_INVALID_ARGUMENT),
])
def test_prefill_rejects_bad_arguments(field, value, status):
    lib = _lib.load()
    a = _valid_prefill_args()
    setattr(a, field, value)
    assert lib.mla_sparse_prefill_fwd(ctypes.byref(a), None) == status
    assert b"mla_sparse_prefill_fwd" in lib.mla_last_error()


@pytest.mark.parametrize("which,k,value", [("q_stride", 1, 100), ("kv_stride", 0, 4), ("kv_stride", 0, 512),
                                           ("idx_stride", 1, -1)])
def test_prefill_rejects_bad_strides(which, k, value):
    lib = _lib.load()
    a = _valid_prefill_args()
    getattr(a, which)[k] = value
    assert lib.mla_sparse_prefill_fwd(ctypes.byref(a), None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_sparse_prefill_fwd(None, None) == _lib.MLA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("edit,status", [
    (lambda a: (setattr(a, "kv_format", 1), a.kv_stride.__setitem__(slice(0, 3), [64 * 656, 656, 656])),
     _lib.MLA_ERR_UNSUPPORTED),                                                 # FP8 keys
    (lambda a: (setattr(a, "indices", 1 << 20), setattr(a, "topk", 4)), _lib.MLA_ERR_UNSUPPORTED),
    (lambda a: a.vc_stride.__setitem__(1, 100), _lib.MLA_ERR_INVALID_ARGUMENT),
    (lambda a: a.vc_stride.__setitem__(1, 256), _lib.MLA_ERR_INVALID_ARGUMENT),  # smaller than a V row
    (lambda a: setattr(a, "vcache", (1 << 20) + 8), _lib.MLA_ERR_INVALID_ARGUMENT),
    (lambda a: a.vc_stride.__setitem__(1, 1 << 24), _lib.MLA_ERR_UNSUPPORTED),   # 64-token page past 2 GiB
])
def test_decode_rejects_bad_vcache(edit, status):
    lib = _lib.load()
    a = _valid_args()
    a.vcache = 1 << 20
    a.vc_stride[:] = [64 * 512, 512, 512]
    edit(a)
    assert lib.mla_decode_kvcache(ctypes.byref(a), None) == status
    assert b"mla_decode_kvcache" in lib.mla_last_error()
