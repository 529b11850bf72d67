// mla_api.cpp -- the C ABI (include/mla.h): argument checks, the host
// scheduler entry point, and dispatch to the HIP kernels.
#include "../../include/mla.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "kernels.h"
#include "plan.h"

namespace {

thread_local std::string g_last_error;

mla_status fail(mla_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

std::mutex g_cu_mutex;
std::unordered_map<int, int> g_cu_cache;

int query_cus(int device) {
  std::lock_guard<std::mutex> lock(g_cu_mutex);
  auto it = g_cu_cache.find(device);
  if (it != g_cu_cache.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return -1;
  }
  g_cu_cache[device] = n;
  return n;
}

int resolve_cus(int num_cus) {
  if (num_cus > 0) return num_cus;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  return query_cus(dev);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

size_t partial_lse_bytes(int slots, int rows, int h_kv) {
  return align256(static_cast<size_t>(slots) * h_kv * rows * sizeof(float));
}

// Partial O: fp32 for tiles of up to 64 rows; fp16 plus one fp32 scale per 64 dims for
// 128-row tiles (wide: rows > 64, or sparse decode, which always runs 128-row tiles).
size_t partial_o_bytes(int slots, int rows, int h_kv, bool wide) {
  const size_t elem = wide ? sizeof(uint16_t) : sizeof(float);
  return align256(static_cast<size_t>(slots) * h_kv * rows * mla::kDv * elem);
}

size_t partial_scale_bytes(int slots, int rows, int h_kv, bool wide) {
  if (!wide) return 0;
  return align256(static_cast<size_t>(slots) * h_kv * rows * (mla::kDv / 64) * sizeof(float));
}

size_t workspace_bytes(int batch, int num_parts, int rows, int h_kv, bool wide) {
  const int slots = batch + num_parts;
  return partial_o_bytes(slots, rows, h_kv, wide) + partial_scale_bytes(slots, rows, h_kv, wide) +
         partial_lse_bytes(slots, rows, h_kv);
}


mla_status check_workspace(const char* fn, const void* workspace, size_t bytes, size_t need) {
  if (!workspace || bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace of %zu bytes, need %zu", fn, bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: workspace must be 256-byte aligned", fn);
  return MLA_OK;
}

// The common tail of the entry points: the grid bound, the partials' places in the
// workspace, and the launch of the split and combine kernels. p holds everything else.
mla_status finish_and_launch(const char* fn, mla::DecodeParams& p, const mla::Plan& plan, int kv_format,
                             void* workspace, int num_parts, int max_splits, void* const events[3],
                             void* hip_stream) {
  const long wgs = static_cast<long>(num_parts) * plan.m_tiles * p.h_kv;
  if (wgs > (1L << 30)) return fail(MLA_ERR_UNSUPPORTED, "%s: grid too large", fn);
  const int slots = p.batch + num_parts;
  char* const ws = static_cast<char*>(workspace);
  p.part_o32 = plan.wide ? nullptr : reinterpret_cast<float*>(ws);
  p.part_o16 = plan.wide ? reinterpret_cast<uint16_t*>(ws) : nullptr;
  p.part_scale = plan.wide ? reinterpret_cast<float*>(ws + partial_o_bytes(slots, p.rows, p.h_kv, true)) : nullptr;
  p.part_lse = reinterpret_cast<float*>(ws + partial_o_bytes(slots, p.rows, p.h_kv, plan.wide) +
                                        partial_scale_bytes(slots, p.rows, p.h_kv, plan.wide));
  p.max_slots = slots;
  p.max_splits = max_splits > 0 ? max_splits : 0;
  p.grid_wgs = static_cast<int>(wgs);
  const hipError_t err = mla::launch_decode(p, plan, kv_format, static_cast<hipStream_t>(hip_stream), events);
  if (err != hipSuccess) return fail(MLA_ERR_HIP, "%s: %s", fn, hipGetErrorString(err));
  return MLA_OK;
}

// Validation, argument packing and launch for both decode entry points.
// use_scratch: the workspace is the library's static scratch (the caller's
// workspace fields are ignored); nothing is allocated either way.
mla_status decode_impl(const mla_decode_args* a, void* hip_stream, bool use_scratch) {
  if (!a) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: args is null");
  if (!a->q || !a->kvcache || !a->block_table || !a->cache_seqlens || !a->tile_metadata || !a->num_splits ||
      !a->o || !a->lse)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: null pointer among q, kvcache, block_table, "
                                          "cache_seqlens, tile_metadata, num_splits, o, lse");
  if (a->batch < 1 || a->s_q < 1 || a->h_q < 1 || a->h_kv < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: batch, s_q, h_q, h_kv must be >= 1");
  if (a->h_q % a->h_kv)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: h_q (%d) is not a multiple of h_kv (%d)", a->h_q,
                a->h_kv);
  if (a->d_qk != mla::kDqk) return fail(MLA_ERR_UNSUPPORTED, "mla_decode_kvcache: d_qk must be 576 (got %d)", a->d_qk);
  if (a->dv != mla::kDv) return fail(MLA_ERR_UNSUPPORTED, "mla_decode_kvcache: dv must be 512 (got %d)", a->dv);
  if (a->kv_format != MLA_KV_BF16 && a->kv_format != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: unknown kv_format %d", a->kv_format);
  if (!(std::isfinite(a->softmax_scale)))
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: softmax_scale must be finite");
  if (a->num_pages < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: num_pages must be >= 1");
  if (a->max_blocks_per_seq < 1 || a->bt_stride < a->max_blocks_per_seq)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: need max_blocks_per_seq >= 1 and bt_stride >= it");
  if (a->max_blocks_per_seq > (1 << 25))
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode_kvcache: max_blocks_per_seq above 2^25 (lengths past 2^31 tokens)");
  if (a->num_parts < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: num_parts must be >= 1");
  if (static_cast<int64_t>(a->batch) * a->s_q * a->h_q > (int64_t{1} << 31) / mla::kDv)
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode_kvcache: output too large");

  // q: bf16, 576 contiguous dims, 16-byte aligned rows.
  for (int k = 0; k < 3; ++k)
    if (a->q_stride[k] < 0 || (a->q_stride[k] % 8) != 0)
      return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: q_stride[%d] = %lld must be a non-negative multiple of 8",
                  k, static_cast<long long>(a->q_stride[k]));
  if (!aligned16(a->q)) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: q must be 16-byte aligned");
  if (a->q_stride[2] < mla::kDqk && a->h_q > 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: q head stride overlaps the 576 dims");
  if (((a->s_q - 1) * a->q_stride[1] + (a->h_q - 1) * a->q_stride[2] + mla::kDqk) * 2 >= (int64_t{1} << 31))
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode_kvcache: the q rows of one sequence must span less than 2 GiB");

  // kvcache rows: contiguous, 16-byte aligned.
  const int64_t elem = (a->kv_format == MLA_KV_BF16) ? 2 : 1;
  const int64_t row_bytes = (a->kv_format == MLA_KV_BF16) ? mla::kDqk * 2 : mla::kFp8Record;
  int64_t kvb[3];
  for (int k = 0; k < 3; ++k) {
    kvb[k] = a->kv_stride[k] * elem;
    if (a->kv_stride[k] < 0 || (kvb[k] % 16) != 0)
      return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: kv_stride[%d] must be non-negative and a multiple "
                  "of 16 bytes", k);
  }
  if (kvb[0] < row_bytes || kvb[1] < row_bytes || (a->h_kv > 1 && kvb[2] < row_bytes))
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: a kv stride is smaller than one cached row (%lld bytes)",
                static_cast<long long>(row_bytes));
  if (!aligned16(a->kvcache)) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: kvcache must be 16-byte aligned");
  if (kvb[1] * mla::kPage >= (int64_t{1} << 31))
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode_kvcache: a 64-token page must span less than 2 GiB (token stride %lld bytes)",
                static_cast<long long>(kvb[1]));
  if ((reinterpret_cast<uintptr_t>(a->o) & 7u) || (reinterpret_cast<uintptr_t>(a->lse) & 3u))
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: o must be 8-byte and lse 4-byte aligned");

  const int group = a->h_q / a->h_kv;
  // sparse decode: every (sequence, query token) pair is a virtual sequence of topk entries
  const bool sparse = a->indices != nullptr;
  const int vbatch = sparse ? a->batch * a->s_q : a->batch;
  const int rows = sparse ? group : a->s_q * group;
  mla::Plan plan = sparse ? mla::make_plan_sparse(group) : mla::make_plan(rows, a->kv_format);
  int64_t vcb[3] = {0, 0, 0};
  if (a->vcache) {
    if (a->kv_format != MLA_KV_BF16)
      return fail(MLA_ERR_UNSUPPORTED, "mla_decode_kvcache: a separate V cache needs bf16 keys (kv_format 0)");
    if (sparse) return fail(MLA_ERR_UNSUPPORTED, "mla_decode_kvcache: a separate V cache with indices");
    for (int k = 0; k < 3; ++k) {
      vcb[k] = a->vc_stride[k] * 2;
      if (a->vc_stride[k] < 0 || (vcb[k] % 16) != 0)
        return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: vc_stride[%d] must be non-negative and a multiple "
                    "of 16 bytes", k);
    }
    const int64_t vrow = mla::kDv * 2;
    if (vcb[0] < vrow || vcb[1] < vrow || (a->h_kv > 1 && vcb[2] < vrow))
      return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: a vcache stride is smaller than one V row (%lld bytes)",
                  static_cast<long long>(vrow));
    if (!aligned16(a->vcache))
      return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: vcache must be 16-byte aligned");
    if (vcb[1] * mla::kPage >= (int64_t{1} << 31))
      return fail(MLA_ERR_UNSUPPORTED, "mla_decode_kvcache: a 64-token V page must span less than 2 GiB");
    // 64-row tiles whatever the row count; the partial format (plan.wide) stays the plain decode's
    plan.m_tile = 64;
    plan.m_tiles = (rows + 63) / 64;
  }
  int64_t pool_bytes = 0;
  if (sparse) {
    if (a->topk < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: topk must be >= 1 with indices");
    if (a->idx_stride[0] < 0 || a->idx_stride[1] < 0)
      return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: idx_stride must be non-negative");
    if (static_cast<int64_t>(a->batch) * a->s_q > (1 << 24) ||
        (static_cast<int64_t>(a->batch - 1) * a->idx_stride[0] + (a->s_q - 1) * a->idx_stride[1] + a->topk) >=
            (int64_t{1} << 31))
      return fail(MLA_ERR_UNSUPPORTED, "mla_decode_kvcache: indices must span less than 2^31 entries");
    if (a->s_q > 1 && a->q_stride[0] != a->s_q * a->q_stride[1])
      return fail(MLA_ERR_UNSUPPORTED, "mla_decode_kvcache: sparse decode needs q's sequence stride to be s_q times its "
                  "token stride");
    pool_bytes = static_cast<int64_t>(a->num_pages) * kvb[0];
    if (pool_bytes > (int64_t{1} << 31) - (int64_t{1} << 16))
      return fail(MLA_ERR_UNSUPPORTED, "mla_decode_kvcache: sparse decode needs the KV pool to span less than 2^31 "
                  "bytes (%lld)", static_cast<long long>(pool_bytes));
  }
  const size_t need = workspace_bytes(vbatch, a->num_parts, rows, a->h_kv, plan.wide);
  void* workspace = a->workspace;
  if (!use_scratch) {
    const mla_status st = check_workspace("mla_decode_kvcache", workspace, a->workspace_bytes, need);
    if (st != MLA_OK) return st;
  }
  if (use_scratch) {
    if (need > mla::kScratchBytes)
      return fail(MLA_ERR_WORKSPACE_TOO_SMALL,
                  "mla_decode_kvcache_noalloc: this call needs %zu bytes of workspace; the static scratch holds %zu "
                  "(fewer num_parts or a smaller batch, or mla_decode_kvcache with a caller workspace)",
                  need, mla::kScratchBytes);
  }
  const long wgs = static_cast<long>(a->num_parts) * plan.m_tiles * a->h_kv;
  if (wgs > (1L << 30)) return fail(MLA_ERR_UNSUPPORTED, "mla_decode_kvcache: grid too large");
  if (use_scratch) {
    const hipError_t e = mla::scratch_workspace(&workspace);   // device address of this device's scratch
    if (e != hipSuccess)
      return fail(MLA_ERR_HIP, "mla_decode_kvcache_noalloc: no address for the static scratch: %s",
                  hipGetErrorString(e));
  }

  mla::DecodeParams p{};
  p.q = static_cast<const uint16_t*>(a->q);
  p.q_sb = a->q_stride[0];
  p.q_ss = a->q_stride[1];
  p.q_sh = a->q_stride[2];
  p.kv = static_cast<const uint8_t*>(a->kvcache);
  p.kv_sp = kvb[0];
  p.kv_st = kvb[1];
  p.kv_sh = kvb[2];
  p.num_pages = a->num_pages;
  p.block_table = a->block_table;
  p.bt_stride = a->bt_stride;
  p.max_blocks = a->max_blocks_per_seq;
  p.seqlens = a->cache_seqlens;
  p.meta = a->tile_metadata;
  p.num_parts = a->num_parts;
  p.num_splits = a->num_splits;
  p.batch = vbatch;
  p.s_q = sparse ? 1 : a->s_q;
  p.h_q = a->h_q;
  p.h_kv = a->h_kv;
  p.group = group;
  p.rows = rows;
  p.causal = (a->causal && !sparse) ? 1 : 0;
  if (sparse) {
    p.q_sb = a->q_stride[1];                // virtual sequence b * s_q + s starts at q[b, s]
    p.indices = a->indices;
    p.idx_sb = a->idx_stride[0];
    p.idx_ss = a->idx_stride[1];
    p.topk = a->topk;
    p.sq_real = a->s_q;
    p.real_causal = a->causal ? 1 : 0;
    p.pool_bytes = pool_bytes;
  }
  if (a->vcache) {
    p.vcache = static_cast<const uint8_t*>(a->vcache);
    p.vc_sp = vcb[0];
    p.vc_st = vcb[1];
    p.vc_sh = vcb[2];
  }
  p.scale_log2 = static_cast<float>(static_cast<double>(a->softmax_scale) * 1.4426950408889634074);
  p.o = static_cast<uint16_t*>(a->o);
  p.lse = a->lse;
  return finish_and_launch("mla_decode_kvcache", p, plan, a->kv_format, workspace, a->num_parts, a->max_splits,
                           a->events, hip_stream);
}

// Sparse prefill: every query token s is virtual sequence s (batch s_q, one query
// token each) of topk entries over the contiguous kv rows; the sparse decode kernels run it.
mla_status prefill_impl(const mla_sparse_prefill_args* a, void* hip_stream) {
  const char* const fn = "mla_sparse_prefill_fwd";
  if (!a) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: args is null", fn);
  if (!a->q || !a->kv || !a->indices || !a->tile_metadata || !a->num_splits || !a->o || !a->lse)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: null pointer among q, kv, indices, tile_metadata, num_splits, o, lse", fn);
  if (a->s_q < 1 || a->s_kv < 1 || a->h_q < 1 || a->h_kv < 1 || a->topk < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: s_q, s_kv, h_q, h_kv, topk must be >= 1", fn);
  if (a->h_q % a->h_kv)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: h_q (%d) is not a multiple of h_kv (%d)", fn, a->h_q, a->h_kv);
  if (a->d_qk != mla::kDqk) return fail(MLA_ERR_UNSUPPORTED, "%s: d_qk must be 576 (got %d)", fn, a->d_qk);
  if (a->dv != mla::kDv) return fail(MLA_ERR_UNSUPPORTED, "%s: dv must be 512 (got %d)", fn, a->dv);
  if (!(std::isfinite(a->softmax_scale))) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: softmax_scale must be finite", fn);
  if (a->num_parts < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: num_parts must be >= 1", fn);
  if (a->s_q > (1 << 24)) return fail(MLA_ERR_UNSUPPORTED, "%s: s_q above 2^24", fn);
  if (static_cast<int64_t>(a->s_q) * a->h_q > (int64_t{1} << 31) / mla::kDv)
    return fail(MLA_ERR_UNSUPPORTED, "%s: output too large", fn);

  // q: bf16 [s_q, h_q, 576], 576 contiguous dims, 16-byte aligned rows.
  for (int k = 0; k < 2; ++k)
    if (a->q_stride[k] < 0 || (a->q_stride[k] % 8) != 0)
      return fail(MLA_ERR_INVALID_ARGUMENT, "%s: q_stride[%d] = %lld must be a non-negative multiple of 8", fn, k,
                  static_cast<long long>(a->q_stride[k]));
  if (!aligned16(a->q)) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: q must be 16-byte aligned", fn);
  if (a->q_stride[1] < mla::kDqk && a->h_q > 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: q head stride overlaps the 576 dims", fn);
  if (((a->h_q - 1) * a->q_stride[1] + mla::kDqk) * 2 >= (int64_t{1} << 31))
    return fail(MLA_ERR_UNSUPPORTED, "%s: the q rows of one token must span less than 2 GiB", fn);

  // kv: bf16 [s_kv, h_kv, 576], rows contiguous and 16-byte aligned.
  int64_t kvb[2];
  for (int k = 0; k < 2; ++k) {
    kvb[k] = a->kv_stride[k] * 2;
    if (a->kv_stride[k] < 0 || (kvb[k] % 16) != 0)
      return fail(MLA_ERR_INVALID_ARGUMENT, "%s: kv_stride[%d] must be non-negative and a multiple of 16 bytes", fn, k);
  }
  const int64_t row_bytes = mla::kDqk * 2;
  if (kvb[0] < row_bytes || (a->h_kv > 1 && kvb[1] < row_bytes))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: a kv stride is smaller than one row (1152 bytes)", fn);
  if (!aligned16(a->kv)) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: kv must be 16-byte aligned", fn);
  const int64_t pool_bytes = static_cast<int64_t>(a->s_kv - 1) * kvb[0] + row_bytes;
  if (kvb[0] * mla::kPage >= (int64_t{1} << 31) || pool_bytes > (int64_t{1} << 31) - (int64_t{1} << 16))
    return fail(MLA_ERR_UNSUPPORTED, "%s: the kv rows of a head must span less than 2^31 bytes (%lld)", fn,
                static_cast<long long>(pool_bytes));

  // indices: int32 [s_q, h_kv, topk], last dim contiguous.
  if (a->idx_stride[0] < 0 || a->idx_stride[1] < 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: idx_stride must be non-negative", fn);
  if (static_cast<int64_t>(a->s_q - 1) * a->idx_stride[0] + static_cast<int64_t>(a->h_kv - 1) * a->idx_stride[1] +
          a->topk >= (int64_t{1} << 31))
    return fail(MLA_ERR_UNSUPPORTED, "%s: indices must span less than 2^31 entries", fn);
  if ((reinterpret_cast<uintptr_t>(a->o) & 7u) || (reinterpret_cast<uintptr_t>(a->lse) & 3u))
    return fail(MLA_ERR_INVALID_ARGUMENT, "%s: o must be 8-byte and lse 4-byte aligned", fn);

  const int group = a->h_q / a->h_kv;
  const mla::Plan plan = mla::make_plan_sparse(group);
  const size_t need = workspace_bytes(a->s_q, a->num_parts, group, a->h_kv, true);
  {
    const mla_status st = check_workspace(fn, a->workspace, a->workspace_bytes, need);
    if (st != MLA_OK) return st;
  }

  mla::DecodeParams p{};
  p.q = static_cast<const uint16_t*>(a->q);
  p.q_sb = a->q_stride[0];                 // virtual sequence s is query token s
  p.q_ss = a->q_stride[0];
  p.q_sh = a->q_stride[1];
  p.kv = static_cast<const uint8_t*>(a->kv);
  p.kv_st = kvb[0];
  p.kv_sp = kvb[0] * mla::kPage;
  p.kv_sh = kvb[1];
  p.num_pages = (a->s_kv + mla::kPage - 1) / mla::kPage;
  p.block_table = nullptr;
  p.bt_stride = 0;
  p.max_blocks = p.num_pages;
  p.seqlens = nullptr;
  p.kv_rows = a->s_kv;
  p.meta = a->tile_metadata;
  p.num_parts = a->num_parts;
  p.num_splits = a->num_splits;
  p.batch = a->s_q;
  p.s_q = 1;
  p.h_q = a->h_q;
  p.h_kv = a->h_kv;
  p.group = group;
  p.rows = group;
  p.causal = 0;
  p.indices = a->indices;
  p.idx_sb = a->idx_stride[0];
  p.idx_ss = 0;
  p.idx_sh = a->idx_stride[1];
  p.topk = a->topk;
  p.sq_real = 1;
  p.real_causal = 0;
  p.pool_bytes = pool_bytes;
  p.scale_log2 = static_cast<float>(static_cast<double>(a->softmax_scale) * 1.4426950408889634074);
  p.o = static_cast<uint16_t*>(a->o);
  p.lse = a->lse;
  return finish_and_launch(fn, p, plan, MLA_KV_BF16, a->workspace, a->num_parts, a->max_splits, a->events,
                           hip_stream);
}

}  // namespace

extern "C" {

const char* mla_last_error(void) { return g_last_error.c_str(); }

const char* mla_version(void) { return "paged_mla_decode_amd 0.1 (gfx950)"; }

size_t mla_decode_args_size(void) { return sizeof(mla_decode_args); }

int mla_device_cu_count(int device) { return query_cus(device); }

int mla_num_parts(int batch, int heads_per_kv, int h_kv, int kv_format, int num_cus) {
  if (batch < 1 || heads_per_kv < 1 || h_kv < 1 ||
      (kv_format != MLA_KV_BF16 && kv_format != MLA_KV_FP8_E4M3)) {
    fail(MLA_ERR_INVALID_ARGUMENT, "mla_num_parts: need batch >= 1, heads_per_kv >= 1, h_kv >= 1 and a known kv_format");
    return -1;
  }
  int cus = resolve_cus(num_cus);
  if (cus <= 0) {
    fail(MLA_ERR_HIP, "mla_num_parts: cannot query the CU count of the current device (pass num_cus > 0)");
    return -1;
  }
  return mla::default_parts(mla::make_plan(heads_per_kv, kv_format), h_kv, cus);
}

mla_status mla_get_metadata(const int32_t* cache_seqlens_host, int batch, int heads_per_kv, int h_kv,
                            int kv_format, int max_blocks_per_seq, int num_cus, int num_parts,
                            int32_t* tile_metadata_host, int32_t* num_splits_host, int* num_parts_out) {
  if (!cache_seqlens_host || !tile_metadata_host || !num_splits_host)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata: null pointer");
  if (batch < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata: batch must be >= 1 (got %d)", batch);
  if (heads_per_kv < 1 || h_kv < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata: heads_per_kv and h_kv must be >= 1");
  if (kv_format != MLA_KV_BF16 && kv_format != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata: unknown kv_format %d", kv_format);
  if (num_parts < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata: num_parts must be >= 0");
  if (max_blocks_per_seq < 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata: max_blocks_per_seq must be >= 0 (0: unchecked)");
  const int64_t max_len = static_cast<int64_t>(max_blocks_per_seq) * mla::kPage;
  for (int b = 0; b < batch; ++b) {
    if (cache_seqlens_host[b] < 0)
      return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata: cache_seqlens[%d] = %d is negative", b,
                  cache_seqlens_host[b]);
    if (max_blocks_per_seq > 0 && cache_seqlens_host[b] > max_len)
      return fail(MLA_ERR_INVALID_ARGUMENT,
                  "mla_get_metadata: cache_seqlens[%d] = %d exceeds the block table (%d entries x 64 tokens)", b,
                  cache_seqlens_host[b], max_blocks_per_seq);
  }
  const mla::Plan plan = mla::make_plan(heads_per_kv, kv_format);
  int parts = num_parts;
  if (parts == 0) {
    int cus = resolve_cus(num_cus);
    if (cus <= 0) return fail(MLA_ERR_HIP, "mla_get_metadata: cannot query the CU count (pass num_cus > 0)");
    parts = mla::default_parts(plan, h_kv, cus);
  }
  mla::schedule(cache_seqlens_host, batch, parts, plan.split_cost, plan.min_pages, tile_metadata_host,
                num_splits_host);
  if (num_parts_out) *num_parts_out = parts;
  return MLA_OK;
}

mla_status mla_get_metadata_device(const int32_t* cache_seqlens, int batch, int heads_per_kv, int h_kv,
                                   int kv_format, int num_cus, int num_parts, int32_t* tile_metadata,
                                   int32_t* num_splits, int* num_parts_out, void* hip_stream) {
  if (!cache_seqlens || !tile_metadata || !num_splits)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata_device: null pointer");
  if (batch < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata_device: batch must be >= 1 (got %d)", batch);
  if (heads_per_kv < 1 || h_kv < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata_device: heads_per_kv and h_kv must be >= 1");
  if (kv_format != MLA_KV_BF16 && kv_format != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata_device: unknown kv_format %d", kv_format);
  if (num_parts < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata_device: num_parts must be >= 0");
  const mla::Plan plan = mla::make_plan(heads_per_kv, kv_format);
  int parts = num_parts;
  if (parts == 0) {
    const int cus = resolve_cus(num_cus);
    if (cus <= 0) return fail(MLA_ERR_HIP, "mla_get_metadata_device: cannot query the CU count (pass num_cus > 0)");
    parts = mla::default_parts(plan, h_kv, cus);
  }
  if (!mla::schedule_device_supported(batch, parts, plan.split_cost, plan.min_pages))
    return fail(MLA_ERR_UNSUPPORTED, "mla_get_metadata_device: supports batch <= 1023 and num_parts <= 1024 "
                "(got %d and %d); use mla_get_metadata", batch, parts);
  const hipError_t err = mla::launch_schedule_device(cache_seqlens, batch, parts, plan.split_cost, tile_metadata,
                                                     num_splits, static_cast<hipStream_t>(hip_stream));
  if (err != hipSuccess) return fail(MLA_ERR_HIP, "mla_get_metadata_device: %s", hipGetErrorString(err));
  if (num_parts_out) *num_parts_out = parts;
  return MLA_OK;
}

size_t mla_workspace_bytes(int batch, int num_parts, int heads_per_kv, int h_kv) {
  if (batch < 1 || num_parts < 1 || heads_per_kv < 1 || h_kv < 1) return 0;
  return workspace_bytes(batch, num_parts, heads_per_kv, h_kv, heads_per_kv > 64);
}

size_t mla_workspace_bytes_sparse(int batch, int s_q, int num_parts, int h_q, int h_kv) {
  if (batch < 1 || s_q < 1 || num_parts < 1 || h_q < 1 || h_kv < 1 || h_q % h_kv) return 0;
  return workspace_bytes(batch * s_q, num_parts, h_q / h_kv, h_kv, true);
}

mla_status mla_get_metadata_sparse(int batch, int s_q, int topk, int h_q, int h_kv, int kv_format, int num_cus,
                                   int num_parts, int32_t* tile_metadata_host, int32_t* num_splits_host,
                                   int* num_parts_out) {
  if (!tile_metadata_host || !num_splits_host)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata_sparse: null pointer");
  if (batch < 1 || s_q < 1 || topk < 1 || h_q < 1 || h_kv < 1 || h_q % h_kv)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata_sparse: need batch, s_q, topk, h_q, h_kv >= 1 and "
                "h_q a multiple of h_kv");
  if (kv_format != MLA_KV_BF16 && kv_format != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata_sparse: unknown kv_format %d", kv_format);
  if (num_parts < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata_sparse: num_parts must be >= 0");
  if (static_cast<int64_t>(batch) * s_q > (1 << 24))
    return fail(MLA_ERR_UNSUPPORTED, "mla_get_metadata_sparse: batch * s_q above 2^24");
  const mla::Plan plan = mla::make_plan_sparse(h_q / h_kv);
  int parts = num_parts;
  if (parts == 0) {
    const int cus = resolve_cus(num_cus);
    if (cus <= 0) return fail(MLA_ERR_HIP, "mla_get_metadata_sparse: cannot query the CU count (pass num_cus > 0)");
    parts = mla::default_parts(plan, h_kv, cus);
  }
  const std::vector<int32_t> lengths(static_cast<size_t>(batch) * s_q, topk);
  mla::schedule(lengths.data(), batch * s_q, parts, plan.split_cost, plan.min_pages, tile_metadata_host,
                num_splits_host);
  if (num_parts_out) *num_parts_out = parts;
  return MLA_OK;
}

mla_status mla_decode_kvcache(const mla_decode_args* a, void* hip_stream) {
  return decode_impl(a, hip_stream, false);
}

mla_status mla_decode_kvcache_noalloc(const mla_decode_args* a, void* hip_stream) {
  return decode_impl(a, hip_stream, true);
}

mla_status mla_sparse_prefill_fwd(const mla_sparse_prefill_args* a, void* hip_stream) {
  return prefill_impl(a, hip_stream);
}

size_t mla_sparse_prefill_args_size(void) { return sizeof(mla_sparse_prefill_args); }

}  // extern "C"
