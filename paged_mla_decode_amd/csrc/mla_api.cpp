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

// Partial O: fp32 for tiles of up to 64 rows; fp16 plus one fp32 scale per 64 dims for
// 128-row tiles (rows > 64).
size_t partial_o_bytes(int slots, int rows, int h_kv) {
  const size_t elem = rows > 64 ? sizeof(uint16_t) : sizeof(float);
  return align256(static_cast<size_t>(slots) * h_kv * rows * mla::kDv * elem);
}

size_t partial_scale_bytes(int slots, int rows, int h_kv) {
  if (rows <= 64) return 0;
  return align256(static_cast<size_t>(slots) * h_kv * rows * (mla::kDv / 64) * sizeof(float));
}

size_t partial_lse_bytes(int slots, int rows, int h_kv) {
  return align256(static_cast<size_t>(slots) * h_kv * rows * sizeof(float));
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
                            int kv_format, int num_cus, int num_parts, int32_t* tile_metadata_host,
                            int32_t* num_splits_host, int* num_parts_out) {
  if (!cache_seqlens_host || !tile_metadata_host || !num_splits_host)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata: null pointer");
  if (batch < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata: batch must be >= 1 (got %d)", batch);
  if (heads_per_kv < 1 || h_kv < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata: heads_per_kv and h_kv must be >= 1");
  if (kv_format != MLA_KV_BF16 && kv_format != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata: unknown kv_format %d", kv_format);
  if (num_parts < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata: num_parts must be >= 0");
  for (int b = 0; b < batch; ++b)
    if (cache_seqlens_host[b] < 0)
      return fail(MLA_ERR_INVALID_ARGUMENT, "mla_get_metadata: cache_seqlens[%d] = %d is negative", b,
                  cache_seqlens_host[b]);
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

size_t mla_workspace_bytes(int batch, int num_parts, int heads_per_kv, int h_kv) {
  if (batch < 1 || num_parts < 1 || heads_per_kv < 1 || h_kv < 1) return 0;
  const int slots = batch + num_parts;
  return partial_o_bytes(slots, heads_per_kv, h_kv) + partial_scale_bytes(slots, heads_per_kv, h_kv) +
         partial_lse_bytes(slots, heads_per_kv, h_kv);
}

mla_status mla_decode_kvcache(const mla_decode_args* a, void* hip_stream) {
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
  const int rows = a->s_q * group;
  const mla::Plan plan = mla::make_plan(rows, a->kv_format);
  const size_t need = mla_workspace_bytes(a->batch, a->num_parts, rows, a->h_kv);
  if (!a->workspace || a->workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "mla_decode_kvcache: workspace of %zu bytes, need %zu", a->workspace_bytes,
                need);
  if (reinterpret_cast<uintptr_t>(a->workspace) & 255u)
    return fail(MLA_ERR_INVALID_ARGUMENT, "mla_decode_kvcache: workspace must be 256-byte aligned");
  const long wgs = static_cast<long>(a->num_parts) * plan.m_tiles * a->h_kv;
  if (wgs > (1L << 30)) return fail(MLA_ERR_UNSUPPORTED, "mla_decode_kvcache: grid too large");

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
  p.batch = a->batch;
  p.s_q = a->s_q;
  p.h_q = a->h_q;
  p.h_kv = a->h_kv;
  p.group = group;
  p.rows = rows;
  p.causal = a->causal ? 1 : 0;
  p.scale_log2 = static_cast<float>(static_cast<double>(a->softmax_scale) * 1.4426950408889634074);
  p.o = static_cast<uint16_t*>(a->o);
  p.lse = a->lse;
  const int slots = a->batch + a->num_parts;
  char* const ws = static_cast<char*>(a->workspace);
  p.part_o32 = plan.wide ? nullptr : reinterpret_cast<float*>(ws);
  p.part_o16 = plan.wide ? reinterpret_cast<uint16_t*>(ws) : nullptr;
  p.part_scale = plan.wide ? reinterpret_cast<float*>(ws + partial_o_bytes(slots, rows, a->h_kv)) : nullptr;
  p.part_lse = reinterpret_cast<float*>(ws + partial_o_bytes(slots, rows, a->h_kv) +
                                        partial_scale_bytes(slots, rows, a->h_kv));
  p.max_slots = slots;
  p.max_splits = a->max_splits > 0 ? a->max_splits : 0;
  p.grid_wgs = static_cast<int>(wgs);

  hipError_t err = mla::launch_decode(p, plan, a->kv_format, static_cast<hipStream_t>(hip_stream), a->events);
  if (err != hipSuccess) return fail(MLA_ERR_HIP, "mla_decode_kvcache: %s", hipGetErrorString(err));
  return MLA_OK;
}

}  // extern "C"
