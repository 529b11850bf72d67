// kernels.h -- the validated argument block the HIP kernels receive.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "plan.h"

namespace mla {

struct DecodeParams {
  const uint16_t* q;          // bf16 bits
  int64_t q_sb, q_ss, q_sh;   // element strides: batch, query token, head
  const uint8_t* kv;          // cache base (bytes)
  int64_t kv_sp, kv_st, kv_sh;  // byte strides: page, token, head
  int num_pages;
  const int32_t* block_table;
  int64_t bt_stride;
  int max_blocks;
  const int32_t* seqlens;
  const int32_t* meta;
  int num_parts;
  const int32_t* num_splits;
  int batch, s_q, h_q, h_kv, group, rows;  // group = h_q / h_kv, rows = s_q * group
  int causal;
  float scale_log2;           // softmax_scale * log2(e)
  uint16_t* o;                // bf16 bits [batch, s_q, h_q, 512]
  float* lse;                 // [batch, h_q, s_q]
  // Partial O of the pieces, [slots, h_kv, rows, 512]: fp32 (part_o32) for tiles of up to 64
  // rows; fp16 (part_o16) with a power-of-two scale per 64-dim block (part_scale,
  // [slots, h_kv, rows, 8]) for 128-row tiles. The other pointer is null.
  float* part_o32;
  uint16_t* part_o16;
  float* part_scale;
  float* part_lse;            // [slots, h_kv, rows]
  int max_slots;
  int max_splits;             // hint: largest piece count of any sequence (0 = unknown)
  int grid_wgs;               // real workgroups of the split kernel (the grid is padded to a multiple of 8)
  // Token-level sparse decode (topk > 0): every (sequence, query token) pair is a virtual
  // sequence vb = b * sq_real + s of topk index entries, so batch = batch_real * sq_real,
  // s_q = 1, rows = group = h_q / h_kv, and q_sb is the query-token stride. indices
  // [batch_real, sq_real, topk] name cached positions of sequence b (-1: none); seqlens holds
  // the real lengths [batch_real].
  const int32_t* indices;
  int64_t idx_sb, idx_ss;     // element strides of indices: sequence, query token
  int64_t idx_sh;             // ... and KV head (0: one list serves every KV head)
  int topk;                   // 0: dense decode
  int sq_real;
  int real_causal;            // sparse: the causal flag (applied to the listed positions)
  int64_t pool_bytes;         // sparse: bytes from a KV head's base to the end of the pool (< 2^31)
  // Sparse prefill (kv_rows > 0): the keys are kv_rows contiguous rows, row t at byte t * kv_st
  // (64-row pages, page i = rows 64 i .. 64 i + 63, kv_sp = 64 kv_st); no block table, no
  // seqlens: every query token's length is kv_rows.
  int kv_rows;
  // A separate V cache (non-null: bf16 rows of kDv dims, byte strides page / token / head;
  // same block table as the keys); bf16 keys, dense decode only.
  const uint8_t* vcache;
  int64_t vc_sp, vc_st, vc_sh;
};

// The row-tile split kernel (mla_kernels_x.hip): 128-row tiles, 8 waves of
// 16 rows each in the S phase (rows_per_wave must be 32: the 4-wave row count
// the plan records for a 128-row tile); grid padded to a multiple of 8.
// ev_start / ev_stop (may be null) take the kernel's start and end timestamps.
hipError_t launch_split_x(const DecodeParams& p, int kv_format, int rows_per_wave, int grid, hipStream_t stream,
                          hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_split_x_sparse(const DecodeParams& p, int kv_format, int grid, hipStream_t stream,
                                 hipEvent_t ev_start, hipEvent_t ev_stop);
// The separate-V-cache split kernel (mla_kernels_x.hip): 64-row tiles, 4 waves;
// fp16 block-scaled partials when p.part_o16 is set (more than 64 rows), else fp32.
hipError_t launch_split_vc(const DecodeParams& p, int grid, hipStream_t stream, hipEvent_t ev_start,
                           hipEvent_t ev_stop);

hipError_t launch_decode(const DecodeParams& p, const Plan& plan, int kv_format, hipStream_t stream,
                         void* const events[3]);

// The tile scheduler on the device (scheduler_device.hip): the same metadata
// as schedule() in scheduler.cpp, from device lengths, by one workgroup.
bool schedule_device_supported(int batch, int num_parts, int split_cost, int min_pages);
hipError_t launch_schedule_device(const int32_t* seqlens, int batch, int num_parts, int split_cost, int32_t* meta,
                                  int32_t* num_splits, hipStream_t stream);

// The library's static device scratch (mla_kernels.hip), the workspace of
// mla_decode_kvcache_noalloc: kScratchBytes per device, held until the process
// ends. *ptr receives its device address on the current device (looked up once
// per device with hipGetSymbolAddress, then cached).
constexpr size_t kScratchBytes = static_cast<size_t>(128) << 20;
hipError_t scratch_workspace(void** ptr);

}  // namespace mla
