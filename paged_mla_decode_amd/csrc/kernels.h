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
};

// The row-tile split kernel (mla_kernels_x.hip): 128-row tiles, 8 waves of
// 16 rows each in the S phase (rows_per_wave must be 32: the 4-wave row count
// the plan records for a 128-row tile); grid padded to a multiple of 8.
// ev_start / ev_stop (may be null) take the kernel's start and end timestamps.
hipError_t launch_split_x(const DecodeParams& p, int kv_format, int rows_per_wave, int grid, hipStream_t stream,
                          hipEvent_t ev_start, hipEvent_t ev_stop);

hipError_t launch_decode(const DecodeParams& p, const Plan& plan, int kv_format, hipStream_t stream,
                         void* const events[3]);

}  // namespace mla
