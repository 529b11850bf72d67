/*
 * mla.h -- C ABI of the MI355X (gfx950) paged MLA decode library (libmla.so).
 *
 * The operation: Multi-head Latent Attention decode over a paged KV cache.
 * For each sequence b, s_q query tokens x h_q heads attend to the L_b cached
 * tokens of one latent KV head per group of G = h_q / h_kv query heads. A
 * cached token is a 576-dim row (512 latent + 64 RoPE dims); V is its first
 * dv = 512 dims. Tokens live in 64-token pages that block_table addresses.
 * Sources (FlashMLA web pages):
 *   - the two calls and their shapes: mmssai.com FlashMLA article, section
 *     "代码解读：flash_api.cpp 核心逻辑" (get_mla_metadata, mha_fwd_kvcache_mla,
 *     q [batch, seqlen_q, num_heads, head_size], kcache [num_blocks,
 *     page_block_size, num_heads_k, head_size], seqlens_k [batch], block_table
 *     [batch, max_num_blocks_per_seq], tile_scheduler_metadata [num_sm_parts,
 *     TileSchedulerMetaDataSize], num_splits [batch + 1]);
 *   - usage (metadata once per decode step, reused by every layer; the call
 *     returns (o, lse)): kdjingpai.com FlashMLA post, "功能 1"; aiboss88.com
 *     FlashMLA page, "FlashMLAを使用する";
 *   - 64-token pages: kdjingpai.com, "功能 2"; head size 576 from
 *     run_mha_fwd_splitkv_mla<bfloat16, 576> (mmssai.com); d_v = 512 from the
 *     sparse-prefill example on the wmrh.cn FlashMLA深度解析 page;
 *   - query heads fold into rows per KV head (row m = s * G + g reads KV head
 *     h // G): deepseekonline.chat day-1 post, "Dynamische Sequenzoptimierung";
 *   - FP8 record, 656 bytes per token: wmrh.cn page, "FP8 KV缓存" table.
 *
 * Conventions. Pointers named *_host are host memory; every other pointer is
 * device memory on the current HIP device. The library allocates nothing and
 * keeps no pointer after a call returns (apart from work already queued on the
 * caller's stream). Calls are thread-safe; the last error message is kept per
 * thread. Every status other than MLA_OK is returned before anything is
 * launched, except MLA_ERR_HIP, which reports a failed launch.
 */
#ifndef PAGED_MLA_DECODE_AMD_MLA_H
#define PAGED_MLA_DECODE_AMD_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_PAGE_TOKENS 64        /* tokens per KV page */
#define MLA_D_QK 576              /* query/key dims: 512 latent + 64 RoPE */
#define MLA_D_V 512               /* value dims: the latent part of each cached row */
#define MLA_D_ROPE 64
#define MLA_FP8_RECORD_BYTES 656  /* 512 e4m3 codes + 4 fp32 scales + 64 bf16 RoPE */
#define MLA_META_INTS 8           /* int32 fields per row of tile_metadata */

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size/stride/alignment, inconsistent shapes */
  MLA_ERR_UNSUPPORTED = 2,        /* well-formed but outside what the kernels implement (d_qk != 576, dv != 512, ...) */
  MLA_ERR_WORKSPACE_TOO_SMALL = 3,
  MLA_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} mla_status;

typedef enum {
  MLA_KV_BF16 = 0,          /* kvcache bf16 [num_pages, 64, h_kv, 576] */
  MLA_KV_FP8_E4M3 = 1       /* kvcache uint8 [num_pages, 64, h_kv, 656]: bytes [0,512) OCP E4M3FN
                               latent codes, [512,528) four little-endian fp32 scales (scale c
                               multiplies latent dims [128c, 128c+128)), [528,656) 64 bf16 RoPE */
} mla_kv_format;

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* mla_last_error(void);

/* Library version string. */
const char* mla_version(void);

/* sizeof(mla_decode_args) as compiled into the library (binding check). */
size_t mla_decode_args_size(void);

/* Compute units of HIP device `device`, or -1 if it cannot be queried. */
int mla_device_cu_count(int device);

/*
 * Rows of tile_metadata that mla_get_metadata fills when num_parts = 0.
 * num_cus: compute units to plan for (pass 0 to query the current device).
 * Returns >= 1, or -1 on invalid arguments (see mla_last_error).
 */
int mla_num_parts(int batch, int heads_per_kv, int h_kv, int kv_format, int num_cus);

/*
 * Host tile scheduler (FlashMLA's get_mla_metadata; the wmrh.cn page, section
 * "计算流水线设计", describes a tile scheduler that spreads requests and KV
 * blocks evenly over the SMs).
 *
 * Splits the ragged work -- sequence b has ceil(L_b / 64) pages -- into
 * num_parts contiguous ranges of (sequence, page), in sequence order, with
 * near-equal cost (pages plus a fixed cost per piece of a sequence). One
 * workgroup (per row tile and KV head) runs each range on the GPU.
 *
 *   cache_seqlens_host  int32 [batch], 0 <= L_b (host memory)
 *   heads_per_kv        rows per KV head, s_q * h_q / h_kv (>= 1)
 *   num_cus             0 = query the current device; else plan for this many CUs
 *   num_parts           0 = mla_num_parts(...); else exactly this many ranges (>= 1)
 *   tile_metadata_host  int32 [num_parts][MLA_META_INTS], written. Row p:
 *                         [0] begin_b   first sequence (-1: empty range)
 *                         [1] begin_page first page of begin_b
 *                         [2] end_b     last sequence (inclusive)
 *                         [3] end_page  one past the last page of end_b
 *                         [4] begin_split index of this piece among begin_b's pieces
 *                         [5..7] 0
 *   num_splits_host     int32 [batch + 1], written: prefix sums of the number
 *                       of pieces per sequence (num_splits[0] = 0); sequence b
 *                       owns partial slots [num_splits[b], num_splits[b+1]).
 *   num_parts_out       the number of rows written (may be NULL).
 *
 * Every sequence, including L_b = 0, belongs to at least one range. The
 * metadata depends only on the lengths, heads_per_kv, h_kv, kv_format and the
 * CU count, so one result serves every layer of a decode step.
 * Capacity: tile_metadata_host must hold num_parts rows (mla_num_parts rows
 * when num_parts = 0).
 */
mla_status mla_get_metadata(const int32_t* cache_seqlens_host, int batch, int heads_per_kv, int h_kv,
                            int kv_format, int num_cus, int num_parts, int32_t* tile_metadata_host,
                            int32_t* num_splits_host, int* num_parts_out);

/*
 * Bytes of device workspace mla_decode_kvcache needs for split partials: per
 * piece of a sequence (at most batch + num_parts pieces) and row, the partial
 * O (fp32; for heads_per_kv > 64, fp16 with a power-of-two fp32 scale per 64
 * dims) and an fp32 LSE.
 * Returns 0 on invalid arguments.
 */
size_t mla_workspace_bytes(int batch, int num_parts, int heads_per_kv, int h_kv);

typedef struct mla_decode_args {
  /* q: bf16 [batch, s_q, h_q, 576]; strides in elements for (batch, s_q, head);
     the 576 dims contiguous; base and strides 16-byte aligned. */
  const void* q;
  int64_t q_stride[3];

  /* kvcache: see mla_kv_format. Strides in elements of the cache dtype (bf16:
     2 bytes, FP8 records: 1 byte) for (page, token, head); each row contiguous;
     base and strides 16-byte aligned. */
  const void* kvcache;
  int64_t kv_stride[3];
  int kv_format;
  int num_pages;              /* pages in the pool: valid block_table entries are [0, num_pages) */

  /* block_table: int32 [batch, max_blocks_per_seq] with row stride bt_stride (elements). */
  const int32_t* block_table;
  int64_t bt_stride;
  int max_blocks_per_seq;

  const int32_t* cache_seqlens;   /* int32 [batch], device */

  /* Device copies of mla_get_metadata's outputs for the same cache_seqlens. */
  const int32_t* tile_metadata;   /* [num_parts][MLA_META_INTS] */
  int num_parts;
  const int32_t* num_splits;      /* [batch + 1] */

  int batch, s_q, h_q, h_kv;
  int d_qk;                   /* must be 576 */
  int dv;                     /* must be 512 */
  int causal;                 /* nonzero: query token s of s_q reads keys t <= L_b - s_q + s */
  float softmax_scale;        /* logits are softmax_scale * <q, k> */

  void* o;                    /* out: bf16 [batch, s_q, h_q, dv], contiguous */
  float* lse;                 /* out: fp32 [batch, h_q, s_q], contiguous; natural log */

  void* workspace;            /* >= mla_workspace_bytes(batch, num_parts, s_q*h_q/h_kv, h_kv) bytes, 256-B aligned */
  size_t workspace_bytes;

  /* Optional hint: 0 = unknown, else the largest number of pieces of any
     sequence (max_b num_splits[b+1] - num_splits[b]). Accepted for
     compatibility; the current combine kernel handles any piece count and
     does not use it (results never depend on it). */
  int max_splits;

  /* Optional timing hooks (hipEvent_t or NULL): events[0] and events[1] take
     the split-KV kernel's own start and end timestamps (the kernel is launched
     with hipExtLaunchKernel), events[2] is recorded after the combine kernel. */
  void* events[3];
} mla_decode_args;

/*
 * Paged MLA decode (FlashMLA's mha_fwd_kvcache_mla / flash_mla_with_kvcache):
 * o = softmax(softmax_scale * q K^T) V and lse = ln sum exp(softmax_scale * q K^T)
 * per (sequence, query token, head), K = the sequence's cached rows in token
 * order, V = their first dv dims.
 * Launches the split-KV kernel, then the combine kernel, on `hip_stream`
 * (a hipStream_t; NULL = the null stream). Asynchronous.
 * Rows with no allowed key (L_b = 0, or causal with L_b < s_q) give o = 0,
 * lse = -inf. A block_table entry outside [0, num_pages) is never
 * dereferenced: the affected sequence's o and lse become NaN instead.
 */
mla_status mla_decode_kvcache(const mla_decode_args* args, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_MLA_DECODE_AMD_MLA_H */
