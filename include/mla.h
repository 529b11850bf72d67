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
 *   max_blocks_per_seq  block-table entries per sequence: every L_b must be
 *                       <= 64 * max_blocks_per_seq, else
 *                       MLA_ERR_INVALID_ARGUMENT. 0 = not checked here (the
 *                       decode then returns NaN o and lse for such a sequence;
 *                       it never reads past the block-table row).
 *   num_cus             0 = query the current device; else plan for this many CUs
 *   num_parts           0 = mla_num_parts(...); else exactly this many ranges (>= 1)
 *   tile_metadata_host  int32 [num_parts][MLA_META_INTS], written. Row p:
 *                         [0] begin_b   first sequence (-1: empty range)
 *                         [1] begin_page first page of begin_b
 *                         [2] end_b     last sequence (inclusive)
 *                         [3] end_page  one past the last page of end_b
 *                         [4] begin_split index of this piece among begin_b's pieces
 *                         [5] checksum of the page counts of sequences
 *                             begin_b .. end_b (0 for an empty range)
 *                         [6] batch
 *                         [7] 0
 *                       The decode recomputes [5] and [6] from its own lengths
 *                       and batch; a range whose values differ (metadata built
 *                       for other page counts) gives NaN o and lse for its
 *                       sequences instead of a silently wrong result.
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
                            int kv_format, int max_blocks_per_seq, int num_cus, int num_parts,
                            int32_t* tile_metadata_host, int32_t* num_splits_host, int* num_parts_out);

/*
 * The tile scheduler on the device, for lengths that live in device memory
 * (no copy to the host, no synchronisation: the call only queues one kernel
 * on hip_stream). Its outputs are those of mla_get_metadata, bit for bit, for
 * the same lengths, heads_per_kv, h_kv, kv_format and number of ranges.
 *   cache_seqlens       int32 [batch], device memory
 *   heads_per_kv, h_kv, kv_format, num_cus, num_parts   as for mla_get_metadata
 *   tile_metadata       int32 [num_parts][MLA_META_INTS], device memory, written
 *   num_splits          int32 [batch + 1], device memory, written
 *   num_parts_out       the number of rows written (host memory; may be NULL)
 * Limits, checked before the launch (else MLA_ERR_UNSUPPORTED): batch <= 1023
 * and num_parts <= 1024. Lengths are not checked (the device cannot return a
 * status): a negative length is scheduled as an empty sequence, and a
 * sequence of more than 2^20 pages (67,108,864 tokens) makes every range
 * empty and every piece count 0; the decode reports the sequences concerned
 * as NaN, as it does for lengths past the block table.
 */
mla_status mla_get_metadata_device(const int32_t* cache_seqlens, int batch, int heads_per_kv, int h_kv,
                                   int kv_format, int num_cus, int num_parts, int32_t* tile_metadata,
                                   int32_t* num_splits, int* num_parts_out, void* hip_stream);

/*
 * Tile-scheduler metadata for token-level sparse decode (get_mla_metadata
 * with topk on the wmrh.cn FlashMLA深度解析 page, "解码阶段使用示例"): the
 * batch * s_q (sequence, query token) pairs are scheduled as sequences of
 * topk entries with h_q / h_kv query rows each. Fills tile_metadata_host
 * [num_parts][MLA_META_INTS] and num_splits_host [batch * s_q + 1] as
 * mla_get_metadata does for those sequences (num_parts = 0: mla_num_parts(
 * batch * s_q, h_q / h_kv, h_kv, kv_format, num_cus) rows). The metadata
 * depends only on these sizes: one result serves every step with the same
 * batch, s_q and topk.
 */
mla_status mla_get_metadata_sparse(int batch, int s_q, int topk, int h_q, int h_kv, int kv_format, int num_cus,
                                   int num_parts, int32_t* tile_metadata_host, int32_t* num_splits_host,
                                   int* num_parts_out);

/* Bytes of device workspace a sparse mla_decode_kvcache call needs (0 on invalid arguments). */
size_t mla_workspace_bytes_sparse(int batch, int s_q, int num_parts, int h_q, int h_kv);

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
     sequence (max_b num_splits[b+1] - num_splits[b]). It selects the combine
     kernel's shape: when some sequence has more than 8 pieces (for tiles of at
     most 64 rows also when the hint is 0), extra workgroups find those
     sequences on the device and merge them in small slices, 64 pieces per
     round of loads. That changes the order in which such a sequence's pieces
     are merged, so results for different hints agree to rounding, not bit for
     bit; any hint gives correct results, and the same hint always gives the
     same bits. */
  int max_splits;

  /* Optional timing hooks (hipEvent_t or NULL): events[0] and events[1] take
     the split-KV kernel's own start and end timestamps (the kernel is launched
     with hipExtLaunchKernel), events[2] is recorded after the combine kernel. */
  void* events[3];

  /* Token-level sparse decode (the indices argument of flash_mla_with_kvcache
     and the topk of get_mla_metadata on the wmrh.cn FlashMLA深度解析 page,
     "解码阶段使用示例"; "token级稀疏注意力" in "实际性能表现与优化效果").
     NULL: dense decode. Otherwise int32 [batch, s_q, topk] (last dim
     contiguous, strides in elements): query token s of sequence b attends only
     to the cached positions indices[b, s, 0..topk) of sequence b (each found
     through block_table like any cached token); -1 is padding and selects
     nothing; a position listed twice counts twice; with causal, positions past
     L_b - s_q + s are dropped. An entry outside [-1, L_b) gives NaN o and lse
     for that query token. Every (b, s) pair is then scheduled on its own: the
     metadata comes from mla_get_metadata_sparse, the workspace size from
     mla_workspace_bytes_sparse. Needs q's sequence stride to equal s_q times
     its token stride, and the KV pool of a head to span less than 2^31 bytes. */
  const int32_t* indices;
  int64_t idx_stride[2];
  int topk;

  /* Optional separate V cache (the vcache_ argument of mha_fwd_kvcache_mla,
     num_blocks x page_block_size x num_heads_k x head_size_v: mmssai.com,
     "代码解读：flash_api.cpp 核心逻辑"). NULL: V is the first dv dims of each
     cached key row. Otherwise bf16 [num_pages, 64, h_kv, dv]: the value of
     cached token t is its row here, at the same page and slot as its key (the
     same block_table); strides in elements for (page, token, head), each row
     contiguous, base and strides 16-byte aligned, a 64-token page spanning less
     than 2 GiB. Needs kv_format MLA_KV_BF16 and dense decode (indices NULL);
     the workspace size is unchanged. Runs on 64-row tiles (ceil(s_q * h_q /
     h_kv / 64) workgroups per range and KV head). */
  const void* vcache;
  int64_t vc_stride[3];
} mla_decode_args;

/*
 * Paged MLA decode (FlashMLA's mha_fwd_kvcache_mla / flash_mla_with_kvcache):
 * o = softmax(softmax_scale * q K^T) V and lse = ln sum exp(softmax_scale * q K^T)
 * per (sequence, query token, head), K = the sequence's cached rows in token
 * order, V = their first dv dims.
 * Launches the split-KV kernel, then the combine kernel, on `hip_stream`
 * (a hipStream_t; NULL = the null stream). Asynchronous.
 * Rows with no allowed key (L_b = 0, or causal with L_b < s_q) give o = 0,
 * lse = -inf. Data-dependent errors that only the device sees are reported in
 * the outputs, never by a fault: a block_table entry outside [0, num_pages)
 * is never dereferenced, a length outside [0, 64 * max_blocks_per_seq] never
 * reads past the block-table row, and metadata built for other page counts
 * is detected (tile_metadata fields 5 and 6); each of these turns the o and
 * lse of the affected sequences into NaN.
 */
mla_status mla_decode_kvcache(const mla_decode_args* args, void* hip_stream);

/* Capacity of the library's static device scratch (bytes per device). */
#define MLA_SCRATCH_BYTES (128u << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * decode as mla_decode_kvcache, with the split partials in a static device
 * array of MLA_SCRATCH_BYTES that the library holds on each device it runs on
 * until the process ends, so nothing is allocated: no hipMalloc, no hipFree,
 * no allocating library call. args->workspace and args->workspace_bytes are
 * ignored; every other field means what it does for mla_decode_kvcache, and
 * the caller still supplies the inputs, o and lse.
 * A call whose workspace (mla_workspace_bytes for its batch, num_parts,
 * s_q * h_q / h_kv and h_kv) exceeds MLA_SCRATCH_BYTES returns
 * MLA_ERR_WORKSPACE_TOO_SMALL before anything is launched.
 * All calls on one device share that device's scratch, which keeps the last
 * call's contents (nothing in it needs to start at zero): calls that may
 * overlap on one device -- on different streams without ordering, or from
 * several threads -- race and give wrong results. Order them on one stream.
 */
mla_status mla_decode_kvcache_noalloc(const mla_decode_args* args, void* hip_stream);

/*
 * Sparse prefill (flash_mla_sparse_fwd(q, kv, indices, sm_scale, d_v=512) on
 * the wmrh.cn FlashMLA深度解析 page, "稀疏预填充使用"): query token s, head h
 * attends to the rows indices[s, h / (h_q / h_kv), 0..topk) of kv's KV head
 * h / (h_q / h_kv); o = softmax(softmax_scale * q K^T) V with V the first dv
 * dims of the listed rows, lse = ln sum exp(softmax_scale * q K^T). -1 is
 * padding; a row listed twice counts twice; an entry outside [-1, s_kv)
 * gives NaN o and lse for that (token, KV head); a token with no listed row
 * gives o = 0, lse = -inf. No causal mask (the list decides).
 * Every query token is scheduled as a sequence of topk entries: tile_metadata
 * and num_splits are device copies of mla_get_metadata_sparse(s_q, 1, topk,
 * h_q, h_kv, MLA_KV_BF16, ...) (one result serves every call with the same
 * s_q, topk, h_q and h_kv), the workspace holds at least
 * mla_workspace_bytes_sparse(s_q, 1, num_parts, h_q, h_kv) bytes.
 */
typedef struct mla_sparse_prefill_args {
  /* q: bf16 [s_q, h_q, 576]; strides in elements for (token, head); the 576
     dims contiguous; base and strides 16-byte aligned. */
  const void* q;
  int64_t q_stride[2];
  /* kv: bf16 [s_kv, h_kv, 576] (latent dims 0..511 are also V); strides in
     elements for (row, head); rows contiguous; base and strides 16-byte
     aligned; the rows of one head span less than 2^31 bytes. */
  const void* kv;
  int64_t kv_stride[2];
  /* indices: int32 [s_q, h_kv, topk], device; strides in elements for
     (token, KV head); the last dim contiguous. */
  const int32_t* indices;
  int64_t idx_stride[2];
  int s_q, s_kv, h_q, h_kv, topk;
  int d_qk;                   /* must be 576 */
  int dv;                     /* must be 512 */
  float softmax_scale;

  const int32_t* tile_metadata;   /* [num_parts][MLA_META_INTS], device */
  int num_parts;
  const int32_t* num_splits;      /* [s_q + 1], device */

  void* o;                    /* out: bf16 [s_q, h_q, dv], contiguous */
  float* lse;                 /* out: fp32 [s_q, h_q], contiguous; natural log */
  void* workspace;            /* 256-byte aligned */
  size_t workspace_bytes;
  int max_splits;             /* as in mla_decode_args */
  void* events[3];            /* as in mla_decode_args */
} mla_sparse_prefill_args;

/* sizeof(mla_sparse_prefill_args), for bindings that check their layout. */
size_t mla_sparse_prefill_args_size(void);

/*
 * Launches the sparse prefill (the split kernel over the listed rows, then the
 * combine kernel) on `hip_stream`. Asynchronous. Argument errors return a
 * status before anything is launched; errors in the index values are reported
 * in the outputs as above, never by a fault.
 */
mla_status mla_sparse_prefill_fwd(const mla_sparse_prefill_args* args, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_MLA_DECODE_AMD_MLA_H */
