// mla_kernels.hip -- split-KV MLA decode and LSE combine for gfx950 (MI355X).
//
// What is computed: softmax attention of query rows over a sequence's cached
// 576-dim latent rows, V = their first 512 dims, with the KV range of a
// sequence cut into pieces whose partial (O, LSE) are merged by LSE. The pages
// name the two kernels (splitkv_mla and combine: wmrh.cn FlashMLA深度解析,
// section "计算流水线设计") and the running max / rescale of the online
// softmax (same page, "跷跷板调度算法突破寄存器资源限制"); the decomposition
// below is designed for CDNA4, not taken from the Hopper design.
//
// Split kernel, one workgroup = 4 wavefronts per (KV range, 16*rb-row tile,
// KV head). For each page of the range:
//   1. all 256 threads gather the page (64 tokens x 1152 B, or 64 x 656-B FP8
//      records dequantised to bf16) with 16-byte loads into LDS; the loads
//      for page i+1 are in flight while page i is computed;
//   2. each wave computes S^T = K Q^T for its 16 rows and its token group on
//      MFMA 16x16x32 bf16: A = 16 tokens x 32 dims of K read from LDS (one
//      16-byte read per lane), B = Q^T held in VGPRs for the whole range;
//   3. the online softmax runs in registers: every lane holds one query row
//      (lane % 16) and 4 tokens, so the row max needs two cross-lane steps and
//      the rescale of the O accumulator is lane-local;
//   4. O^T += V^T P^T on MFMA: P^T is the bf16 softmax tile exactly as the
//      S^T MFMA left it in registers (the token order inside a 32-token chunk
//      is permuted identically on both operands), V^T is read from the same
//      LDS page.
// Waves that split a page's tokens merge (m, l, O) through LDS at the end of
// each sequence piece. A piece that is a whole sequence writes bf16 O and LSE
// directly; otherwise it writes fp32 O / l and its LSE to its partial slot.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kLdsRow = 584;                   // bf16 per token row in LDS: 576 + 8 pad (1168 B)
constexpr int kLdsPage = kPage * kLdsRow;      // 37376 bf16 = 74752 B
constexpr int kFmtBf16 = 0;
constexpr int kFmtFp8 = 1;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;


__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));   // round to nearest even
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// OCP E4M3FN code (low 8 bits of c) -> float; S.1111.111 -> NaN.
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t c) {
  const uint32_t mag = c & 0x7Fu;
  const uint32_t e = mag >> 3, m = mag & 7u;
  float v = (e == 0) ? static_cast<float>(m) * 0.001953125f                 // m * 2^-9
                     : __uint_as_float(((e + 120u) << 23) | (m << 20));     // 2^(e-7) * (1 + m/8)
  v = (mag == 0x7Fu) ? __builtin_nanf("") : v;
  return (c & 0x80u) ? -v : v;
}

// ----------------------------------------------------------------------------
// Page loaders: global -> registers (prefetch), registers -> LDS.
// ----------------------------------------------------------------------------

template <int FMT>
struct PageLoader;

template <>
struct PageLoader<kFmtBf16> {
  static constexpr int kChunks = kPage * (kDqk * 2 / 16) / kThreads;   // 4608 / 256 = 18
  u32x4 v[kChunks];

  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int j = 0; j < kChunks; ++j) v[j] = u32x4{0u, 0u, 0u, 0u};
  }
  // base: start of (page, token 0, kv head); token stride st in bytes.
  __device__ __forceinline__ void load(const uint8_t* base, int64_t st, int tid) {
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int c = j * kThreads + tid;
      const int tok = c / 72, col = c - tok * 72;
      v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + tok * st + col * 16));
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int c = j * kThreads + tid;
      const int tok = c / 72, col = c - tok * 72;
      *reinterpret_cast<u32x4*>(lds + tok * kLdsRow + col * 8) = v[j];
    }
  }
};

// FP8 record: [0,512) e4m3 codes, [512,528) 4 fp32 scales, [528,656) 64 bf16 RoPE.
// Thread t dequantises latent chunk (t % 32) -- 16 codes, dims 16*(t%32).. --
// of tokens t/32 + 8k, k < 8, and copies RoPE chunk t % 8 of tokens t/8 + 32k, k < 2.
template <>
struct PageLoader<kFmtFp8> {
  u32x4 lat[8];
  float sc[8];
  u32x4 rope[2];

  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int k = 0; k < 8; ++k) { lat[k] = u32x4{0u, 0u, 0u, 0u}; sc[k] = 0.f; }
#pragma unroll
    for (int k = 0; k < 2; ++k) rope[k] = u32x4{0u, 0u, 0u, 0u};
  }
  __device__ __forceinline__ void load(const uint8_t* base, int64_t st, int tid) {
    const int ch = tid & 31;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint8_t* rec = base + (tid / 32 + 8 * k) * st;
      lat[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rec + ch * 16));
      sc[k] = *reinterpret_cast<const float*>(rec + 512 + 4 * (ch / 8));
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint8_t* rec = base + (tid / 8 + 32 * k) * st;
      rope[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rec + 528 + (tid & 7) * 16));
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
    const int ch = tid & 31;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int tok = tid / 32 + 8 * k;
      const uint32_t w[4] = {lat[k][0], lat[k][1], lat[k][2], lat[k][3]};
      uint32_t out[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float lo = e4m3fn_to_f32(w[i] >> (16 * h)) * sc[k];
          const float hi = e4m3fn_to_f32(w[i] >> (16 * h + 8)) * sc[k];
          out[2 * i + h] = static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
        }
      }
      u32x4* dst = reinterpret_cast<u32x4*>(lds + tok * kLdsRow + ch * 16);
      dst[0] = u32x4{out[0], out[1], out[2], out[3]};
      dst[1] = u32x4{out[4], out[5], out[6], out[7]};
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int tok = tid / 8 + 32 * k;
      *reinterpret_cast<u32x4*>(lds + tok * kLdsRow + 512 + (tid & 7) * 8) = rope[k];
    }
  }
};

__device__ __forceinline__ float wave_max16(float v) {
  // reduce over the 4 lanes that share lane % 16
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float wave_sum16(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// ----------------------------------------------------------------------------
// Split-KV kernel
// ----------------------------------------------------------------------------

template <int RB, int TG, int FMT>
__global__ void __launch_bounds__(kThreads) splitkv_kernel(DecodeParams p) {
  static_assert(RB * TG == kWaves, "4 waves per workgroup");
  constexpr int NT = 4 / TG;          // 16-token tiles per wave per page
  constexpr int M_TILE = 16 * RB;

  __shared__ __attribute__((aligned(16))) uint16_t lds[kLdsPage];
  __shared__ float red_m[kWaves][16];
  __shared__ float red_l[kWaves][16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int rb = wave % RB, tg = wave / RB;
  const int r16 = lane & 15, q4 = lane >> 4;

  // Workgroup i runs on XCD i % 8: give each XCD a contiguous block of
  // logical ids so the row tiles of one KV range share that XCD's L2.
  const int per_xcd = gridDim.x / 8;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= p.grid_wgs) return;
  const int m_tiles = (p.rows + M_TILE - 1) / M_TILE;
  const int mt = logical % m_tiles;
  const int kvh = (logical / m_tiles) % p.h_kv;
  const int part = logical / (m_tiles * p.h_kv);

  const int32_t* meta = p.meta + part * kMetaInts;
  const int begin_b = meta[0];
  if (begin_b < 0 || begin_b >= p.batch) return;
  const int begin_page = meta[1];
  const int end_b = min(meta[2], p.batch - 1);
  const int end_page = meta[3];
  const int split0 = meta[4];

  const int row = mt * M_TILE + rb * 16 + r16;   // this lane's query row within the KV head
  const bool row_ok = row < p.rows;
  const int s_idx = row_ok ? row / p.group : 0;
  const int head = kvh * p.group + (row_ok ? row % p.group : 0);

  const int max_len = p.max_blocks * kPage;
  PageLoader<FMT> ld;

  for (int b = begin_b; b <= end_b; ++b) {
    int L = p.seqlens[b];
    L = L < 0 ? 0 : (L > max_len ? max_len : L);
    const int np = (L + kPage - 1) / kPage;
    const int pg0 = (b == begin_b) ? max(begin_page, 0) : 0;
    const int pg1 = (b == end_b) ? min(end_page, np) : np;
    const int split_idx = (b == begin_b) ? split0 : 0;
    const int slot0 = p.num_splits[b];
    const int nsplit = p.num_splits[b + 1] - slot0;
    const int last_allowed_base = p.causal ? (L - p.s_q) : (L - 1);   // + s_idx if causal
    const int last_allowed = p.causal ? last_allowed_base + s_idx : last_allowed_base;

    // Q^T operand: 18 chunks of 8 dims (dims 32c + 8*q4 .. +8) of this lane's row.
    bf16x8 qf[18];
    {
      const uint16_t* qrow = p.q + b * p.q_sb + s_idx * p.q_ss + head * p.q_sh;
#pragma unroll
      for (int c = 0; c < 18; ++c) {
        u32x4 v = row_ok ? *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * q4) : u32x4{0u, 0u, 0u, 0u};
        qf[c] = __builtin_bit_cast(bf16x8, v);
      }
    }

    float m_run = kNegInf, l_run = 0.f;
    f32x4 acc[32];
#pragma unroll
    for (int d = 0; d < 32; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool bad = false;

    const uint8_t* kv_head = p.kv + kvh * p.kv_sh;
    auto page_ptr = [&](int pi, bool& ok) -> const uint8_t* {
      const int pg = p.block_table[static_cast<int64_t>(b) * p.bt_stride + pi];
      ok = (pg >= 0 && pg < p.num_pages);
      return kv_head + static_cast<int64_t>(ok ? pg : 0) * p.kv_sp;
    };

    if (pg0 < pg1) {
      bool ok;
      const uint8_t* ptr = page_ptr(pg0, ok);
      if (ok) ld.load(ptr, p.kv_st, tid); else { ld.clear(); bad = true; }
    }

    for (int pi = pg0; pi < pg1; ++pi) {
      __syncthreads();                 // every wave is done with the previous page
      ld.store(lds, tid);
      __syncthreads();
      if (pi + 1 < pg1) {
        bool ok;
        const uint8_t* ptr = page_ptr(pi + 1, ok);
        if (ok) ld.load(ptr, p.kv_st, tid); else { ld.clear(); bad = true; }
      }

      // ---- S^T tiles: rows = tokens, columns = query rows --------------------
      f32x4 s[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint16_t* krow = lds + (16 * (tg * NT + t) + r16) * kLdsRow + 8 * q4;
#pragma unroll
        for (int c = 0; c < 18; ++c) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 32 * c);
          s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[c], s[t], 0, 0, 0);
        }
      }

      // ---- mask, online softmax ----------------------------------------------
      const int tok_base = pi * kPage + 16 * tg * NT + 4 * q4;
      float mx = kNegInf;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = tok_base + 16 * t + i;
          const bool ok = tok < L && tok <= last_allowed;
          const float v = ok ? s[t][i] * p.scale_log2 : kNegInf;
          s[t][i] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = wave_max16(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = fast_exp2(s[t][i] - m_use);
          s[t][i] = e;
          psum += e;
        }
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int d = 0; d < 32; ++d) acc[d] *= alpha;

      // ---- O^T += V^T P^T ----------------------------------------------------
      if constexpr (NT >= 2) {
#pragma unroll
        for (int u = 0; u < NT / 2; ++u) {
          bf16x8 pb;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            pb[j] = static_cast<__bf16>(s[2 * u][j]);
            pb[4 + j] = static_cast<__bf16>(s[2 * u + 1][j]);
          }
          const int tok0 = 16 * (tg * NT + 2 * u) + 4 * q4;   // k-slots j<4: tok0+j ; j>=4: tok0+16+j-4
          const __bf16* vb = reinterpret_cast<const __bf16*>(lds);
#pragma unroll
          for (int d = 0; d < 32; ++d) {
            const int dim = 16 * d + r16;
            bf16x8 a;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              a[j] = vb[(tok0 + j) * kLdsRow + dim];
              a[4 + j] = vb[(tok0 + 16 + j) * kLdsRow + dim];
            }
            acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, acc[d], 0, 0, 0);
          }
        }
      } else {
        s16x4 pb;
#pragma unroll
        for (int j = 0; j < 4; ++j) pb[j] = static_cast<short>(f32_to_bf16(s[0][j]));
        const int tok0 = 16 * tg + 4 * q4;
#pragma unroll
        for (int d = 0; d < 32; ++d) {
          const int dim = 16 * d + r16;
          s16x4 a;
#pragma unroll
          for (int j = 0; j < 4; ++j) a[j] = static_cast<short>(lds[(tok0 + j) * kLdsRow + dim]);
          acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, acc[d], 0, 0, 0);
        }
      }
    }

    // ---- merge the token groups, then write -----------------------------------
    float l_row = wave_sum16(l_run);
    float m_fin = m_run;
    if constexpr (TG > 1) {
      __syncthreads();                 // all waves done with the LDS page
      if (lane < 16) {
        red_m[wave][r16] = m_run;
        red_l[wave][r16] = l_row;
      }
      __syncthreads();
      float M = kNegInf;
#pragma unroll
      for (int k = 0; k < TG; ++k) M = fmaxf(M, red_m[rb + RB * k][r16]);
      const float M_use = (M == kNegInf) ? 0.f : M;
      float ltot = 0.f;
#pragma unroll
      for (int k = 0; k < TG; ++k) ltot += red_l[rb + RB * k][r16] * fast_exp2(red_m[rb + RB * k][r16] - M_use);
      const float f = fast_exp2(m_run - M_use);
#pragma unroll
      for (int d = 0; d < 32; ++d) acc[d] *= f;
      l_row = ltot;
      m_fin = M;
      // Sum the TG accumulators of each row block through LDS (fp32 [16 rows][512]).
      float* red = reinterpret_cast<float*>(lds);
      auto slot_ptr = [&](int slot) { return red + slot * (16 * 512); };
      auto put = [&](float* base) {
#pragma unroll
        for (int d = 0; d < 32; ++d)
          *reinterpret_cast<f32x4*>(base + r16 * 512 + 16 * d + 4 * q4) = acc[d];
      };
      auto add = [&](const float* base) {
#pragma unroll
        for (int d = 0; d < 32; ++d) acc[d] += *reinterpret_cast<const f32x4*>(base + r16 * 512 + 16 * d + 4 * q4);
      };
      if constexpr (TG == 4) {                 // RB == 1: waves 0..3 hold the same rows
        if (wave >= 2) put(slot_ptr(wave - 2));
        __syncthreads();
        if (wave < 2) add(slot_ptr(wave));
        __syncthreads();
        if (wave == 1) put(slot_ptr(0));
        __syncthreads();
        if (wave == 0) add(slot_ptr(0));
      } else {                                  // TG == 2, RB == 2
        if (tg == 1) put(slot_ptr(rb));
        __syncthreads();
        if (tg == 0) add(slot_ptr(rb));
      }
    }

    if (tg == 0 && row_ok) {
      const bool valid = !bad;
      const float inv = (l_row > 0.f) ? 1.f / l_row : 0.f;
      float lse = (l_row > 0.f) ? (m_fin + __log2f(l_row)) * kLn2 : kNegInf;
      if (!valid) lse = __builtin_nanf("");
      if (nsplit == 1) {
        uint16_t* orow = p.o + ((static_cast<int64_t>(b) * p.s_q + s_idx) * p.h_q + head) * kDv + 4 * q4;
#pragma unroll
        for (int d = 0; d < 32; ++d) {
          u32x2 w;
          const float x0 = valid ? acc[d][0] * inv : __builtin_nanf("");
          const float x1 = valid ? acc[d][1] * inv : __builtin_nanf("");
          const float x2 = valid ? acc[d][2] * inv : __builtin_nanf("");
          const float x3 = valid ? acc[d][3] * inv : __builtin_nanf("");
          w[0] = static_cast<uint32_t>(f32_to_bf16(x0)) | (static_cast<uint32_t>(f32_to_bf16(x1)) << 16);
          w[1] = static_cast<uint32_t>(f32_to_bf16(x2)) | (static_cast<uint32_t>(f32_to_bf16(x3)) << 16);
          *reinterpret_cast<u32x2*>(orow + 16 * d) = w;
        }
        if (q4 == 0) p.lse[(static_cast<int64_t>(b) * p.h_q + head) * p.s_q + s_idx] = lse;
      } else {
        const int slot = slot0 + split_idx;
        if (slot >= 0 && slot < p.max_slots && split_idx < nsplit) {
          float* prow = p.part_o + ((static_cast<int64_t>(slot) * p.h_kv + kvh) * p.rows + row) * kDv + 4 * q4;
#pragma unroll
          for (int d = 0; d < 32; ++d) {
            f32x4 v = acc[d] * inv;
            if (!valid) v = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
            *reinterpret_cast<f32x4*>(prow + 16 * d) = v;
          }
          if (q4 == 0) p.part_lse[(static_cast<int64_t>(slot) * p.h_kv + kvh) * p.rows + row] = lse;
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Combine: LSE = ln sum_i exp(LSE_i), O = sum_i exp(LSE_i - LSE) O_i
// One wave per (sequence, row, KV head); lane l owns dims 8l .. 8l+7.
// ----------------------------------------------------------------------------

__global__ void __launch_bounds__(kThreads) combine_kernel(DecodeParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.x, kvh = blockIdx.z;
  const int row = blockIdx.y * kWaves + wave;
  if (row >= p.rows) return;
  const int slot0 = p.num_splits[b];
  const int n = p.num_splits[b + 1] - slot0;
  if (n <= 1) return;
  const int s_idx = row / p.group;
  const int head = kvh * p.group + row % p.group;
  uint16_t* orow = p.o + ((static_cast<int64_t>(b) * p.s_q + s_idx) * p.h_q + head) * kDv + 8 * lane;
  float* lse_out = p.lse + (static_cast<int64_t>(b) * p.h_q + head) * p.s_q + s_idx;
  if (slot0 < 0 || slot0 + n > p.max_slots) {
    const u32x4 nan4 = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
    *reinterpret_cast<u32x4*>(orow) = nan4;
    if (lane == 0) *lse_out = __builtin_nanf("");
    return;
  }
  const int64_t stride = static_cast<int64_t>(p.h_kv) * p.rows;             // slots apart
  const float* lse_in = p.part_lse + static_cast<int64_t>(slot0) * stride + static_cast<int64_t>(kvh) * p.rows + row;
  const float* o_in = p.part_o + (static_cast<int64_t>(slot0) * stride + static_cast<int64_t>(kvh) * p.rows + row) * kDv
                      + 8 * lane;

  float mx = kNegInf;
  for (int i = lane; i < n; i += 64) mx = fmaxf(mx, lse_in[i * stride]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  const bool any = mx != kNegInf;
  const float mxu = any ? mx : 0.f;
  float sum = 0.f;
  for (int i = lane; i < n; i += 64) sum += __expf(lse_in[i * stride] - mxu);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  const float lse = any ? mxu + __logf(sum) : kNegInf;

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (any) {
    for (int i = 0; i < n; ++i) {
      const float w = __expf(lse_in[i * stride] - lse);
      const f32x4 a = *reinterpret_cast<const f32x4*>(o_in + i * stride * kDv);
      const f32x4 c = *reinterpret_cast<const f32x4*>(o_in + i * stride * kDv + 4);
      if (w != 0.f) {
        acc[0] += w * a[0]; acc[1] += w * a[1]; acc[2] += w * a[2]; acc[3] += w * a[3];
        acc[4] += w * c[0]; acc[5] += w * c[1]; acc[6] += w * c[2]; acc[7] += w * c[3];
      }
    }
  }
  u32x4 outw;
  outw[0] = static_cast<uint32_t>(f32_to_bf16(acc[0])) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
  outw[1] = static_cast<uint32_t>(f32_to_bf16(acc[2])) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
  outw[2] = static_cast<uint32_t>(f32_to_bf16(acc[4])) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
  outw[3] = static_cast<uint32_t>(f32_to_bf16(acc[6])) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
  *reinterpret_cast<u32x4*>(orow) = outw;
  if (lane == 0) *lse_out = lse;
}

template <int RB, int TG>
hipError_t launch_split(const DecodeParams& p, int kv_format, int grid, hipStream_t stream) {
  if (kv_format == kFmtFp8)
    hipLaunchKernelGGL((splitkv_kernel<RB, TG, kFmtFp8>), dim3(grid), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((splitkv_kernel<RB, TG, kFmtBf16>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, const Plan& plan, int kv_format, hipStream_t stream,
                         void* const events[3]) {
  const int grid = (p.grid_wgs + 7) / 8 * 8;
  hipError_t err;
  if (events && events[0]) {
    err = hipEventRecord(static_cast<hipEvent_t>(events[0]), stream);
    if (err != hipSuccess) return err;
  }
  if (plan.rb == 1) err = launch_split<1, 4>(p, kv_format, grid, stream);
  else if (plan.rb == 2) err = launch_split<2, 2>(p, kv_format, grid, stream);
  else err = launch_split<4, 1>(p, kv_format, grid, stream);
  if (err != hipSuccess) return err;
  if (events && events[1]) {
    err = hipEventRecord(static_cast<hipEvent_t>(events[1]), stream);
    if (err != hipSuccess) return err;
  }
  const dim3 cgrid(p.batch, (p.rows + kWaves - 1) / kWaves, p.h_kv);
  hipLaunchKernelGGL(combine_kernel, cgrid, dim3(kThreads), 0, stream, p);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (events && events[2]) {
    err = hipEventRecord(static_cast<hipEvent_t>(events[2]), stream);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace mla
