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
// Split kernel: one workgroup = 4 wavefronts per (KV range, row tile, KV head).
//   * Pages stream into a two-slot LDS ring with buffer_load_dwordx4 ... lds:
//     64 lanes x 16 B land in 1 KB of LDS per instruction, so no VGPRs hold
//     in-flight data, and page i+1 loads while page i is computed (its loads
//     are issued right after the barrier that frees the slot). The 16-byte
//     chunks of a 1152-byte token row are XOR-swizzled (chunk ^ f(token)) so
//     both the K reads and the transposed V reads below hit distinct banks.
//   * FP8 pages (656-byte records) stream raw into the ring; one LDS pass turns
//     the e4m3 codes into bf16 (exact: 4 significant bits fit in 8) and copies
//     RoPE and the per-128-dim scales. The scales are applied in fp32 on the
//     logits (per scale group) and folded into P for the PV product, so K and V
//     enter the MFMA without rounding.
//   * Each wave owns 16 query rows (lane % 16) and a token group of every page:
//     S^T = K Q^T on MFMA 16x16x32 bf16 (A = 16 tokens x 32 dims of K from LDS,
//     one 16-byte read; B = Q^T kept in VGPRs), online softmax in registers
//     (two cross-lane steps for the row max; the O rescale is lane-local), then
//     O^T += V^T P^T on MFMA with P^T straight from the S^T registers and V^T
//     from LDS through ds_read_b64_tr_b16 (the transposing LDS read of gfx950).
//   * Waves that split a page's tokens merge (m, l, O) through LDS at the end of
//     a sequence piece. A piece that is the whole sequence writes bf16 O and LSE;
//     otherwise fp32 O / l and its LSE go to the piece's partial slot.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <mutex>
#include <type_traits>
#include <unordered_map>

#include "device_common.h"
#include "kernels.h"

namespace mla {
namespace {

using namespace dev;

// ----------------------------------------------------------------------------
// Split-KV kernel
// ----------------------------------------------------------------------------

// Issue the direct loads of one page (bf16 rows, or raw FP8 records) from
// `src` (`extent` bytes: 64 token strides) into the LDS slot `dst`: MUBUF
// loads to LDS (buffer_load_dwordx4 ... lds), 16 bytes per lane at the
// per-lane offsets `ld_off`. Unlike the FLAT form they count on vmcnt only,
// so the LDS waits of the compute that follows never wait for them.
template <int FMT>
__device__ __forceinline__ void issue_page(const uint8_t* src, int extent, uint8_t* dst, const uint32_t* ld_off,
                                           int wave) {
  constexpr int kLoads = (FMT == kFmtFp8) ? kFp8Loads : kBf16Loads;
  constexpr int kLoadsPerWave = (kLoads + kWaves - 1) / kWaves;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), 0, extent, 0x00020000);
#pragma unroll
  for (int j = 0; j < kLoadsPerWave; ++j) {
    const int k = wave + kWaves * j;
    if (k < kLoads)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, dst + 1024 * k), 16, ld_off[j], 0, 0,
                                               kPageLoadPolicy);
  }
}

// One page of the pipeline. `cur` holds the page (bf16 rows, or raw FP8
// records), `conv` (FP8 only) holds the converted bf16 page and its scales;
// the next page is in flight into the other ring slot. The regions are
// disjoint; the restrict qualifiers let the compiler see that the reads of
// this page never touch the loads in flight.
template <int TG, int FMT>
__device__ __forceinline__ void page_step(uint8_t* __restrict__ cur, uint8_t* __restrict__ conv,
                                          const Lane& ln, int L, int last_allowed,
                                          int pi, bool this_ok, float scale_log2, const bf16x8 (&qf)[18],
                                          f32x4 (&acc)[32], float& m_run, float& l_run) {
  constexpr int NT = 4 / TG;
  constexpr bool kFp8 = (FMT == kFmtFp8);
  constexpr int NG = kFp8 ? 4 : 1;    // scale groups folded into P
  const int tid = ln.tid, tg = ln.tg, r16 = ln.r16, q4 = ln.q4;

  const int valid = min(L - pi * kPage, kPage);      // tokens of this page inside the sequence
  const uint8_t* page;
  const float* scale_tab = nullptr;
  if constexpr (kFp8) {
    // raw records -> bf16 page (codes exact), RoPE copy, scales; tail tokens and a bad page -> 0
    float* scales = reinterpret_cast<float*>(conv + kPageBytes);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int item = tid + kThreads * j;
      const int t = item >> 5, ch = item & 31;
      const u32x4 w = *reinterpret_cast<const u32x4*>(cur + t * kFp8Record + 16 * ch);
      const bool keep = this_ok && t < valid;
      u32x4 lo, hi;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t a = w[i], c = w[i + 2];
        uint32_t x0, x1, y0, y1;
        e4m3x4_to_bf16(a, x0, x1);
        e4m3x4_to_bf16(c, y0, y1);
        lo[2 * i] = x0;
        lo[2 * i + 1] = x1;
        hi[2 * i] = y0;
        hi[2 * i + 1] = y1;
      }
      if (!keep) {
        lo = u32x4{0u, 0u, 0u, 0u};
        hi = lo;
      }
      *reinterpret_cast<u32x4*>(conv + chunk_off(t, 2 * ch)) = lo;
      *reinterpret_cast<u32x4*>(conv + chunk_off(t, 2 * ch + 1)) = hi;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int item = tid + kThreads * j;
      const int t = item >> 3, rr = item & 7;
      u32x4 w = *reinterpret_cast<const u32x4*>(cur + t * kFp8Record + 528 + 16 * rr);
      if (!(this_ok && t < valid)) w = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(conv + chunk_off(t, 64 + rr)) = w;
    }
    {
      const int t = tid >> 2, c = tid & 3;
      const float sv = *reinterpret_cast<const float*>(cur + t * kFp8Record + 512 + 4 * c);
      scales[tid] = (this_ok && t < valid) ? sv : 0.f;
    }
    lds_barrier_keep_loads();
    page = conv;
    scale_tab = scales;
  } else {
    if (valid < kPage || !this_ok) {
      // zero the rows past the sequence end (all rows of a bad page) so that
      // stale bytes never meet a zero weight in P V (0 * NaN = NaN)
      const int z0 = this_ok ? valid : 0;
      // (asm stores: see merge_put)
      for (int x = z0 * kRowBytes + 16 * tid; x < kPageBytes; x += 16 * kThreads)
        lds_store16(lds_addr(cur + x), f32x4{0.f, 0.f, 0.f, 0.f});
      lds_barrier_keep_loads();
    }
    page = cur;
  }

  // ---- S^T tiles: rows = tokens, columns = query rows --------------------------
  // K chunk 4c + q4 of token row T sits at 16 * ((4c + q4) ^ swz(T)); with
  // c = 2k + h that is 128k + 16 * ((4h + q4) ^ swz): two lane bases plus an
  // immediate offset per read.
  const int kb0 = 16 * ((q4) ^ ln.sw_k), kb1 = 16 * ((4 + q4) ^ ln.sw_k);
  f32x4 s[NT];
  if constexpr (kFp8) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint8_t* krow = page + (16 * (tg * NT + t) + r16) * kRowBytes;
      f32x4 grp[5];
#pragma unroll
      for (int g = 0; g < 5; ++g) grp[g] = f32x4{0.f, 0.f, 0.f, 0.f};
      // round-robin over the scale groups so consecutive MFMAs are independent
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int g = 0; g < 5; ++g) {
          if (g == 4 && j >= 2) continue;
          const int c = (g < 4) ? 4 * g + j : 16 + j;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 128 * (c >> 1) + ((c & 1) ? kb1 : kb0));
          grp[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[c], grp[g], 0, 0, 0);
        }
      }
      // logits of tokens 16*tile + 4*q4 + i: RoPE part + scale-weighted latent groups
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 sc = *reinterpret_cast<const f32x4*>(scale_tab + 4 * (16 * (tg * NT + t) + 4 * q4 + i));
        s[t][i] = grp[4][i] + sc[0] * grp[0][i] + sc[1] * grp[1][i] + sc[2] * grp[2][i] + sc[3] * grp[3][i];
      }
    }
  } else {
    // NT tiles x CH partial chains = 4 independent accumulations in flight. The K
    // operands are read in inline asm, KB chunks per block, each block waited inside
    // it: a plain LDS read here made the compiler wait for the next page's loads in
    // flight (it cannot tell the two slots of the ring apart). The MFMAs of a block
    // run while the next block's reads are in flight.
    constexpr int CH = (NT >= 4) ? 1 : 4 / NT;
    constexpr int KB = (NT >= 4) ? 2 : 3;            // chunks per read block (18 % KB == 0)
    f32x4 part[NT][CH];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int h = 0; h < CH; ++h) part[t][h] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t kbase = lds_addr(page + (16 * tg * NT + r16) * kRowBytes);
    auto kaddr = [&](int c, int t) -> uint32_t {
      return kbase + 16 * t * kRowBytes + 128 * (c >> 1) + ((c & 1) ? kb1 : kb0);
    };
#pragma unroll
    for (int c0 = 0; c0 < 18; c0 += KB) {
      bf16x8 kv[KB * NT];
      uint32_t ka[KB * NT];
#pragma unroll
      for (int j = 0; j < KB; ++j)
#pragma unroll
        for (int t = 0; t < NT; ++t) ka[j * NT + t] = kaddr(c0 + j, t);
      lds_read16_block<KB * NT>(ka, kv);
#pragma unroll
      for (int j = 0; j < KB; ++j)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          part[t][(c0 + j) % CH] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[j * NT + t], qf[c0 + j], part[t][(c0 + j) % CH], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      s[t] = part[t][0];
#pragma unroll
      for (int h = 1; h < CH; ++h) s[t] += part[t][h];
    }
  }

  // ---- mask, online softmax ----------------------------------------------------
  const int tok_base = pi * kPage + 16 * tg * NT + 4 * q4;
  float mx = kNegInf;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = tok_base + 16 * t + i;
      const bool ok = tok < L && tok <= last_allowed;
      const float v = ok ? s[t][i] * scale_log2 : kNegInf;
      s[t][i] = v;
      mx = fmaxf(mx, v);
    }
  }
  mx = max4lanes(mx);
  if (mx > m_run + kRescaleSlack) {          // the 4 lanes of a row agree on this
    const float alpha = fast_exp2(m_run - mx);
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < 32; ++d) acc[d] *= alpha;
    m_run = mx;
  }
  const float m_use = (m_run == kNegInf) ? 0.f : m_run;
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
  l_run += psum;

  // ---- O^T += V^T P^T ------------------------------------------------------------
  // Transposed read of dims 16d.. : 16 * ((2d + hh) ^ sw_v) = 128 * (d / 4) + vb[d % 4].
  int vb[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) vb[r] = 16 * ((2 * r + ln.tr_hh) ^ ln.sw_v) + 8 * ln.tr_half;
  if constexpr (NT >= 2) {
#pragma unroll
    for (int u = 0; u < NT / 2; ++u) {
      const int tb = 16 * (tg * NT + 2 * u);
      const uint8_t* v0 = page + (tb + ln.tr_tok) * kRowBytes;
      // P^T operand; k-slot j < 4 is token tb + 4*q4 + j, j >= 4 is token tb + 16 + 4*q4 + j - 4
      bf16x8 pb[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float x0 = s[2 * u][j], x1 = s[2 * u + 1][j];
          if constexpr (kFp8) {
            x0 *= scale_tab[4 * (tb + 4 * q4 + j) + g];
            x1 *= scale_tab[4 * (tb + 16 + 4 * q4 + j) + g];
          }
          pb[g][j] = static_cast<__bf16>(x0);
          pb[g][4 + j] = static_cast<__bf16>(x1);
        }
      }
      if constexpr (kFp8) {
        // the dequantised page sits in its own buffer (no load in flight to it)
        auto vload = [&](int d) -> bf16x8 {
          const uint8_t* a0 = v0 + 128 * (d >> 2) + vb[d & 3];
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, a0));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, a0 + 16 * kRowBytes));
          return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        constexpr int kAhead = 4;
        bf16x8 va[kAhead];
#pragma unroll
        for (int d = 0; d < kAhead; ++d) va[d] = vload(d);
#pragma unroll
        for (int d = 0; d < 32; ++d) {
          const bf16x8 a = va[d % kAhead];
          if (d + kAhead < 32) va[d % kAhead] = vload(d + kAhead);
          acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[d >> 3], acc[d], 0, 0, 0);
        }
        continue;  // next pair of token tiles
      }
      // transposed V reads in inline asm, 4 dims (8 reads) per asm block, as the K reads
      const uint32_t vbase = lds_addr(v0);
#pragma unroll
      for (int d0 = 0; d0 < 32; d0 += 4) {
        uint32_t va[8];
        u32x2 vr[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          va[2 * j] = vbase + 128 * ((d0 + j) >> 2) + vb[(d0 + j) & 3];
          va[2 * j + 1] = va[2 * j] + 16 * kRowBytes;
        }
        lds_read_tr8_block(va, vr);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x4 lo = __builtin_bit_cast(bf16x4, vr[2 * j]), hi = __builtin_bit_cast(bf16x4, vr[2 * j + 1]);
          const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          const int d = d0 + j;
          acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[0], acc[d], 0, 0, 0);
        }
      }
    }
  } else {
    const int tb = 16 * tg;
    const uint8_t* v0 = page + (tb + ln.tr_tok) * kRowBytes;
    s16x4 pb[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = s[0][j];
        if constexpr (kFp8) x *= scale_tab[4 * (tb + 4 * q4 + j) + g];
        pb[g][j] = static_cast<short>(f32_to_bf16(x));
      }
    }
    if constexpr (kFp8) {
      auto vload = [&](int d) -> s16x4 {
        return __builtin_bit_cast(
            s16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, v0 + 128 * (d >> 2) + vb[d & 3])));
      };
      constexpr int kAhead = 4;
      s16x4 va[kAhead];
#pragma unroll
      for (int d = 0; d < kAhead; ++d) va[d] = vload(d);
#pragma unroll
      for (int d = 0; d < 32; ++d) {
        const s16x4 a = va[d % kAhead];
        if (d + kAhead < 32) va[d % kAhead] = vload(d + kAhead);
        acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb[d >> 3], acc[d], 0, 0, 0);
      }
      return;
    }
    // transposed V reads in inline asm, 8 dims per asm block, as the K reads
    const uint32_t vbase = lds_addr(v0);
#pragma unroll
    for (int d0 = 0; d0 < 32; d0 += 8) {
      uint32_t va[8];
      u32x2 vr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) va[j] = vbase + 128 * ((d0 + j) >> 2) + vb[(d0 + j) & 3];
      lds_read_tr8_block(va, vr);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = d0 + j;
        acc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vr[j]), pb[0], acc[d], 0, 0, 0);
      }
    }
  }
}

// Token-group merge through LDS (fp32 [16 rows][512] per slot sl of the scratch
// `red`): the 16-byte chunk 4 d + q4 of row r16 sits at chunk (4 d + q4) ^ r16 --
// with 2 KB rows the 16 rows of one store would otherwise all hit the same
// banks. The accesses are inline asm: the compiler cannot tell them from the
// page loads in flight (which write LDS) and would wait for all of those first.
// The reads wait for their own data inside the asm block (early-clobber
// outputs, so no address register is reused while a read is in flight).
__device__ __forceinline__ void merge_put(float* red, int sl, int r16, int q4, const f32x4 (&acc)[32]) {
  const uint32_t base = lds_addr(red + sl * (16 * 512) + r16 * 512);
#pragma unroll
  for (int d = 0; d < 32; ++d) lds_store16(base + 16 * ((4 * d + q4) ^ r16), acc[d]);
}
__device__ __forceinline__ void merge_add(const float* red, int sl, int r16, int q4, f32x4 (&acc)[32]) {
  const uint32_t base = lds_addr(red + sl * (16 * 512) + r16 * 512);
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    f32x4 x0, x1, x2, x3;
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
        : "v"(base + 16 * ((4 * (4 * g + 0) + q4) ^ r16)), "v"(base + 16 * ((4 * (4 * g + 1) + q4) ^ r16)),
          "v"(base + 16 * ((4 * (4 * g + 2) + q4) ^ r16)), "v"(base + 16 * ((4 * (4 * g + 3) + q4) ^ r16))
        : "memory");
    acc[4 * g + 0] += x0;
    acc[4 * g + 1] += x1;
    acc[4 * g + 2] += x2;
    acc[4 * g + 3] += x3;
  }
}

// The token-group merge of four waves that hold the same 16 rows (each over its own tokens), as
// two exchanges through LDS in which all four waves take part: waves w and w ^ 2 swap halves of
// the 512 dims (wave w keeps half w >> 1), then waves w and w ^ 1 swap quarters of the kept half
// (wave w keeps quarter w, acc[8w .. 8w + 8), and writes it). Step-1 blocks are 16 rows x 256
// fp32 (16 KB, one per sending wave), step-2 blocks 16 rows x 128 fp32 (8 KB); 16-byte chunk c of
// a row sits at chunk c ^ r16 (no bank conflicts between the 16 rows).
template <int D0, int N>
__device__ __forceinline__ void red_put(uint32_t base, int r16, int q4, const f32x4 (&acc)[32]) {
#pragma unroll
  for (int j = 0; j < N; ++j) lds_store16(base + 16 * ((4 * j + q4) ^ r16), acc[D0 + j]);
}
template <int D0, int N>
__device__ __forceinline__ void red_add(uint32_t base, int r16, int q4, f32x4 (&acc)[32]) {
#pragma unroll
  for (int g = 0; g < N; g += 8) {
    uint32_t a[8];
    bf16x8 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = base + 16 * ((4 * (g + k) + q4) ^ r16);
    lds_read16_block<8>(a, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[D0 + g + k] += __builtin_bit_cast(f32x4, v[k]);
  }
}

template <int RB, int TG, int FMT>
__global__ void __launch_bounds__(kThreads) splitkv_kernel(DecodeParams p) {
  static_assert(RB * TG == kWaves, "4 waves per workgroup");
  constexpr int M_TILE = 16 * RB;
  constexpr bool kFp8 = (FMT == kFmtFp8);
  constexpr int kLoads = kFp8 ? kFp8Loads : kBf16Loads;
  constexpr int kLoadsPerWave = (kLoads + kWaves - 1) / kWaves;
  constexpr int kSlotBytes = kFp8 ? kRawPageBytes : kPageBytes;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[kFp8 ? kLdsFp8 : kLdsBf16];
  __shared__ float red_m[kWaves][16];
  __shared__ float red_l[kWaves][16];
  uint8_t* const ring = smem;                                        // two load slots
  uint8_t* const conv = smem + 2 * kRawPageBytes;                    // fp8: converted page + scales

  Lane ln;
  ln.tid = threadIdx.x;
  ln.lane = ln.tid & 63;
  ln.wave = ln.tid >> 6;
  const int rb = ln.wave % RB;
  ln.tg = ln.wave / RB;
  ln.r16 = ln.lane & 15;
  ln.q4 = ln.lane >> 4;
  ln.sw_k = swz(ln.r16);
  ln.tr_tok = 4 * ln.q4 + (ln.r16 >> 2);
  ln.sw_v = swz(ln.tr_tok);
  ln.tr_half = ln.r16 & 1;
  ln.tr_hh = (ln.r16 & 3) >> 1;
  const int lane = ln.lane, wave = ln.wave, tg = ln.tg, r16 = ln.r16, q4 = ln.q4;

  // Workgroup i runs on XCD i % 8: give each XCD a contiguous block of
  // logical ids so the row tiles of one KV range share that XCD's L2.
  const int per_xcd = gridDim.x / 8;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= p.grid_wgs) return;
  const int m_tiles = (p.rows + M_TILE - 1) / M_TILE;
  const int mt = logical % m_tiles;
  const int kvh = (logical / m_tiles) % p.h_kv;
  const int part = logical / (m_tiles * p.h_kv);

  Range r;
  if (!read_range(p, part, r)) return;

  const int row = mt * M_TILE + rb * 16 + r16;   // this lane's query row within the KV head
  const bool row_ok = row < p.rows;
  const int s_idx = row_ok ? row / p.group : 0;
  const int head = kvh * p.group + (row_ok ? row % p.group : 0);

  // Per-lane byte offsets (within a page of this KV head) of the direct loads.
  uint32_t ld_off[kLoadsPerWave];
#pragma unroll
  for (int j = 0; j < kLoadsPerWave; ++j) {
    const int k = wave + kWaves * j;
    const int x = 1024 * k + 16 * lane;            // byte in the LDS slot
    if constexpr (kFp8) {
      const int t = x / kFp8Record;
      ld_off[j] = static_cast<uint32_t>(t * p.kv_st + (x - t * kFp8Record));
    } else {
      const int pc = x / 16;
      const int t = pc / 72;
      const int lc = (pc - 72 * t) ^ swz(t);
      ld_off[j] = static_cast<uint32_t>(t * p.kv_st + 16 * lc);
    }
  }
  const uint8_t* const kv_head = p.kv + kvh * p.kv_sh;
  const int page_extent = kPage * static_cast<int>(p.kv_st);

  // Block-table window: lane i holds entry win_pi + i of sequence win_b's row
  // (-1 past the row). Refilled with one vector load when a page falls outside
  // it (a new sequence, or every 64 pages), so pages need no scalar load each.
  int bt_win = -1, win_b = -1, win_pi = 0;
  // Global address of page `pi` of sequence `b`; nullptr for a block-table
  // entry outside the pool (never dereferenced).
  auto page_src = [&](int b, int pi) -> const uint8_t* {
    if (b != win_b || pi < win_pi || pi >= win_pi + 64) {
      win_b = b;
      win_pi = pi;
      const int e = pi + lane;
      bt_win = e < p.max_blocks ? p.block_table[static_cast<int64_t>(b) * p.bt_stride + e] : -1;
      wait_vm_all();
    }
    const int pg = __builtin_amdgcn_readlane(bt_win, pi - win_pi);
    if (pg < 0 || pg >= p.num_pages) return nullptr;
    return kv_head + static_cast<int64_t>(pg) * p.kv_sp;
  };

  // ---- pipeline: two pages in flight ------------------------------------------------
  // q0 is the page computed next (ring slot `slot`), q1 the one after it (slot ^ 1).
  // q1's loads go out as soon as its slot is free -- right after the barrier that
  // ends the compute of the page before -- so q1 streams in while q0 lands; q0 is
  // then waited with a count that leaves this wave's loads of q1 in flight (vmcnt
  // falls in issue order). (nb2, npi2, src2) is the page after q1, looked up one
  // page early so no lookup sits in front of an issue. At the last page of a
  // sequence whose token groups are merged through LDS, the page after q1 is held
  // back (its slot is the merge scratch) and issued when the next sequence starts.
  constexpr bool kMergeScratch = (TG > 1) && !kFp8;
  int slot = 0;
  bool q0_ok = true, q1_ok = true;
  int q1_state = 0;                  // 0: no page, 1: loads issued (none if !q1_ok), 2: held back
  const uint8_t* q1_src = nullptr;
  int nb2 = r.end_b + 1, npi2 = 0;
  const uint8_t* src2 = nullptr;
  // the page after (b_, pi_) inside the range (b_ > r.end_b: none); e_ = end page of b_ if known (else -1)
  auto advance = [&](int b_, int pi_, int e_, int& nb, int& npi) {
    if (e_ < 0) {
      int L_, a_;
      seq_pages(p, r, b_, L_, a_, e_);
    }
    if (pi_ + 1 < e_) {
      nb = b_;
      npi = pi_ + 1;
    } else {
      next_with_pages(p, r, b_ + 1, nb, npi);
    }
  };
  // wait until q0 has landed, leaving this wave's loads of q1 (issued after q0's) in flight
  auto wait_q0 = [&]() {
    if (q1_state == 1 && q1_ok) {
      if constexpr (kLoads % kWaves == 0) {
        wait_vmcnt<kLoads / kWaves>();
      } else {
        if (wave < kLoads % kWaves)
          wait_vmcnt<kLoads / kWaves + 1>();
        else
          wait_vmcnt<kLoads / kWaves>();
      }
    } else {
      wait_vm_all();
    }
  };
  {
    int nb, npi;
    next_with_pages(p, r, r.begin_b, nb, npi);
    if (nb <= r.end_b) {
      const uint8_t* src = page_src(nb, npi);
      q0_ok = src != nullptr;
      if (q0_ok) issue_page<FMT>(src, page_extent, ring, ld_off, wave);
      int nb1, npi1;
      advance(nb, npi, -1, nb1, npi1);
      if (nb1 <= r.end_b) {
        q1_src = page_src(nb1, npi1);
        q1_ok = q1_src != nullptr;
        if (kMergeScratch && nb != r.begin_b) {
          q1_state = 2;                // sequences with no pages come first: their merges use slot 1
        } else {
          if (q1_ok) issue_page<FMT>(q1_src, page_extent, ring + kSlotBytes, ld_off, wave);
          q1_state = 1;
        }
        advance(nb1, npi1, -1, nb2, npi2);
        if (nb2 <= r.end_b) src2 = page_src(nb2, npi2);
      }
    }
  }

  for (int b = r.begin_b; b <= r.end_b; ++b) {
    int L, pg0, pg1;
    bool len_ok;
    seq_pages(p, r, b, L, pg0, pg1, len_ok);
    const int split_idx = (b == r.begin_b) ? r.split0 : 0;
    const int slot0 = ld_meta(p.num_splits + b);
    const int nsplit = ld_meta(p.num_splits + b + 1) - slot0;
    const int last_allowed = p.causal ? (L - p.s_q + s_idx) : (L - 1);

    // Q^T operand: 18 chunks of 8 dims (dims 32c + 8*q4 .. +8) of this lane's row.
    bf16x8 qf[18];
    {
      const uint16_t* qrow = p.q + b * p.q_sb + s_idx * p.q_ss + head * p.q_sh;
#pragma unroll
      for (int c = 0; c < 18; ++c) {
        u32x4 v = row_ok ? *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * q4) : u32x4{0u, 0u, 0u, 0u};
        qf[c] = __builtin_bit_cast(bf16x8, v);
      }
      // Q must be in registers before the page loop: otherwise the first MFMA
      // would wait on every load in flight, the next page's included.
      wait_vm_all();
    }
    // a page held back at the end of an earlier sequence: its slot is free again (the merge is
    // done). Not for a sequence with no pages here: its merge still uses that slot.
    if (q1_state == 2 && pg0 < pg1) {
      if (q1_ok) issue_page<FMT>(q1_src, page_extent, ring + (slot ^ 1) * kSlotBytes, ld_off, wave);
      q1_state = 1;
    }

    float m_run = kNegInf, l_run = 0.f;
    f32x4 acc[32];
#pragma unroll
    for (int d = 0; d < 32; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool bad = r.stale || !len_ok;

    for (int pi = pg0; pi < pg1; ++pi) {
      // page (b, pi) = q0 is in flight into `slot`, q1 (if any) into slot ^ 1
      const bool this_ok = q0_ok;
      bad |= !this_ok;
      wait_q0();
      lds_barrier_keep_loads();                   // q0's bytes are in LDS for every wave
      page_step<TG, FMT>(ring + slot * kSlotBytes, conv, ln, L, last_allowed, pi, this_ok, p.scale_log2, qf, acc,
                         m_run, l_run);
      lds_barrier_keep_loads();                   // every wave is done with `slot`
      // q1 becomes q0; the page after it becomes q1, its loads into `slot`
      q0_ok = q1_ok;
      if (q1_state != 0 && nb2 <= r.end_b) {
        q1_src = src2;
        q1_ok = src2 != nullptr;
        if (kMergeScratch && pi + 1 == pg1) {
          q1_state = 2;
        } else {
          if (q1_ok) issue_page<FMT>(src2, page_extent, ring + slot * kSlotBytes, ld_off, wave);
          q1_state = 1;
        }
        int nb3, npi3;
        advance(nb2, npi2, nb2 == b ? pg1 : -1, nb3, npi3);
        nb2 = nb3;
        npi2 = npi3;
        src2 = (nb2 <= r.end_b) ? page_src(nb2, npi2) : nullptr;
      } else {
        q1_state = 0;
      }
      slot ^= 1;
    }

    // ---- merge the token groups, then write -------------------------------------------
    float l_row = sum4lanes(l_run);
    float m_fin = m_run;
    if constexpr (TG > 1) {
      lds_barrier_keep_loads();                   // all waves done with the LDS page
      if (lane < 16) {
        red_m[wave][r16] = m_run;
        red_l[wave][r16] = l_row;
      }
      lds_barrier_keep_loads();
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
      // Sum the TG accumulators of each row block through LDS, in the slot not
      // receiving a page (bf16) or the converted page (fp8).
      uint8_t* red = kFp8 ? conv : ring + (slot ^ 1) * kSlotBytes;
      if constexpr (TG == 4) {                 // RB == 1: waves 0..3 hold the same rows
        const uint32_t s1 = lds_addr(red) + r16 * 1024, s2 = lds_addr(red) + r16 * 512;
        if (wave < 2)
          red_put<16, 16>(s1 + wave * 16384, r16, q4, acc);
        else
          red_put<0, 16>(s1 + wave * 16384, r16, q4, acc);
        lds_barrier_keep_loads();
        if (wave < 2)
          red_add<0, 16>(s1 + (wave ^ 2) * 16384, r16, q4, acc);
        else
          red_add<16, 16>(s1 + (wave ^ 2) * 16384, r16, q4, acc);
        lds_barrier_keep_loads();
        switch (wave) {
          case 0: red_put<8, 8>(s2, r16, q4, acc); break;
          case 1: red_put<0, 8>(s2 + 8192, r16, q4, acc); break;
          case 2: red_put<24, 8>(s2 + 2 * 8192, r16, q4, acc); break;
          default: red_put<16, 8>(s2 + 3 * 8192, r16, q4, acc); break;
        }
        lds_barrier_keep_loads();
        switch (wave) {
          case 0: red_add<0, 8>(s2 + 8192, r16, q4, acc); break;
          case 1: red_add<8, 8>(s2, r16, q4, acc); break;
          case 2: red_add<16, 8>(s2 + 3 * 8192, r16, q4, acc); break;
          default: red_add<24, 8>(s2 + 2 * 8192, r16, q4, acc); break;
        }
      } else {                                  // TG == 2, RB == 2
        float* redf = reinterpret_cast<float*>(red);
        if (tg == 1) merge_put(redf, rb, r16, q4, acc);
        lds_barrier_keep_loads();
        if (tg == 0) merge_add(redf, rb, r16, q4, acc);
      }
      lds_barrier_keep_loads();                            // scratch free again before the next page lands
    }

    // the rows' dims [16 D0, 16 (D0 + N)) (acc[D0 .. D0 + N)): 4 waves write a quarter each
    // after the four-way merge, else the waves of token group 0 write all of them
    auto store = [&](auto d0_c, auto n_c) {
      constexpr int D0 = decltype(d0_c)::value, N = decltype(n_c)::value;
      const bool ok = !bad;
      const float inv = (l_row > 0.f) ? 1.f / l_row : 0.f;
      float lse = (l_row > 0.f) ? (m_fin + __log2f(l_row)) * kLn2 : kNegInf;
      if (!ok) lse = __builtin_nanf("");
      const bool lse_lane = q4 == 0 && (TG < 4 || wave == 0);
      if (nsplit == 1) {
        uint16_t* orow = p.o + ((static_cast<int64_t>(b) * p.s_q + s_idx) * p.h_q + head) * kDv + 4 * q4;
        const float nan = __builtin_nanf("");
#pragma unroll
        for (int d = D0; d < D0 + N; ++d) {
          u32x2 w;
          const float x0 = ok ? acc[d][0] * inv : nan;
          const float x1 = ok ? acc[d][1] * inv : nan;
          const float x2 = ok ? acc[d][2] * inv : nan;
          const float x3 = ok ? acc[d][3] * inv : nan;
          w[0] = static_cast<uint32_t>(f32_to_bf16(x0)) | (static_cast<uint32_t>(f32_to_bf16(x1)) << 16);
          w[1] = static_cast<uint32_t>(f32_to_bf16(x2)) | (static_cast<uint32_t>(f32_to_bf16(x3)) << 16);
          *reinterpret_cast<u32x2*>(orow + 16 * d) = w;
        }
        if (lse_lane) p.lse[lse_index(p, b, head, s_idx)] = lse;
      } else {
        const int pslot = slot0 + split_idx;
        if (pslot >= 0 && pslot < p.max_slots && split_idx < nsplit) {
          float* prow = p.part_o32 + ((static_cast<int64_t>(pslot) * p.h_kv + kvh) * p.rows + row) * kDv + 4 * q4;
          const float nan = __builtin_nanf("");
#pragma unroll
          for (int d = D0; d < D0 + N; ++d) {
            f32x4 v = acc[d] * inv;
            if (!ok) v = f32x4{nan, nan, nan, nan};
            *reinterpret_cast<f32x4*>(prow + 16 * d) = v;
          }
          if (lse_lane) p.part_lse[(static_cast<int64_t>(pslot) * p.h_kv + kvh) * p.rows + row] = lse;
        }
      }
    };
    if (row_ok) {
      if constexpr (TG == 4) {
        switch (wave) {
          case 0: store(std::integral_constant<int, 0>{}, std::integral_constant<int, 8>{}); break;
          case 1: store(std::integral_constant<int, 8>{}, std::integral_constant<int, 8>{}); break;
          case 2: store(std::integral_constant<int, 16>{}, std::integral_constant<int, 8>{}); break;
          default: store(std::integral_constant<int, 24>{}, std::integral_constant<int, 8>{}); break;
        }
      } else if (tg == 0) {
        store(std::integral_constant<int, 0>{}, std::integral_constant<int, 32>{});
      }
    }
  }
  wait_vm_all();   // nothing may still be landing in LDS when the workgroup ends
}

// ----------------------------------------------------------------------------
// Combine: LSE = ln sum_i exp(LSE_i), O = sum_i exp(LSE_i - LSE) O_i
// (the split epilogue of the wmrh.cn page, "计算流水线设计"; O_i are the
// pieces' normalised partial outputs). The narrow kernel reads each piece's
// LSE and O together and merges them online -- a running max M,
// l = sum exp(LSE_i - M) and acc = sum exp(LSE_i - M) O_i, rescaled when M
// grows -- so the partials are read in one pass with all loads of a group of
// pieces in flight.
// Empty pieces (LSE = -inf, O = 0) add nothing; a NaN LSE (a piece with a
// page outside the pool) makes l NaN for good, and with it O and LSE.
// ----------------------------------------------------------------------------

struct MergeState {
  float m = kNegInf;      // running max of the LSEs seen
  float l = 0.f;          // sum exp(LSE_i - m)
  f32x4 a0 = f32x4{0.f, 0.f, 0.f, 0.f}, a1 = f32x4{0.f, 0.f, 0.f, 0.f};   // sum exp(LSE_i - m) O_i (8 dims)
};

// Merge up to N pieces (valid[i]) whose LSE and 8 dims of O are already in registers.
template <int N>
__device__ __forceinline__ void merge_group(MergeState& st, const float (&lse)[N], const f32x4 (&x0)[N],
                                            const f32x4 (&x1)[N], int n_valid) {
  float mc = kNegInf;
  bool nan = false;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i < n_valid) {
      mc = fmaxf(mc, lse[i]);
      nan |= lse[i] != lse[i];
    }
  }
  if (nan) st.l = __builtin_nanf("");
  const float mn = fmaxf(st.m, mc);
  if (mn == kNegInf) return;                 // nothing allowed so far
  const float sc = (st.m == kNegInf) ? 0.f : __expf(st.m - mn);
  st.l *= sc;
  st.a0 *= sc;
  st.a1 *= sc;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i < n_valid) {
      const float w = __expf(lse[i] - mn);
      st.l += w;
      if (w != 0.f) {                        // an empty piece has w = 0 and O = 0
        st.a0 += w * x0[i];
        st.a1 += w * x1[i];
      }
    }
  }
  st.m = mn;
}

// 1 / l for the final normalisation: 0 when nothing was allowed (O = 0), NaN for NaN.
__device__ __forceinline__ float merge_inv(float l) { return (l > 0.f) ? 1.f / l : ((l != l) ? l : 0.f); }

// LSE of a merged state: -inf when nothing was allowed, NaN for NaN.
__device__ __forceinline__ float merge_lse(const MergeState& st) {
  return (st.l > 0.f || st.l != st.l) ? st.m + __logf(st.l) : kNegInf;
}

__device__ __forceinline__ u32x4 pack_bf16x8(const f32x4& a0, const f32x4& a1) {
  u32x4 w;
  w[0] = static_cast<uint32_t>(f32_to_bf16(a0[0])) | (static_cast<uint32_t>(f32_to_bf16(a0[1])) << 16);
  w[1] = static_cast<uint32_t>(f32_to_bf16(a0[2])) | (static_cast<uint32_t>(f32_to_bf16(a0[3])) << 16);
  w[2] = static_cast<uint32_t>(f32_to_bf16(a1[0])) | (static_cast<uint32_t>(f32_to_bf16(a1[1])) << 16);
  w[3] = static_cast<uint32_t>(f32_to_bf16(a1[2])) | (static_cast<uint32_t>(f32_to_bf16(a1[3])) << 16);
  return w;
}

constexpr int kCombDims = 128;                  // dims per workgroup
constexpr int kCombGroup = 4;                   // pieces whose loads are in flight together
constexpr int kFewPieces = 2 * kCombGroup;      // one round of loads per lane (two groups of 4)

// One workgroup's share of a sequence cut into 2..n_max pieces: 16 rows of one KV head, one
// 128-dim quarter; 16 lanes per row, 8 dims per lane, the pieces in groups of kCombGroup with
// all their loads in flight at once. Sequences of one piece (written by the split kernel) and
// of more than n_max pieces (left to other workgroups) are skipped.
template <bool F16>
__device__ __forceinline__ void combine_rows_task(const DecodeParams& p, int b, int rt, int z, int n_max) {
  const int tid = threadIdx.x;
  const int row = rt * 16 + tid / 16;
  const int l16 = tid & 15;
  const int kvh = z / (kDv / kCombDims);
  const int quarter = z % (kDv / kCombDims);
  const int slot0 = ld_meta(p.num_splits + b);
  const int n = ld_meta(p.num_splits + b + 1) - slot0;
  if (n == 1 || n > n_max || row >= p.rows) return;
  const int s_idx = row / p.group;
  const int head = kvh * p.group + row % p.group;
  const int dim0 = quarter * kCombDims + 8 * l16;
  uint16_t* orow = p.o + ((static_cast<int64_t>(b) * p.s_q + s_idx) * p.h_q + head) * kDv + dim0;
  float* lse_out = p.lse + lse_index(p, b, head, s_idx);
  // no piece (num_splits inconsistent with the ranges) or slots outside the workspace: NaN, never
  // a read of partials nobody wrote
  if (n <= 0 || slot0 < 0 || slot0 + n > p.max_slots) {
    *reinterpret_cast<u32x4*>(orow) = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
    if (l16 == 0 && quarter == 0) *lse_out = __builtin_nanf("");
    return;
  }
  const int64_t stride = static_cast<int64_t>(p.h_kv) * p.rows;
  const float* lse_in = p.part_lse + static_cast<int64_t>(slot0) * stride + static_cast<int64_t>(kvh) * p.rows + row;
  const int64_t row0 = static_cast<int64_t>(slot0) * stride + static_cast<int64_t>(kvh) * p.rows + row;
  MergeState st;
  for (int i0 = 0; i0 < n; i0 += kCombGroup) {
    float lse[kCombGroup];
    f32x4 x0[kCombGroup], x1[kCombGroup];
    if constexpr (F16) {
      const uint16_t* o_in = p.part_o16 + row0 * kDv + dim0;
      const float* sc_in = p.part_scale + row0 * kPartBlocks + (dim0 >> 6);
      float sc[kCombGroup];
      u32x4 h[kCombGroup];
      // all loads of the group first (converting right after each load would wait for it)
#pragma unroll
      for (int j = 0; j < kCombGroup; ++j) {
        const int i = i0 + j;
        if (i < n) {
          lse[j] = lse_in[i * stride];
          h[j] = *reinterpret_cast<const u32x4*>(o_in + i * stride * kDv);
          sc[j] = sc_in[i * stride * kPartBlocks];
        } else {
          lse[j] = kNegInf;
          h[j] = u32x4{0u, 0u, 0u, 0u};
          sc[j] = 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < kCombGroup; ++j) {
        x0[j] = f32x4{f16_lo(h[j][0]), f16_hi(h[j][0]), f16_lo(h[j][1]), f16_hi(h[j][1])} * sc[j];
        x1[j] = f32x4{f16_lo(h[j][2]), f16_hi(h[j][2]), f16_lo(h[j][3]), f16_hi(h[j][3])} * sc[j];
      }
    } else {
      const float* o_in = p.part_o32 + row0 * kDv + dim0;
#pragma unroll
      for (int j = 0; j < kCombGroup; ++j) {
        const int i = i0 + j;
        if (i < n) {
          lse[j] = lse_in[i * stride];
          x0[j] = *reinterpret_cast<const f32x4*>(o_in + i * stride * kDv);
          x1[j] = *reinterpret_cast<const f32x4*>(o_in + i * stride * kDv + 4);
        } else {
          lse[j] = kNegInf;
          x0[j] = f32x4{0.f, 0.f, 0.f, 0.f};
          x1[j] = x0[j];
        }
      }
    }
    merge_group<kCombGroup>(st, lse, x0, x1, min(n - i0, kCombGroup));
  }
  const float inv = merge_inv(st.l);
  *reinterpret_cast<u32x4*>(orow) = pack_bf16x8(st.a0 * inv, st.a1 * inv);
  if (l16 == 0 && quarter == 0) *lse_out = merge_lse(st);
}

// One workgroup per (sequence, 16 rows, KV head, 128-dim quarter).
template <bool F16>
__global__ void __launch_bounds__(kThreads) combine_rows_kernel(DecodeParams p) {
  combine_rows_task<F16>(p, blockIdx.x, blockIdx.y, blockIdx.z, INT_MAX);
}


// Sequences of at most 8 pieces: one workgroup per (sequence, 16 rows, KV head, QPL
// 128-dim quarters); each lane merges its row's 8 dims in each of the QPL quarters, so
// the loads of QPL quarters of PG pieces are in flight together (the merge is latency
// bound: fewer, fuller waves). The running max and sum are shared by the quarters.
template <bool F16, int QPL>
__global__ void __launch_bounds__(kThreads) combine_q_kernel(DecodeParams p) {
  constexpr int PG = QPL >= 4 ? 2 : 4;           // pieces whose loads are in flight together
  constexpr int kGroups = kDv / (kCombDims * QPL);
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int row = blockIdx.y * 16 + tid / 16;
  const int l16 = tid & 15;
  const int kvh = blockIdx.z / kGroups;
  const int q0 = (blockIdx.z % kGroups) * QPL;
  const int slot0 = ld_meta(p.num_splits + b);
  const int n = ld_meta(p.num_splits + b + 1) - slot0;
  if (n == 1 || row >= p.rows) return;          // one piece: written by the split kernel
  const int s_idx = row / p.group;
  const int head = kvh * p.group + row % p.group;
  const int dim0 = q0 * kCombDims + 8 * l16;
  uint16_t* orow = p.o + ((static_cast<int64_t>(b) * p.s_q + s_idx) * p.h_q + head) * kDv + dim0;
  float* lse_out = p.lse + lse_index(p, b, head, s_idx);
  if (n <= 0 || slot0 < 0 || slot0 + n > p.max_slots) {
#pragma unroll
    for (int qq = 0; qq < QPL; ++qq)
      *reinterpret_cast<u32x4*>(orow + qq * kCombDims) = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
    if (l16 == 0 && q0 == 0) *lse_out = __builtin_nanf("");
    return;
  }
  const int64_t stride = static_cast<int64_t>(p.h_kv) * p.rows;
  const int64_t row0 = static_cast<int64_t>(slot0) * stride + static_cast<int64_t>(kvh) * p.rows + row;
  const float* lse_in = p.part_lse + row0;
  float m = kNegInf, l = 0.f;
  f32x4 a0[QPL], a1[QPL];
#pragma unroll
  for (int qq = 0; qq < QPL; ++qq) a0[qq] = a1[qq] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < n; i0 += PG) {
    float lse[PG];
    f32x4 x0[PG][QPL], x1[PG][QPL];
    if constexpr (F16) {
      const uint16_t* o_in = p.part_o16 + row0 * kDv + dim0;
      const float* sc_in = p.part_scale + row0 * kPartBlocks + (dim0 >> 6);
      float sc[PG][QPL];
      u32x4 h[PG][QPL];
      // all loads first (converting right after each load would wait for it)
#pragma unroll
      for (int j = 0; j < PG; ++j) {
        const int i = i0 + j;
        lse[j] = (i < n) ? lse_in[i * stride] : kNegInf;
#pragma unroll
        for (int qq = 0; qq < QPL; ++qq) {
          h[j][qq] = (i < n) ? *reinterpret_cast<const u32x4*>(o_in + i * stride * kDv + qq * kCombDims)
                             : u32x4{0u, 0u, 0u, 0u};
          sc[j][qq] = (i < n) ? sc_in[i * stride * kPartBlocks + qq * (kCombDims / 64)] : 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < PG; ++j)
#pragma unroll
        for (int qq = 0; qq < QPL; ++qq) {
          const u32x4 w = h[j][qq];
          x0[j][qq] = f32x4{f16_lo(w[0]), f16_hi(w[0]), f16_lo(w[1]), f16_hi(w[1])} * sc[j][qq];
          x1[j][qq] = f32x4{f16_lo(w[2]), f16_hi(w[2]), f16_lo(w[3]), f16_hi(w[3])} * sc[j][qq];
        }
    } else {
      const float* o_in = p.part_o32 + row0 * kDv + dim0;
#pragma unroll
      for (int j = 0; j < PG; ++j) {
        const int i = i0 + j;
        lse[j] = (i < n) ? lse_in[i * stride] : kNegInf;
#pragma unroll
        for (int qq = 0; qq < QPL; ++qq) {
          x0[j][qq] = (i < n) ? *reinterpret_cast<const f32x4*>(o_in + i * stride * kDv + qq * kCombDims)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
          x1[j][qq] = (i < n) ? *reinterpret_cast<const f32x4*>(o_in + i * stride * kDv + qq * kCombDims + 4)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    // the online merge of merge_group, with the max and sum shared by the quarters
    const int nv = min(n - i0, PG);
    float mc = kNegInf;
    bool nan = false;
#pragma unroll
    for (int j = 0; j < PG; ++j)
      if (j < nv) {
        mc = fmaxf(mc, lse[j]);
        nan |= lse[j] != lse[j];
      }
    if (nan) l = __builtin_nanf("");
    const float mn = fmaxf(m, mc);
    if (mn == kNegInf) continue;                  // nothing allowed so far
    const float scl = (m == kNegInf) ? 0.f : __expf(m - mn);
    l *= scl;
#pragma unroll
    for (int qq = 0; qq < QPL; ++qq) {
      a0[qq] *= scl;
      a1[qq] *= scl;
    }
#pragma unroll
    for (int j = 0; j < PG; ++j)
      if (j < nv) {
        const float w = __expf(lse[j] - mn);
        l += w;
        if (w != 0.f) {                           // an empty piece has w = 0 and O = 0
#pragma unroll
          for (int qq = 0; qq < QPL; ++qq) {
            a0[qq] += w * x0[j][qq];
            a1[qq] += w * x1[j][qq];
          }
        }
      }
    m = mn;
  }
  const float inv = merge_inv(l);
#pragma unroll
  for (int qq = 0; qq < QPL; ++qq)
    *reinterpret_cast<u32x4*>(orow + qq * kCombDims) = pack_bf16x8(a0[qq] * inv, a1[qq] * inv);
  if (l16 == 0 && q0 == 0) {
    MergeState st;
    st.m = m;
    st.l = l;
    *lse_out = merge_lse(st);
  }
}

// Merge a second state (m2, l2, b0, b1) into st: the online-softmax merge of two partial
// results; two states that allowed nothing stay empty, NaN in either stays NaN.
__device__ __forceinline__ void merge_states(MergeState& st, float m2, float l2, const f32x4& b0, const f32x4& b1) {
  const float mn = fmaxf(st.m, m2);
  const float s1 = (st.m == kNegInf) ? 0.f : __expf(st.m - mn);
  const float s2 = (m2 == kNegInf) ? 0.f : __expf(m2 - mn);
  st.l = st.l * s1 + l2 * s2;
  st.a0 = st.a0 * s1 + b0 * s2;
  st.a1 = st.a1 * s1 + b1 * s2;
  st.m = mn;
}

// Metadata in which some sequence is cut into more than kFewPieces pieces. The last
// batch x row tiles x KV heads x 4 workgroups are combine_rows_task's (sequences of up to
// kFewPieces pieces); the first ones, the helpers (dispatched first: theirs is the longest
// chain of loads), find the sequences of more pieces themselves (their count is not known
// on the host) and share their tasks: (listed sequence, 2 rows, KV head, 32-dim slice).
// Small tasks spread a long sequence's partials over many workgroups (a workgroup's time
// grows with the cache lines it requests, and one row's 32 fp32 dims are one line). In a
// task 32 piece groups of 8 lanes (4 lanes of 8 dims per row) take every 32nd piece, 2
// pieces each with their loads in flight together (64 pieces per round of loads); the 8
// groups of a wave merge by lane exchange, the 4 waves through LDS.
constexpr int kListRows = 2;
constexpr int kListDims = 32;
constexpr int kListLanes = kListRows * (kListDims / 8);
constexpr int kListGroups = kThreads / kListLanes;
constexpr int kListInFlight = 2;
constexpr int kListWgs = 256;                  // helpers (at most)

template <bool F16>
__global__ void __launch_bounds__(kThreads) combine_many_kernel(DecodeParams p) {
  const int rt_n = (p.rows + 15) / 16;
  const int zq = p.h_kv * (kDv / kCombDims);
  const int nb = p.batch * rt_n * zq;
  const int helpers = static_cast<int>(gridDim.x) - nb;
  if (static_cast<int>(blockIdx.x) >= helpers) {
    const int w = blockIdx.x - helpers;
    const int r = w / p.batch;
    combine_rows_task<F16>(p, w - r * p.batch, r % rt_n, r / rt_n, kFewPieces);
    return;
  }
  __shared__ int list_b[kThreads], list_slot[kThreads], list_n[kThreads];
  __shared__ int wave_cnt[kThreads / 64];
  __shared__ float xs[kThreads / 64 - 1][10][kListLanes];
  const int tid = threadIdx.x;
  const int grp = tid / kListLanes;
  const int lane = tid % kListLanes;
  const int slices = kDv / kListDims;
  const int per_seq = (p.rows + kListRows - 1) / kListRows * p.h_kv * slices;   // tasks of one listed sequence
  const int64_t stride = static_cast<int64_t>(p.h_kv) * p.rows;
  int base = 0;                                  // first task of the current chunk
  int t = blockIdx.x;                            // this helper's next task
  for (int c0 = 0; c0 < p.batch; c0 += kThreads) {
    // the chunk's sequences of more than kFewPieces pieces, in order
    const int b = c0 + tid;
    int slot0 = 0, n = 1;
    if (b < p.batch) {
      slot0 = p.num_splits[b];
      n = p.num_splits[b + 1] - slot0;
    }
    const bool listed = n > kFewPieces;
    const uint64_t ball = __ballot(listed);
    const int w = tid >> 6;
    if ((tid & 63) == 0) wave_cnt[w] = __popcll(ball);
    __syncthreads();
    int off = 0, cnt = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) {
      off += (i < w) ? wave_cnt[i] : 0;
      cnt += wave_cnt[i];
    }
    if (listed) {
      const int pos = off + __popcll(ball & ((1ull << (tid & 63)) - 1ull));
      list_b[pos] = b;
      list_slot[pos] = slot0;
      list_n[pos] = n;
    }
    __syncthreads();
    const int end = base + cnt * per_seq;
    for (; t < end; t += helpers) {              // uniform over the workgroup
      const int tl = t - base;
      const int li = tl / per_seq;
      int r = tl - li * per_seq;
      const int slice = r % slices;
      r /= slices;
      const int kvh = r % p.h_kv;
      const int rt = r / p.h_kv;
      const int sb = list_b[li];
      const int s0 = list_slot[li];
      const int sn = list_n[li];
      const int row = rt * kListRows + lane / (kListDims / 8);
      const bool row_ok = row < p.rows;
      const int rowc = row_ok ? row : p.rows - 1;  // loads of rows past the end stay inside the workspace
      const int s_idx = rowc / p.group;
      const int head = kvh * p.group + rowc % p.group;
      const int dim0 = slice * kListDims + 8 * (lane % (kListDims / 8));
      uint16_t* orow = p.o + ((static_cast<int64_t>(sb) * p.s_q + s_idx) * p.h_q + head) * kDv + dim0;
      float* lse_out = p.lse + lse_index(p, sb, head, s_idx);
      const bool lse_lane = lane % (kListDims / 8) == 0 && slice == 0;
      if (s0 < 0 || s0 + sn > p.max_slots) {     // slots outside the workspace: NaN
        if (row_ok && grp == 0) {
          *reinterpret_cast<u32x4*>(orow) = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
          if (lse_lane) *lse_out = __builtin_nanf("");
        }
        continue;
      }
      const int64_t row0 = static_cast<int64_t>(s0) * stride + static_cast<int64_t>(kvh) * p.rows + rowc;
      MergeState st;
      for (int i0 = grp; i0 < sn; i0 += kListGroups * kListInFlight) {
        float lse[kListInFlight];
        f32x4 x0[kListInFlight], x1[kListInFlight];
        // every load issued before any is used: indices past the last piece repeat it
        if constexpr (F16) {
          u32x4 h[kListInFlight];
          float sc[kListInFlight];
#pragma unroll
          for (int j = 0; j < kListInFlight; ++j) {
            const int64_t ri = row0 + min(i0 + kListGroups * j, sn - 1) * stride;
            lse[j] = p.part_lse[ri];
            h[j] = *reinterpret_cast<const u32x4*>(p.part_o16 + ri * kDv + dim0);
            sc[j] = p.part_scale[ri * kPartBlocks + (dim0 >> 6)];
          }
          // the values are taken here, after the last load was issued: otherwise the compiler
          // moves the O loads behind the LSE test of the merge (two rounds of loads)
          asm volatile("" ::: "memory");
#pragma unroll
          for (int j = 0; j < kListInFlight; ++j) asm volatile("" : "+v"(lse[j]), "+v"(h[j]), "+v"(sc[j]));
#pragma unroll
          for (int j = 0; j < kListInFlight; ++j) {
            x0[j] = f32x4{f16_lo(h[j][0]), f16_hi(h[j][0]), f16_lo(h[j][1]), f16_hi(h[j][1])} * sc[j];
            x1[j] = f32x4{f16_lo(h[j][2]), f16_hi(h[j][2]), f16_lo(h[j][3]), f16_hi(h[j][3])} * sc[j];
          }
        } else {
#pragma unroll
          for (int j = 0; j < kListInFlight; ++j) {
            const int64_t ri = row0 + min(i0 + kListGroups * j, sn - 1) * stride;
            lse[j] = p.part_lse[ri];
            x0[j] = *reinterpret_cast<const f32x4*>(p.part_o32 + ri * kDv + dim0);
            x1[j] = *reinterpret_cast<const f32x4*>(p.part_o32 + ri * kDv + dim0 + 4);
          }
          asm volatile("" ::: "memory");
#pragma unroll
          for (int j = 0; j < kListInFlight; ++j) asm volatile("" : "+v"(lse[j]), "+v"(x0[j]), "+v"(x1[j]));
        }
        merge_group<kListInFlight>(st, lse, x0, x1, min(kListInFlight, (sn - i0 + kListGroups - 1) / kListGroups));
      }
      // the wave's groups (lanes kListLanes apart), then the 4 waves
#pragma unroll
      for (int sh = kListLanes; sh < 64; sh *= 2) {
        f32x4 b0, b1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          b0[i] = __shfl_xor(st.a0[i], sh);
          b1[i] = __shfl_xor(st.a1[i], sh);
        }
        merge_states(st, __shfl_xor(st.m, sh), __shfl_xor(st.l, sh), b0, b1);
      }
      if (w > 0 && (tid & 63) < kListLanes) {
        float* x = &xs[w - 1][0][lane];
        x[0] = st.m;
        x[kListLanes] = st.l;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[(2 + i) * kListLanes] = st.a0[i];
          x[(6 + i) * kListLanes] = st.a1[i];
        }
      }
      __syncthreads();
      if (tid < kListLanes) {
#pragma unroll
        for (int g = 0; g < kThreads / 64 - 1; ++g) {
          const float* x = &xs[g][0][lane];
          f32x4 b0, b1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            b0[i] = x[(2 + i) * kListLanes];
            b1[i] = x[(6 + i) * kListLanes];
          }
          merge_states(st, x[0], x[kListLanes], b0, b1);
        }
        if (row_ok) {
          const float inv = merge_inv(st.l);
          *reinterpret_cast<u32x4*>(orow) = pack_bf16x8(st.a0 * inv, st.a1 * inv);
          if (lse_lane) *lse_out = merge_lse(st);
        }
      }
      __syncthreads();                           // xs is written again by the next task
    }
    base = end;
    __syncthreads();                             // the lists are written again by the next chunk
  }
}

template <int RB, int TG>
hipError_t launch_split(const DecodeParams& p, int kv_format, int grid, hipStream_t stream, hipEvent_t ev_start,
                        hipEvent_t ev_stop) {
  if (kv_format == kFmtFp8)
    hipExtLaunchKernelGGL((splitkv_kernel<RB, TG, kFmtFp8>), dim3(grid), dim3(kThreads), 0, stream, ev_start, ev_stop,
                          0, p);
  else
    hipExtLaunchKernelGGL((splitkv_kernel<RB, TG, kFmtBf16>), dim3(grid), dim3(kThreads), 0, stream, ev_start,
                          ev_stop, 0, p);
  return hipGetLastError();
}

}  // namespace

// Workspace for callers that cannot allocate (mla_decode_kvcache_noalloc):
// one static array per device, so no call allocates. Host code never uses the
// array's name as an address (on the host it only names the symbol): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t scratch_workspace(void** ptr) {
  static std::mutex mu;
  static std::unordered_map<int, void*> addr;     // device -> address of its copy of `scratch`
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with `dev` current
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    it = addr.emplace(dev, p).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, const Plan& plan, int kv_format, hipStream_t stream,
                         void* const events[3]) {
  const int grid = (p.grid_wgs + 7) / 8 * 8;
  // events[0] / events[1] take the split kernel's own start / end timestamps
  // (hipExtLaunchKernelGGL), events[2] is recorded after the combine kernel.
  hipEvent_t ev0 = events ? static_cast<hipEvent_t>(events[0]) : nullptr;
  hipEvent_t ev1 = events ? static_cast<hipEvent_t>(events[1]) : nullptr;
  hipEvent_t ev2 = events ? static_cast<hipEvent_t>(events[2]) : nullptr;
  hipError_t err;
  if (p.topk > 0) {
    err = launch_split_x_sparse(p, kv_format, grid, stream, ev0, ev1);
  } else if (p.vcache != nullptr) {
    err = launch_split_vc(p, grid, stream, ev0, ev1);
  } else if (plan.wide) {
    err = launch_split_x(p, kv_format, plan.m_tile / 4, grid, stream, ev0, ev1);
  } else if (plan.rb == 1) {
    err = launch_split<1, 4>(p, kv_format, grid, stream, ev0, ev1);
  } else if (plan.rb == 2) {
    err = launch_split<2, 2>(p, kv_format, grid, stream, ev0, ev1);
  } else {
    err = launch_split<4, 1>(p, kv_format, grid, stream, ev0, ev1);
  }
  if (err != hipSuccess) return err;
  {
    const dim3 cgrid(p.batch, (p.rows + 15) / 16, p.h_kv * (kDv / kCombDims));
    // some sequence cut into more than kFewPieces pieces (the host metadata's largest piece
    // count), or that count unknown (metadata built on the device) with fp32 partials: helper
    // workgroups for those sequences (with none, they only read num_splits). At most
    // (ranges - 1) / kFewPieces sequences have that many pieces (each piece past a sequence's
    // first starts a range).
    const bool many = p.max_splits > kFewPieces || (p.max_splits == 0 && !plan.wide);
    const int64_t per_quarters = static_cast<int64_t>(p.batch) * ((p.rows + 15) / 16) * p.h_kv * (kDv / kCombDims);
    const int64_t helper_tasks = static_cast<int64_t>(std::max(1, (p.grid_wgs - 1) / kFewPieces)) *
                                 ((p.rows + kListRows - 1) / kListRows) * p.h_kv * (kDv / kListDims);
    const dim3 mgrid(static_cast<unsigned>(per_quarters + std::min<int64_t>(helper_tasks, kListWgs)));
    // fp16 partials of at most 8 pieces: two quarters per lane (mtp's combine 20.6 -> 16.8 us,
    // compute_heavy's 10.4 -> 9.6; four quarters per lane time the same, the fp32 partials of
    // the narrow tiles gain nothing)
    const dim3 cgrid_q2(p.batch, (p.rows + 15) / 16, p.h_kv * (kDv / (2 * kCombDims)));
    if (plan.wide && many)
      hipLaunchKernelGGL((combine_many_kernel<true>), mgrid, dim3(kThreads), 0, stream, p);
    else if (plan.wide)
      hipLaunchKernelGGL((combine_q_kernel<true, 2>), cgrid_q2, dim3(kThreads), 0, stream, p);
    else if (many)
      hipLaunchKernelGGL((combine_many_kernel<false>), mgrid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((combine_rows_kernel<false>), cgrid, dim3(kThreads), 0, stream, p);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (ev2) {
    err = hipEventRecord(ev2, stream);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace mla
