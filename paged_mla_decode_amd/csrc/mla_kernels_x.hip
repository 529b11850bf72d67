// mla_kernels_x.hip -- split-KV MLA decode kernels for more than 64 query rows
// per KV head on gfx950 (MI355X): 128-row tiles, 8 wavefronts. FP8 pages use
// splitkv_x_kernel (two barriers per unit: the conversion buffer of a unit
// must outlive its S and PV phases); bf16 pages use splitkv_x1_kernel (one
// barrier per unit, see its section).
//
// Same computation as the 64-row kernel in mla_kernels.hip (softmax attention
// of query rows over a sequence's cached latent rows, V = their first 512
// dims; pieces of a sequence leave partial O / LSE for the combine kernel:
// wmrh.cn FlashMLA深度解析, "计算流水线设计"), organised so that V is read from
// LDS once per workgroup and two wavefronts share each SIMD.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "kernels.h"

namespace mla {
namespace {

using namespace dev;

// ----------------------------------------------------------------------------
// 128-row tiles (more than 64 rows per KV head)
//
// Each workgroup covers 128 query rows with 8 wavefronts, two per SIMD, so
// one wave's LDS waits, softmax and barrier waits overlap the other's MFMA
// work. Work advances in units of 32 tokens (half a page); the phases below
// are shared by both kernels (FP8 pages: a two-slot ring of raw records and
// two barriers per unit; bf16 pages: a three-slot ring and one barrier):
//   S phase  -- wave w owns rows 16w .. 16w + 15: S^T = K Q^T on MFMA
//               16x16x32 bf16 (A = 16 tokens x 32 dims of K from LDS,
//               B = Q^T); 9 of the 18 32-dim Q chunks stay in VGPRs, 9 in LDS.
//   exchange -- each wave writes bf16 P^T of its rows, its rescale factors
//               and a flag; one barrier.
//   PV phase -- wave w accumulates O^T for value dims 64w .. 64w + 63 of all
//               128 rows (128 accumulator registers): it reads only its
//               eighth of V (transposed) and every wave's P^T.
// FP8 pages (656-byte records) stream raw into the ring; one LDS pass per
// unit (and one more barrier) turns the e4m3 codes into bf16 exactly (4 significant bits fit in 8)
// and copies RoPE and the 4 per-128-dim scales. The S phase applies the fp32
// scales to the per-group partial logits; in the PV phase wave w's dims lie
// in scale group w / 2, so it multiplies its P^T operand by that group's
// per-token scales and V enters the MFMA as the exact codes.
// ----------------------------------------------------------------------------

constexpr int kWW = 8;                                      // wavefronts per workgroup
constexpr int kWThreads = 64 * kWW;
constexpr int kLoadWaves = 4;                               // waves that issue the unit loads
constexpr int kXHalf = 32;                                  // tokens per unit
constexpr int kXHalfBytes = kXHalf * kRowBytes;             // 36864 = 36 x 1 KB: bf16 rows
constexpr int kXRawBytes = kXHalf * kFp8Record;             // 20992: FP8 records

// LDS layout of the FP8 kernel (bytes): the two-slot ring of raw 32-record
// units; the converted unit (bf16 rows, the chunk-group-major layout below)
// and the scales [4 groups][32 tokens]; then P^T, rescale factors, the flag
// word, and the Q^T chunks kept in LDS for all 128 rows (chunks 0 .. 6, 16,
// 17; the other chunks of each row stay in VGPRs).
struct XLayout {
  static constexpr int kRows = 128;                         // rows per tile
  static constexpr int kSlot = 21 * 1024;
  static constexpr int kSlots = 2;
  static constexpr int kRing = 0;
  static constexpr int kConv = kRing + kSlots * kSlot;
  static constexpr int kScale = kConv + kXHalfBytes;
  static constexpr int kP = kScale + 4 * kXHalf * 4;
  static constexpr int kAlpha = kP + kRows * kXHalf * 2;    // P^T: [rows][32 tokens] bf16
  static constexpr int kFlag = kAlpha + kRows * 4;          // alpha: [rows] fp32
  static constexpr int kQ = kFlag + 64;                     // rescale flag word (64 bytes reserved)
  static constexpr int kQChunks = 9;
  static constexpr int kQChunkBytes = kRows * 64;           // one 32-dim Q^T chunk of all rows
  static constexpr int kTotal = kQ + kQChunks * kQChunkBytes;
  static constexpr int kLoads = 21;                         // 1 KB direct loads per unit
  static constexpr int kLoadsPerWave = (kLoads + kLoadWaves - 1) / kLoadWaves;   // 6
  static constexpr int kLow = 7;                            // chunks 0 .. 6 in LDS, then 16, 17
  // LDS slot of Q^T chunk c, or -1 when it lives in VGPRs
  static constexpr int qslot(int c) { return c < kLow ? c : (c >= 16 ? c - 16 + kLow : -1); }
  static constexpr int kRegChunks = 18 - kQChunks;
  // register index of chunk c
  static constexpr int qreg(int c) { return c - kLow; }
  // LDS chunk index qs -> Q chunk
  static constexpr int qchunk(int qs) { return qs < kLow ? qs : 16 - kLow + qs; }
};
static_assert(XLayout::kTotal <= 163840, "LDS budget");
static_assert(XLayout::kSlot >= kXRawBytes, "FP8 slot holds a unit");

// Q^T chunks and P^T rows in LDS: 64 bytes per row (4 x 16 B); the 16-byte
// slot is XOR-swizzled with (row >> 1) & 3 so 8 consecutive rows hit 8
// distinct bank groups.
//   Q^T chunk c, slot s: dims 32 c + 8 s .. + 7.
//   P^T slot s: tokens 4 s + 0..3, then 16 + 4 s + 0..3.
__device__ __forceinline__ int xrow_off(int row, int slot16) { return row * 64 + 16 * (slot16 ^ ((row >> 1) & 3)); }

// One unit of work: half `hf` of page `pi` of sequence `b`, with that
// sequence's length L and end page pg1 inside the range (so stepping through a
// sequence reads no metadata).
struct XUnit {
  int b, pi, hf, L, pg1;
};

// First unit at or after sequence b inside range r (b > r.end_b when there is none).
__device__ __forceinline__ XUnit x_seek(const DecodeParams& p, const Range& r, int b) {
  for (; b <= r.end_b; ++b) {
    int L, pg0, pg1;
    seq_pages(p, r, b, L, pg0, pg1);
    if (pg0 < pg1) return XUnit{b, pg0, 0, L, pg1};
  }
  return XUnit{r.end_b + 1, 0, 0, 0, 0};
}

// Next unit after u inside range r.
__device__ __forceinline__ XUnit x_next(const DecodeParams& p, const Range& r, const XUnit& u) {
  if (u.hf == 0 && u.L - u.pi * kPage > kXHalf) return XUnit{u.b, u.pi, 1, u.L, u.pg1};
  if (u.pi + 1 < u.pg1) return XUnit{u.b, u.pi + 1, 0, u.L, u.pg1};
  return x_seek(p, r, u.b + 1);
}

// bf16 unit layout in LDS (32 tokens x 1152 B = 36 KB), chunk-group major:
// 16-byte chunk c of token t sits at
//   4096 (c / 8) + 128 t + 16 ((c % 8) ^ (t % 8)).
// Each 128-byte column block of the 32 rows is 4 KB; inside it the XOR keeps
// the K reads (16 consecutive tokens, one chunk) and the transposed V reads
// (4 tokens x 2 chunks per 16 lanes) on distinct banks, as with 1152-byte
// rows (consecutive tokens again sit half a bank window apart). This layout
// lets one direct load cover 8 tokens x 128 B with a per-lane source offset
// that does not depend on the load: lane l reads token l / 8 of the block,
// chunk (l % 8) ^ (l / 8).
__device__ __forceinline__ int xk_off(int t, int c) { return 4096 * (c >> 3) + 128 * t + 16 * ((c & 7) ^ (t & 7)); }

// Per-lane source offset of the direct loads (bf16: above, the load-dependent
// part goes into the scalar offset; FP8: records land unchanged and the part
// of the last load past the 32 records lies outside the buffer and reads
// zeros -- one offset per load).
template <int FMT>
__device__ __forceinline__ uint32_t x_load_off(int k, int lane, int st) {
  if constexpr (FMT == kFmtFp8) {
    const int x = 1024 * k + 16 * lane;
    const int t = x / kFp8Record;
    return static_cast<uint32_t>(t * st + (x - kFp8Record * t));
  } else {
    (void)k;
    return static_cast<uint32_t>((lane >> 3) * st + 16 * ((lane & 7) ^ (lane >> 3)));
  }
}

// Buffer resource word 3 for raw (unformatted, stride 0) buffer access on gfx9-family GPUs.
constexpr int kRawBufferWord3 = 0x00020000;

// Issue the direct loads of one FP8 unit (32 records starting at `src`, token
// stride `st`) into `dst` (waves 0 .. 3 issue them): MUBUF loads to LDS
// (buffer_load_dwordx4 ... lds), 16 bytes per lane, with the unit as the
// buffer (the part of the last load past the 32 records reads zeros). Load k
// brings LDS bytes 1024 k .. + 1023 of the records. The buffer form keeps the
// LDS read waits of the compute phases partial (the FLAT form makes every LDS
// wait a full drain while a load is in flight).
__device__ __forceinline__ void x_issue(const uint8_t* src, uint8_t* dst, int wave, const uint32_t (&off)[6], int st) {
  using X = XLayout;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), 0, kXHalf * st, kRawBufferWord3);
#pragma unroll
  for (int j = 0; j < X::kLoadsPerWave; ++j) {
    const int k = wave + kLoadWaves * j;
    if (k < X::kLoads)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, dst + 1024 * k), 16, off[j], 0, 0, kPageLoadPolicy);
  }
}

// Lane-constant indices. MFMA 16x16x32: lane l supplies A[i = l % 16][k-slots
// 8 (l / 16) .. + 7] and B[the same k-slots][j = l % 16]; D register i of lane
// l is D[4 (l / 16) + i][l % 16].
struct XLane {
  int tid, lane, wave;
  int r16, q4;          // lane % 16, lane / 16
  int k_off[2];         // S phase: K row r16, logical chunks q4 and 4 + q4 (swizzled), bytes
  int v_off[4];         // PV phase: transposed V read offsets, by 16-dim block d & 3
  uint32_t ld_off[6];   // FP8 direct loads: per-lane source offset of each load
};

// One unit of the FP8 pipeline. `cur` holds the unit (32 FP8 records), `nxt`
// receives the next unit, `work` is the LDS after the ring (conversion
// buffers, P^T, rescale factors, flag, Q^T chunks). The regions are disjoint;
// the restrict qualifiers let the compiler see that the LDS reads of this
// unit never touch the direct loads in flight into `nxt`.
__device__ __forceinline__ void x_step(uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt,
                                       uint8_t* __restrict__ work, const uint8_t* next_src, int st, const XLane& ln,
                                       int L, int last_ok, int tok0, int valid, bool this_ok, float scale_log2,
                                       int unit_id, const bf16x8 (&qf)[XLayout::kRegChunks], f32x4 (&acc)[4][8],
                                       float& m_run, float& l_run) {
  using X = XLayout;
  const int tid = ln.tid, wave = ln.wave, r16 = ln.r16, q4 = ln.q4;
  uint8_t* const lds = work - X::kConv;
  const float* sct = reinterpret_cast<const float*>(lds + X::kScale);   // [group][token] scales

  // ---- stage the unit: codes -> bf16 rows, RoPE and scales copied; rows past the end -> 0 --
  uint8_t* const page = lds + X::kConv;           // bf16 rows (chunk-group-major, swizzled)
  {
    uint8_t* conv = page;
    float* scw = reinterpret_cast<float*>(lds + X::kScale);
    if (tid < 4 * kXHalf) {
      const int g = tid >> 5, t = tid & 31;
      scw[tid] = (this_ok && t < valid) ? *reinterpret_cast<const float*>(cur + t * kFp8Record + 512 + 4 * g) : 0.f;
    }
#pragma unroll 1
    for (int j = 0; j < 2; ++j) {
      const int item = tid + kWThreads * j;         // 32 tokens x 32 chunks of 16 codes
      const int t = item >> 5, ch = item & 31;
      const u32x4 w = *reinterpret_cast<const u32x4*>(cur + t * kFp8Record + 16 * ch);
      u32x4 lo, hi;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t k01, k23;
        e4m3x4_to_bf16(w[i], k01, k23);
        if (i < 2) {
          lo[2 * i] = k01;
          lo[2 * i + 1] = k23;
        } else {
          hi[2 * i - 4] = k01;
          hi[2 * i - 3] = k23;
        }
      }
      if (!(this_ok && t < valid)) {
        lo = u32x4{0u, 0u, 0u, 0u};
        hi = lo;
      }
      *reinterpret_cast<u32x4*>(conv + xk_off(t, 2 * ch)) = lo;
      *reinterpret_cast<u32x4*>(conv + xk_off(t, 2 * ch + 1)) = hi;
    }
    if (tid < 8 * kXHalf) {
      const int t = tid >> 3, rr = tid & 7;         // 32 tokens x 8 RoPE chunks
      u32x4 w = *reinterpret_cast<const u32x4*>(cur + t * kFp8Record + 528 + 16 * rr);
      if (!(this_ok && t < valid)) w = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(conv + xk_off(t, 64 + rr)) = w;
    }
    lds_barrier_keep_loads();
  }

  // ---- the next unit -> nxt (waves 0 .. 3) ------------------------------------------------
  if (next_src != nullptr && wave < kLoadWaves) x_issue(next_src, nxt, wave, ln.ld_off, st);

  // ---- S phase: S^T[token 16 tt + 4 q4 + i][row 16 w + r16] --------------------------------
  const uint8_t* qlds = lds + X::kQ;
  auto qop = [&](int c) -> bf16x8 {
    const int qs = X::qslot(c);
    if (qs >= 0)
      return *reinterpret_cast<const bf16x8*>(qlds + qs * X::kQChunkBytes + xrow_off(16 * wave + r16, q4));
    return qf[X::qreg(c)];
  };
  // K: token 16 tt + r16, dims 32 c + 8 q4 .. + 7 = logical chunk 8 (c / 2) + 4 (c & 1) + q4
  auto kload = [&](int c, int tt) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(page + ln.k_off[c & 1] + 16 * tt * 128 + 4096 * (c >> 1));
  };
  f32x4 s[2];                                     // [token tile]
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // chunk order: the RoPE chunks 16, 17 first (unscaled), then the 4 latent
  // groups of 4 chunks, each group's partial logits scaled and added
  auto corder = [](int i) { return i < 2 ? 16 + i : i - 2; };
  // (padding rows of the last tile run through the phases like real rows: their
  // Q^T is zero and nothing of theirs is written)
  {
    // the K and Q^T operands of chunk i + 1 are read while chunk i's MFMAs run
    bf16x8 kbuf[2][2], qbuf[2];
    f32x4 part[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) kbuf[0][tt] = kload(corder(0), tt);
    qbuf[0] = qop(corder(0));
#pragma unroll
    for (int i = 0; i < 18; ++i) {
      if (i + 1 < 18) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) kbuf[(i + 1) & 1][tt] = kload(corder(i + 1), tt);
        qbuf[(i + 1) & 1] = qop(corder(i + 1));
      }
      const bf16x8 qv = qbuf[i & 1];
      if (i < 2) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kbuf[i & 1][tt], qv, s[tt], 0, 0, 0);
      } else {
        const int g = (i - 2) >> 2, j = (i - 2) & 3;
        if (j == 0) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) part[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          part[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kbuf[i & 1][tt], qv, part[tt], 0, 0, 0);
        if (j == 3) {
          // tokens 16 tt + 4 q4 + 0..3 of this lane, scale group g
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const f32x4 sc = *reinterpret_cast<const f32x4*>(sct + g * kXHalf + 16 * tt + 4 * q4);
#pragma unroll
            for (int e = 0; e < 4; ++e) s[tt][e] += sc[e] * part[tt][e];
          }
        }
      }
    }
  }

  // ---- softmax of this wave's rows; P^T, rescale factor and a flag -> LDS -----------------
  uint8_t* pbuf = lds + X::kP;
  float* alpha_buf = reinterpret_cast<float*>(lds + X::kAlpha);
  int* flags = reinterpret_cast<int*>(lds + X::kFlag);
  // token tok0 + 16 tt + 4 q4 + i is allowed iff 16 tt + i <= lim
  const int lim = min(L - 1, last_ok) - tok0 - 4 * q4;
  float mx = kNegInf;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = (16 * tt + i <= lim) ? s[tt][i] * scale_log2 : kNegInf;
      s[tt][i] = v;
      mx = fmaxf(mx, v);
    }
  mx = max4lanes(mx);
  // the running max moves only when it grows by more than the slack; a row's
  // first allowed tokens need no rescale (its O and l are still 0)
  const bool grow = mx > m_run + kRescaleSlack;
  const bool had = m_run != kNegInf;
  const float alpha = (grow && had) ? fast_exp2(m_run - mx) : 1.f;
  const bool rescaled = grow && had;
  l_run *= alpha;
  m_run = grow ? mx : m_run;
  const float m_use = (m_run == kNegInf) ? 0.f : m_run;
  bf16x8 pv;
  float psum = 0.f;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = fast_exp2(s[tt][i] - m_use);
      psum += e;
      pv[4 * tt + i] = static_cast<__bf16>(e);
    }
  l_run += psum;
  {
    const int row = 16 * wave + r16;
    // slot q4 of the row holds tokens 4 q4 .. 4 q4 + 3 and 16 + 4 q4 .. 16 + 4 q4 + 3
    *reinterpret_cast<bf16x8*>(pbuf + xrow_off(row, q4)) = pv;
    if (q4 == 0) alpha_buf[row] = alpha;
  }
  // one flag word: every wave with a rescaled row writes this unit's id there
  // (the same value, so concurrent writes agree)
  if (ln.lane == 0 && __builtin_amdgcn_ballot_w64(rescaled) != 0) flags[0] = unit_id;
  lds_barrier_keep_loads();

  // ---- PV phase: O^T[dim 64 w + 16 dd + 4 q4 + i][row 16 rr + r16] += V^T P^T -------------
  {
    // The flag word is read in inline asm (the wait inside the same block):
    // the compiler cannot tell that this fixed LDS address is not a target of
    // the direct loads in flight and would otherwise wait for all of them here.
    int fl;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(fl)
                 : "v"(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(flags)))
                 : "memory");
    if (__builtin_amdgcn_readfirstlane(fl) == unit_id) {
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const float a = alpha_buf[16 * rr + r16];
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) acc[dd][rr] *= a;
      }
    }
  }
  // transposed V reads: k-slots 0..3 = tokens 4 q4 + 0..3, 4..7 = the same + 16,
  // the token order of P^T slot q4; 16-dim block d = 4 w + dd
  bf16x8 va[4];
#pragma unroll
  for (int dd = 0; dd < 4; ++dd) {
    const uint8_t* a0 = page + ln.v_off[dd] + 4096 * wave;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, a0));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, a0 + 16 * 128));
    va[dd] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // this wave's dims are scale group w / 2: the per-token scales of its
  // k-slot tokens (4 q4 + 0..3, 16 + 4 q4 + 0..3) are folded into P^T
  const f32x4 sa = *reinterpret_cast<const f32x4*>(sct + (wave >> 1) * kXHalf + 4 * q4);
  const f32x4 sb = *reinterpret_cast<const f32x4*>(sct + (wave >> 1) * kXHalf + 16 + 4 * q4);
  auto pload = [&](int rr) -> bf16x8 {
    bf16x8 pb = *reinterpret_cast<const bf16x8*>(pbuf + xrow_off(16 * rr + r16, q4));
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(static_cast<float>(pb[e]) * (e < 4 ? sa[e] : sb[e - 4]));
    return pb;
  };
  bf16x8 pb[2];
  pb[0] = pload(0);
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    if (rr + 1 < 8) pb[(rr + 1) & 1] = pload(rr + 1);
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
      acc[dd][rr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dd], pb[rr & 1], acc[dd][rr], 0, 0, 0);
  }
}

__global__ void __launch_bounds__(kWThreads) splitkv_x_kernel(DecodeParams p) {
  using X = XLayout;
  constexpr int M_TILE = X::kRows;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[X::kTotal];

  XLane ln;
  ln.tid = threadIdx.x;
  ln.lane = ln.tid & 63;
  ln.wave = __builtin_amdgcn_readfirstlane(ln.tid >> 6);
  ln.r16 = ln.lane & 15;
  ln.q4 = ln.lane >> 4;
  {
    // K reads: token 16 tt + r16 (the swizzle depends on t % 8 only), chunk
    // 8 (c / 2) + 4 (c & 1) + q4: lane part for c even / odd, the rest immediate
    ln.k_off[0] = xk_off(ln.r16, ln.q4);
    ln.k_off[1] = xk_off(ln.r16, 4 + ln.q4);
    // transposed V reads: lane i of a 16-lane group addresses token 4 q4 + i / 4
    // (+16) and dims 4 (i % 4) .. + 3 of each 16-dim block
    const int tok = 4 * ln.q4 + (ln.r16 >> 2);
    const int hh = (ln.r16 & 3) >> 1, half8 = ln.r16 & 1;
#pragma unroll
    for (int e = 0; e < 4; ++e) ln.v_off[e] = xk_off(tok, 2 * e + hh) + 8 * half8;
  }
  const int tid = ln.tid, wave = ln.wave, r16 = ln.r16, q4 = ln.q4;
  const int st = static_cast<int>(p.kv_st);
#pragma unroll
  for (int j = 0; j < X::kLoadsPerWave; ++j)
    ln.ld_off[j] = x_load_off<kFmtFp8>((wave & (kLoadWaves - 1)) + kLoadWaves * j, ln.lane, st);

  // XCD-aware order: consecutive logical workgroups share an XCD (and its L2)
  const int per_xcd = gridDim.x / 8;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= p.grid_wgs) return;
  const int m_tiles = (p.rows + M_TILE - 1) / M_TILE;
  const int mt = logical % m_tiles;
  const int kvh = (logical / m_tiles) % p.h_kv;
  const int part = logical / (m_tiles * p.h_kv);

  Range r;
  if (!read_range(p, part, r)) return;

  if (tid == 0) reinterpret_cast<int*>(lds + X::kFlag)[0] = -1;

  // S-phase row of this lane
  const int srow = mt * M_TILE + 16 * wave + r16;
  const bool srow_ok = srow < p.rows;
  const int s_idx = srow_ok ? srow / p.group : 0;
  const int shead = kvh * p.group + (srow_ok ? srow % p.group : 0);

  const uint8_t* const kv_head = p.kv + kvh * p.kv_sh;
  // Page-address window: lane i holds the global address of page win_pi + i
  // of sequence win_b (0 for an entry past the row or outside the pool).
  // Refilled with one vector load of the block-table row when a unit falls
  // outside it (a new sequence, or every 64 pages), so a unit's address costs
  // two lane reads and an add.
  uint32_t win_lo = 0, win_hi = 0;
  int win_b = -1, win_pi = 0;
  const int64_t half_bytes = static_cast<int64_t>(kXHalf) * st;
  // global address of a unit (nullptr: block-table entry outside the pool)
  auto unit_src = [&](const XUnit& u) -> const uint8_t* {
    if (u.b != win_b || u.pi < win_pi || u.pi >= win_pi + 64) {
      win_b = u.b;
      win_pi = u.pi;
      const int e = u.pi + ln.lane;
      const int pg = e < p.max_blocks ? p.block_table[static_cast<int64_t>(u.b) * p.bt_stride + e] : -1;
      const uint64_t a = (pg >= 0 && pg < p.num_pages)
                             ? reinterpret_cast<uint64_t>(kv_head + static_cast<int64_t>(pg) * p.kv_sp)
                             : 0ull;
      win_lo = static_cast<uint32_t>(a);
      win_hi = static_cast<uint32_t>(a >> 32);
      wait_vm_all();
    }
    const uint32_t lo = __builtin_amdgcn_readlane(win_lo, u.pi - win_pi);
    const uint32_t hi = __builtin_amdgcn_readlane(win_hi, u.pi - win_pi);
    const uint64_t a = (static_cast<uint64_t>(hi) << 32) | lo;
    if (a == 0) return nullptr;
    return reinterpret_cast<const uint8_t*>(a) + (u.hf ? half_bytes : 0);
  };

  // ---- prime the ring: the first unit in flight into slot 0 -------------------------------
  // uq = the next unit to compute, okq = its page is valid (a unit is issued
  // iff it is inside the range and ok)
  XUnit uq = x_seek(p, r, r.begin_b);
  bool okq = true;
  if (uq.b <= r.end_b) {
    const uint8_t* src = unit_src(uq);
    okq = src != nullptr;
    if (okq && wave < kLoadWaves) x_issue(src, lds + X::kRing, wave, ln.ld_off, st);
  }
  int slot = 0;
  int unit_id = 0;

  for (int b = r.begin_b; b <= r.end_b; ++b) {
    int L, pg0, pg1;
    bool len_ok;
    seq_pages(p, r, b, L, pg0, pg1, len_ok);
    const int split_idx = (b == r.begin_b) ? r.split0 : 0;
    const int slot0 = ld_meta(p.num_splits + b);
    const int nsplit = ld_meta(p.num_splits + b + 1) - slot0;
    const int last_ok = p.causal ? (L - p.s_q + s_idx) : (L - 1);

    // Q^T of this sequence: chunks 7..15 of the lane's row in VGPRs, chunks
    // 0..6, 16, 17 of all 128 rows in LDS
    bf16x8 qf[X::kRegChunks];
    {
      const uint16_t* qrow = p.q + b * p.q_sb + s_idx * p.q_ss + shead * p.q_sh;
#pragma unroll
      for (int c = 0; c < 18; ++c) {
        if (X::qslot(c) >= 0) continue;
        const u32x4 v = srow_ok ? *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * q4) : u32x4{0u, 0u, 0u, 0u};
        qf[X::qreg(c)] = __builtin_bit_cast(bf16x8, v);
      }
    }
    lds_barrier_keep_loads();                 // no wave still reads the previous sequence's Q^T chunks
    {
      // Q^T chunks of the 128 rows straight into LDS: one direct load per 16
      // rows of a chunk (lane l: row 16 i + l / 4, stored slot l % 4, i.e. the
      // logical slot (l % 4) ^ ((row >> 1) & 3)); rows past p.rows read zeros
      // (their offset lies outside the buffer)
      const uint16_t* qb = p.q + b * p.q_sb;
      const int q_bytes = 2 * static_cast<int>((p.s_q - 1) * p.q_ss + (p.h_q - 1) * p.q_sh + kDqk);
      const __amdgpu_buffer_rsrc_t qrsrc =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(qb), 0, q_bytes, kRawBufferWord3);
      const int lrow = ln.lane >> 2, pslot = ln.lane & 3;
#pragma unroll
      for (int j = 0; j < (X::kQChunks * 8 + kWW - 1) / kWW; ++j) {
        const int k = wave + kWW * j;
        if (k < X::kQChunks * 8) {
          const int qs = k >> 3, i = k & 7;
          const int row = 16 * i + lrow;
          const int sl = pslot ^ ((row >> 1) & 3);
          const int grow = mt * M_TILE + row;
          uint32_t off = 0xFFFFFFF0u;
          if (grow < p.rows) {
            const int sg = grow / p.group, hg = kvh * p.group + grow % p.group;
            off = static_cast<uint32_t>(2 * (sg * p.q_ss + hg * p.q_sh + 32 * X::qchunk(qs) + 8 * sl));
          }
          __builtin_amdgcn_raw_ptr_buffer_load_lds(qrsrc, LDS_PTR(void, lds + X::kQ + qs * X::kQChunkBytes + 1024 * i),
                                                   16, off, 0, 0, 0);
        }
      }
    }
    wait_vm_all();
    lds_barrier();

    float m_run = kNegInf, l_run = 0.f;
    f32x4 acc[4][8];                          // [16-dim block of this wave][16-row block]
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) acc[dd][rr] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool bad = r.stale || !len_ok;

    while (uq.b == b) {
      const XUnit u = uq;
      const bool this_ok = okq;
      bad |= !this_ok;
      wait_vm_all();                          // this wave's loads of u landed
      lds_barrier_keep_loads();               // every wave's loads of u landed; unit u - 1 is done everywhere
      const XUnit un = x_next(p, r, u);
      const uint8_t* src_n = nullptr;
      bool ok_n = true;
      if (un.b <= r.end_b) {
        src_n = unit_src(un);
        ok_n = src_n != nullptr;
      }
      const int tok0 = u.pi * kPage + u.hf * kXHalf;
      const int valid = min(L - tok0, kXHalf);
      x_step(lds + X::kRing + slot * X::kSlot, lds + X::kRing + (slot ^ 1) * X::kSlot, lds + X::kConv, src_n, st,
                  ln, L, last_ok, tok0, valid, this_ok, p.scale_log2, unit_id, qf, acc, m_run, l_run);
      ++unit_id;
      slot ^= 1;
      uq = un;
      okq = ok_n;
    }

    // ---- epilogue: l of every row through LDS; each wave writes its 64 dims ----
    lds_barrier_keep_loads();                 // the P^T buffer is free
    float* lrow = reinterpret_cast<float*>(lds + X::kP);   // [rows] l
    {
      const float l_tot = sum4lanes(l_run);
      if (q4 == 0) lrow[16 * wave + r16] = l_tot;
      if (q4 == 0 && srow_ok) {
        float lse = (l_tot > 0.f) ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
        if (bad) lse = __builtin_nanf("");
        if (nsplit == 1)
          p.lse[(static_cast<int64_t>(b) * p.h_q + shead) * p.s_q + s_idx] = lse;
        else if (slot0 + split_idx < p.max_slots && split_idx < nsplit)
          p.part_lse[(static_cast<int64_t>(slot0 + split_idx) * p.h_kv + kvh) * p.rows + srow] = lse;
      }
    }
    lds_barrier_keep_loads();
    // lane l holds, per (dd, rr), row 16 rr + r16 and dims 64 w + 16 dd + 4 q4 + 0..3
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int rloc = 16 * rr + r16;
      const int row = mt * M_TILE + rloc;
      if (row >= p.rows) continue;
      const float l_row = lrow[rloc];
      const float inv = (l_row > 0.f) ? 1.f / l_row : 0.f;
      const int si = row / p.group, hh = kvh * p.group + row % p.group;
      if (nsplit == 1) {
        uint16_t* orow = p.o + ((static_cast<int64_t>(b) * p.s_q + si) * p.h_q + hh) * kDv + 64 * wave + 4 * q4;
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = bad ? nan : acc[dd][rr][i] * inv;
          u32x2 w;
          w[0] = static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
          w[1] = static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
          *reinterpret_cast<u32x2*>(orow + 16 * dd) = w;
        }
      } else {
        const int pslot = slot0 + split_idx;
        if (pslot >= 0 && pslot < p.max_slots && split_idx < nsplit) {
          // fp16 with a power-of-two scale per 64-dim block: this wave's dims are block `wave`
          const int64_t prow = (static_cast<int64_t>(pslot) * p.h_kv + kvh) * p.rows + mt * M_TILE + rloc;
          f32x4 v[4];
          float mx = 0.f;
#pragma unroll
          for (int dd = 0; dd < 4; ++dd)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              v[dd][i] = bad ? nan : acc[dd][rr][i] * inv;
              mx = fmaxf(mx, finite_abs(v[dd][i]));
            }
          float scl, bi;
          part_block_scale(max4lanes(mx), scl, bi);
          uint16_t* const po = p.part_o16 + prow * kDv + 64 * wave;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u32x2 a, c;
            a[0] = pack_f16x2(v[2 * h][0] * bi, v[2 * h][1] * bi);
            a[1] = pack_f16x2(v[2 * h][2] * bi, v[2 * h][3] * bi);
            c[0] = pack_f16x2(v[2 * h + 1][0] * bi, v[2 * h + 1][1] * bi);
            c[1] = pack_f16x2(v[2 * h + 1][2] * bi, v[2 * h + 1][3] * bi);
            int off;
            const u32x4 w = span_f16x8(a, c, q4, &off);
            *reinterpret_cast<u32x4*>(po + 32 * h + off) = w;
          }
          if (q4 == 0) p.part_scale[prow * kPartBlocks + wave] = scl;
        }
      }
    }
  }
  wait_vm_all();
}


// ----------------------------------------------------------------------------
// 128-row tiles, bf16 pages: one barrier per unit
//
// The same S / softmax / PV phases on 8 waves, but P^T, the rescale factors
// and the flag word are double-buffered by unit parity and the ring has three
// slots, so one barrier per unit suffices: between the barriers of units
// u - 1 and u a wave runs PV of u - 1 and then S and the softmax of u, and a
// wave that finishes PV early goes on with S while the others still multiply
// (the two waves on a SIMD drift into different phases). Rows past the
// sequence end read zeros straight from the loads (the buffer resource ends at
// the unit's last valid token), so the unit needs no zeroing pass.
// ----------------------------------------------------------------------------

struct X1Layout {
  static constexpr int kRows = 128;
  static constexpr int kSlot = kXHalfBytes;
  static constexpr int kSlots = 3;
  static constexpr int kRing = 0;
  static constexpr int kP = kRing + kSlots * kSlot;
  static constexpr int kPBytes = kRows * kXHalf * 2;          // one P^T buffer: 8 KB
  static constexpr int kAlpha = kP + 2 * kPBytes;             // [2][128] fp32
  static constexpr int kFlag = kAlpha + 2 * kRows * 4;        // [2] flag words (64 B reserved)
  static constexpr int kQ = kFlag + 64;
  static constexpr int kQChunks = 4;                          // Q^T chunks 0, 1, 16, 17 of all rows
  static constexpr int kQChunkBytes = kRows * 64;
  static constexpr int kTotal = kQ + kQChunks * kQChunkBytes;
  static constexpr int kLow = 2;
  static constexpr int qslot(int c) { return c < kLow ? c : (c >= 16 ? c - 16 + kLow : -1); }
  static constexpr int kRegChunks = 18 - kQChunks;
  static constexpr int qreg(int c) { return c - kLow; }
  static constexpr int qchunk(int qs) { return qs < kLow ? qs : 16 - kLow + qs; }
};
static_assert(X1Layout::kTotal <= 163840, "LDS budget");

// Direct loads of one bf16 unit (waves 0..3), the buffer ending after the
// unit's `valid` tokens: rows past them read zeros.
__device__ __forceinline__ void x1_issue(const uint8_t* src, int valid, uint8_t* dst, int wave, uint32_t off, int st) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), 0, valid * st, kRawBufferWord3);
#pragma unroll
  for (int j = 0; j < 9; ++j) {
    const int k = wave + kLoadWaves * j;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, dst + 1024 * k), 16, off, 8 * wave * st + 128 * j, 0,
                                             kPageLoadPolicy);
  }
}

// S phase and softmax of one unit for this wave's 16 rows; P^T, rescale factor
// and flag into the buffers of parity `par`.
__device__ __forceinline__ void x1_s(const uint8_t* __restrict__ page, uint8_t* __restrict__ work, const XLane& ln,
                                     int par, int L, int last_ok, int tok0, float scale_log2, int unit_id,
                                     const bf16x8 (&qf)[X1Layout::kRegChunks], float& m_run, float& l_run) {
  using X = X1Layout;
  const int wave = ln.wave, r16 = ln.r16, q4 = ln.q4;
  uint8_t* const lds = work - X::kP;
  const uint8_t* qlds = lds + X::kQ;
  auto qop = [&](int c) -> bf16x8 {
    const int qs = X::qslot(c);
    if (qs >= 0) return *reinterpret_cast<const bf16x8*>(qlds + qs * X::kQChunkBytes + xrow_off(16 * wave + r16, q4));
    return qf[X::qreg(c)];
  };
  auto kload = [&](int c, int tt) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(page + ln.k_off[c & 1] + 16 * tt * 128 + 4096 * (c >> 1));
  };
  f32x4 s[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    bf16x8 kbuf[2][2], qbuf[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) kbuf[0][tt] = kload(0, tt);
    qbuf[0] = qop(0);
#pragma unroll
    for (int c = 0; c < 18; ++c) {
      if (c + 1 < 18) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) kbuf[(c + 1) & 1][tt] = kload(c + 1, tt);
        qbuf[(c + 1) & 1] = qop(c + 1);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kbuf[c & 1][tt], qbuf[c & 1], s[tt], 0, 0, 0);
    }
  }
  const int lim = min(L - 1, last_ok) - tok0 - 4 * q4;
  float mx = kNegInf;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = (16 * tt + i <= lim) ? s[tt][i] * scale_log2 : kNegInf;
      s[tt][i] = v;
      mx = fmaxf(mx, v);
    }
  mx = max4lanes(mx);
  const bool grow = mx > m_run + kRescaleSlack;
  const bool had = m_run != kNegInf;
  const float alpha = (grow && had) ? fast_exp2(m_run - mx) : 1.f;
  const bool rescaled = grow && had;
  l_run *= alpha;
  m_run = grow ? mx : m_run;
  const float m_use = (m_run == kNegInf) ? 0.f : m_run;
  bf16x8 pv;
  float psum = 0.f;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = fast_exp2(s[tt][i] - m_use);
      psum += e;
      pv[4 * tt + i] = static_cast<__bf16>(e);
    }
  l_run += psum;
  const int row = 16 * wave + r16;
  *reinterpret_cast<bf16x8*>(lds + X::kP + par * X::kPBytes + xrow_off(row, q4)) = pv;
  if (q4 == 0) reinterpret_cast<float*>(lds + X::kAlpha)[par * X::kRows + row] = alpha;
  if (ln.lane == 0 && __builtin_amdgcn_ballot_w64(rescaled) != 0)
    reinterpret_cast<int*>(lds + X::kFlag)[par] = unit_id;
}

// PV phase of one unit (parity `par`): O^T[dims 64 w + 16 dd + 4 q4 + i][rows 16 rr + r16].
__device__ __forceinline__ void x1_pv(const uint8_t* __restrict__ page, uint8_t* __restrict__ work, const XLane& ln,
                                      int par, int unit_id, f32x4 (&acc)[4][8]) {
  using X = X1Layout;
  const int wave = ln.wave, r16 = ln.r16, q4 = ln.q4;
  uint8_t* const lds = work - X::kP;
  {
    // the flag word is read in inline asm (waited inside the block): the
    // compiler cannot tell that this fixed LDS address is not a target of the
    // direct loads in flight and would otherwise wait for all of them
    int fl;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(fl)
                 : "v"(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds + X::kFlag + 4 * par)))
                 : "memory");
    if (__builtin_amdgcn_readfirstlane(fl) == unit_id) {
      const float* alpha_buf = reinterpret_cast<const float*>(lds + X::kAlpha) + par * X::kRows;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const float a = alpha_buf[16 * rr + r16];
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) acc[dd][rr] *= a;
      }
    }
  }
  bf16x8 va[4];
#pragma unroll
  for (int dd = 0; dd < 4; ++dd) {
    const uint8_t* a0 = page + ln.v_off[dd] + 4096 * wave;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, a0));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, a0 + 16 * 128));
    va[dd] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  const uint8_t* pbuf = lds + X::kP + par * X::kPBytes;
  bf16x8 pb[2];
  pb[0] = *reinterpret_cast<const bf16x8*>(pbuf + xrow_off(r16, q4));
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    if (rr + 1 < 8) pb[(rr + 1) & 1] = *reinterpret_cast<const bf16x8*>(pbuf + xrow_off(16 * (rr + 1) + r16, q4));
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
      acc[dd][rr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dd], pb[rr & 1], acc[dd][rr], 0, 0, 0);
  }
}

__global__ void __launch_bounds__(kWThreads) splitkv_x1_kernel(DecodeParams p) {
  using X = X1Layout;
  constexpr int M_TILE = X::kRows;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[X::kTotal];

  XLane ln;
  ln.tid = threadIdx.x;
  ln.lane = ln.tid & 63;
  ln.wave = __builtin_amdgcn_readfirstlane(ln.tid >> 6);
  ln.r16 = ln.lane & 15;
  ln.q4 = ln.lane >> 4;
  {
    ln.k_off[0] = xk_off(ln.r16, ln.q4);
    ln.k_off[1] = xk_off(ln.r16, 4 + ln.q4);
    const int tok = 4 * ln.q4 + (ln.r16 >> 2);
    const int hh = (ln.r16 & 3) >> 1, half8 = ln.r16 & 1;
#pragma unroll
    for (int e = 0; e < 4; ++e) ln.v_off[e] = xk_off(tok, 2 * e + hh) + 8 * half8;
  }
  const int tid = ln.tid, wave = ln.wave, r16 = ln.r16, q4 = ln.q4;
  const int st = static_cast<int>(p.kv_st);
  const uint32_t ld_off = x_load_off<kFmtBf16>(0, ln.lane, st);

  const int per_xcd = gridDim.x / 8;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= p.grid_wgs) return;
  const int m_tiles = (p.rows + M_TILE - 1) / M_TILE;
  const int mt = logical % m_tiles;
  const int kvh = (logical / m_tiles) % p.h_kv;
  const int part = logical / (m_tiles * p.h_kv);

  Range r;
  if (!read_range(p, part, r)) return;

  if (tid < 2) reinterpret_cast<int*>(lds + X::kFlag)[tid] = -1;

  const int srow = mt * M_TILE + 16 * wave + r16;
  const bool srow_ok = srow < p.rows;
  const int s_idx = srow_ok ? srow / p.group : 0;
  const int shead = kvh * p.group + (srow_ok ? srow % p.group : 0);

  const uint8_t* const kv_head = p.kv + kvh * p.kv_sh;
  uint32_t win_lo = 0, win_hi = 0;
  int win_b = -1, win_pi = 0;
  const int64_t half_bytes = static_cast<int64_t>(kXHalf) * st;
  auto unit_src = [&](const XUnit& u) -> const uint8_t* {
    if (u.b != win_b || u.pi < win_pi || u.pi >= win_pi + 64) {
      win_b = u.b;
      win_pi = u.pi;
      const int e = u.pi + ln.lane;
      const int pg = e < p.max_blocks ? p.block_table[static_cast<int64_t>(u.b) * p.bt_stride + e] : -1;
      const uint64_t a = (pg >= 0 && pg < p.num_pages)
                             ? reinterpret_cast<uint64_t>(kv_head + static_cast<int64_t>(pg) * p.kv_sp)
                             : 0ull;
      win_lo = static_cast<uint32_t>(a);
      win_hi = static_cast<uint32_t>(a >> 32);
      wait_vm_all();
    }
    const uint32_t lo = __builtin_amdgcn_readlane(win_lo, u.pi - win_pi);
    const uint32_t hi = __builtin_amdgcn_readlane(win_hi, u.pi - win_pi);
    const uint64_t a = (static_cast<uint64_t>(hi) << 32) | lo;
    if (a == 0) return nullptr;
    return reinterpret_cast<const uint8_t*>(a) + (u.hf ? half_bytes : 0);
  };
  auto unit_valid = [&](const XUnit& u) { return min(u.L - (u.pi * kPage + u.hf * kXHalf), kXHalf); };

  // ---- prime the ring: units 0 and 1 into slots 0 and 1 ---------------------------------
  XUnit uq[2];
  bool okq[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i == 0)
      uq[0] = x_seek(p, r, r.begin_b);
    else
      uq[1] = (uq[0].b <= r.end_b) ? x_next(p, r, uq[0]) : uq[0];
    okq[i] = true;
    if (uq[i].b <= r.end_b) {
      const uint8_t* src = unit_src(uq[i]);
      okq[i] = src != nullptr;
      if (okq[i] && wave < kLoadWaves) x1_issue(src, unit_valid(uq[i]), lds + X::kRing + i * X::kSlot, wave, ld_off, st);
    }
  }
  int slot = 0;
  int unit_id = 0;
  uint8_t* const work = lds + X::kP;

  for (int b = r.begin_b; b <= r.end_b; ++b) {
    int L, pg0, pg1;
    bool len_ok;
    seq_pages(p, r, b, L, pg0, pg1, len_ok);
    const int split_idx = (b == r.begin_b) ? r.split0 : 0;
    const int slot0 = ld_meta(p.num_splits + b);
    const int nsplit = ld_meta(p.num_splits + b + 1) - slot0;
    const int last_ok = p.causal ? (L - p.s_q + s_idx) : (L - 1);

    bf16x8 qf[X::kRegChunks];
    {
      const uint16_t* qrow = p.q + b * p.q_sb + s_idx * p.q_ss + shead * p.q_sh;
#pragma unroll
      for (int c = 0; c < 18; ++c) {
        if (X::qslot(c) >= 0) continue;
        const u32x4 v = srow_ok ? *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * q4) : u32x4{0u, 0u, 0u, 0u};
        qf[X::qreg(c)] = __builtin_bit_cast(bf16x8, v);
      }
    }
    lds_barrier_keep_loads();                 // no wave still reads the previous sequence's Q^T chunks
    {
      const uint16_t* qb = p.q + b * p.q_sb;
      const int q_bytes = 2 * static_cast<int>((p.s_q - 1) * p.q_ss + (p.h_q - 1) * p.q_sh + kDqk);
      const __amdgpu_buffer_rsrc_t qrsrc =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(qb), 0, q_bytes, kRawBufferWord3);
      const int lrow = ln.lane >> 2, pslot = ln.lane & 3;
#pragma unroll
      for (int j = 0; j < (X::kQChunks * 8 + kWW - 1) / kWW; ++j) {
        const int k = wave + kWW * j;
        if (k < X::kQChunks * 8) {
          const int qs = k >> 3, i = k & 7;
          const int row = 16 * i + lrow;
          const int sl = pslot ^ ((row >> 1) & 3);
          const int grow = mt * M_TILE + row;
          uint32_t off = 0xFFFFFFF0u;
          if (grow < p.rows) {
            const int sg = grow / p.group, hg = kvh * p.group + grow % p.group;
            off = static_cast<uint32_t>(2 * (sg * p.q_ss + hg * p.q_sh + 32 * X::qchunk(qs) + 8 * sl));
          }
          __builtin_amdgcn_raw_ptr_buffer_load_lds(qrsrc, LDS_PTR(void, lds + X::kQ + qs * X::kQChunkBytes + 1024 * i),
                                                   16, off, 0, 0, 0);
        }
      }
    }
    wait_vm_all();                            // Q, and every unit in flight, landed
    lds_barrier();

    float m_run = kNegInf, l_run = 0.f;
    f32x4 acc[4][8];
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) acc[dd][rr] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool bad = r.stale || !len_ok;

    // Invariant at the top: unit uq[0] is in LDS and visible to every wave,
    // the loads of uq[1] (if any) are in flight or landed.
    while (uq[0].b == b) {
      const XUnit u = uq[0];
      bad |= !okq[0];
      const int par = unit_id & 1;
      uint8_t* const cur = lds + X::kRing + slot * X::kSlot;
      const int tok0 = u.pi * kPage + u.hf * kXHalf;
      x1_s(cur, work, ln, par, L, last_ok, tok0, p.scale_log2, unit_id, qf, m_run, l_run);
      wait_vm_all();                          // this wave's loads of uq[1] landed
      lds_barrier_keep_loads();               // P^T of u and uq[1] visible; every wave is past PV of u - 1
      const XUnit un = (uq[1].b <= r.end_b) ? x_next(p, r, uq[1]) : uq[1];
      bool ok_n = true;
      if (un.b <= r.end_b) {
        const uint8_t* src_n = unit_src(un);
        ok_n = src_n != nullptr;
        // the slot of u - 1: its last reader was PV of u - 1, before this barrier
        if (ok_n && wave < kLoadWaves)
          x1_issue(src_n, unit_valid(un), lds + X::kRing + ((slot + 2) % 3) * X::kSlot, wave, ld_off, st);
      }
      x1_pv(cur, work, ln, par, unit_id, acc);
      ++unit_id;
      slot = (slot + 1) % 3;
      uq[0] = uq[1];
      okq[0] = okq[1];
      uq[1] = un;
      okq[1] = ok_n;
    }

    // ---- epilogue: l of every row through LDS; each wave writes its 64 dims ----
    lds_barrier_keep_loads();                 // every wave's PV is done: the P^T buffers are free
    float* lrow = reinterpret_cast<float*>(lds + X::kP);
    {
      const float l_tot = sum4lanes(l_run);
      if (q4 == 0) lrow[16 * wave + r16] = l_tot;
      if (q4 == 0 && srow_ok) {
        float lse = (l_tot > 0.f) ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
        if (bad) lse = __builtin_nanf("");
        if (nsplit == 1)
          p.lse[(static_cast<int64_t>(b) * p.h_q + shead) * p.s_q + s_idx] = lse;
        else if (slot0 + split_idx < p.max_slots && split_idx < nsplit)
          p.part_lse[(static_cast<int64_t>(slot0 + split_idx) * p.h_kv + kvh) * p.rows + srow] = lse;
      }
    }
    lds_barrier_keep_loads();
    const float nan = __builtin_nanf("");
    // The lane's row is made opaque here so that the row-dependent address arithmetic
    // below is done here: hoisted out of the sequence loop it was spilled, and every
    // reload of a spilled value waited for all the stores in flight.
    int lane_row = r16;
    asm volatile("" : "+v"(lane_row));
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int rloc = 16 * rr + lane_row;
      const int row = mt * M_TILE + rloc;
      if (row >= p.rows) continue;
      const float l_row = lrow[rloc];
      const float inv = (l_row > 0.f) ? 1.f / l_row : 0.f;
      const int si = row / p.group, hh = kvh * p.group + row % p.group;
      if (nsplit == 1) {
        uint16_t* orow = p.o + ((static_cast<int64_t>(b) * p.s_q + si) * p.h_q + hh) * kDv + 64 * wave + 4 * q4;
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = bad ? nan : acc[dd][rr][i] * inv;
          u32x2 w;
          w[0] = static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
          w[1] = static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
          *reinterpret_cast<u32x2*>(orow + 16 * dd) = w;
        }
      } else {
        const int pslot = slot0 + split_idx;
        if (pslot >= 0 && pslot < p.max_slots && split_idx < nsplit) {
          // fp16 with a power-of-two scale per 64-dim block: this wave's dims are block `wave`
          const int64_t prow = (static_cast<int64_t>(pslot) * p.h_kv + kvh) * p.rows + mt * M_TILE + rloc;
          f32x4 v[4];
          float mx = 0.f;
#pragma unroll
          for (int dd = 0; dd < 4; ++dd)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              v[dd][i] = bad ? nan : acc[dd][rr][i] * inv;
              mx = fmaxf(mx, finite_abs(v[dd][i]));
            }
          float scl, bi;
          part_block_scale(max4lanes(mx), scl, bi);
          uint16_t* const po = p.part_o16 + prow * kDv + 64 * wave;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u32x2 a, c;
            a[0] = pack_f16x2(v[2 * h][0] * bi, v[2 * h][1] * bi);
            a[1] = pack_f16x2(v[2 * h][2] * bi, v[2 * h][3] * bi);
            c[0] = pack_f16x2(v[2 * h + 1][0] * bi, v[2 * h + 1][1] * bi);
            c[1] = pack_f16x2(v[2 * h + 1][2] * bi, v[2 * h + 1][3] * bi);
            int off;
            const u32x4 w = span_f16x8(a, c, q4, &off);
            *reinterpret_cast<u32x4*>(po + 32 * h + off) = w;
          }
          if (q4 == 0) p.part_scale[prow * kPartBlocks + wave] = scl;
        }
      }
    }
  }
  wait_vm_all();
}

}  // namespace

hipError_t launch_split_x(const DecodeParams& p, int kv_format, int rows_per_wave, int grid, hipStream_t stream,
                          hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (rows_per_wave != 32) return hipErrorInvalidValue;
  const dim3 g(grid), blk(kWThreads);
  if (kv_format == kFmtFp8)
    hipExtLaunchKernelGGL(splitkv_x_kernel, g, blk, 0, stream, ev_start, ev_stop, 0, p);
  else
    hipExtLaunchKernelGGL(splitkv_x1_kernel, g, blk, 0, stream, ev_start, ev_stop, 0, p);
  return hipGetLastError();
}

}  // namespace mla
