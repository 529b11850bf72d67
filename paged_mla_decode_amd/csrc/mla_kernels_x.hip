// mla_kernels_x.hip -- split-KV MLA decode kernels for more than 64 query rows
// per KV head on gfx950 (MI355X): 128-row tiles, 8 wavefronts, one barrier per
// 32-token unit (splitkv_x1_kernel, instantiated for bf16 pages and for FP8
// records).
//
// Same computation as the 64-row kernel in mla_kernels.hip (softmax attention
// of query rows over a sequence's cached latent rows, V = their first 512
// dims; pieces of a sequence leave partial O / LSE for the combine kernel:
// wmrh.cn FlashMLA深度解析, "计算流水线设计"), organised so that V is read from
// LDS once per workgroup and two wavefronts share each SIMD.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

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
// work. Work advances in units of 32 tokens (half a page) through a three-slot
// ring; both cache formats share the phases:
//   S phase  -- wave w owns rows 16w .. 16w + 15: S^T = K Q^T on MFMA
//               (A = 16 tokens of K from LDS, B = Q^T of the wave's rows).
//   exchange -- each wave writes bf16 P^T of its rows, its rescale factors
//               and a flag; one barrier.
//   PV phase -- wave w accumulates O^T for value dims 64w .. 64w + 63 of all
//               128 rows (128 accumulator registers): it reads only its
//               eighth of V (transposed) and every wave's P^T.
// ----------------------------------------------------------------------------

constexpr int kWW = 8;                                      // wavefronts per workgroup
constexpr int kWThreads = 64 * kWW;
constexpr int kLoadWaves = 4;                               // waves that issue the unit loads
constexpr int kXHalf = 32;                                  // tokens per unit
constexpr int kXHalfBytes = kXHalf * kRowBytes;             // 36864 = 36 x 1 KB: bf16 rows

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

// Per-lane source offset of a unit's direct loads: lane l reads token l / 8 of
// an 8-token block, chunk (l % 8) ^ (l / 8) of a 128-byte column block (the
// layout above); the load-dependent part (which 8 tokens, which column block)
// goes into the scalar offset. FP8 units use it for their code and RoPE chunks.
__device__ __forceinline__ uint32_t x_load_off(int lane, int st) {
  return static_cast<uint32_t>((lane >> 3) * st + 16 * ((lane & 7) ^ (lane >> 3)));
}

// Buffer resource word 3 for raw (unformatted, stride 0) buffer access on gfx9-family GPUs.
constexpr int kRawBufferWord3 = 0x00020000;

// Lane-constant indices. MFMA 16x16x32: lane l supplies A[i = l % 16][k-slots
// 8 (l / 16) .. + 7] and B[the same k-slots][j = l % 16]; D register i of lane
// l is D[4 (l / 16) + i][l % 16].
struct XLane {
  int tid, lane, wave;
  int r16, q4;          // lane % 16, lane / 16
  int k_off[2];         // S phase: K row r16, logical chunks q4 and 4 + q4 (swizzled), bytes
  int v_off[4];         // PV phase: transposed V read offsets, by 16-dim block d & 3
};

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
// SPARSE: token 16 tt + 4 q4 + i of the unit is masked unless bit (16 tt + 4 q4 + i) of tokmask is set.
template <bool SPARSE>
__device__ __forceinline__ void x1_s(const uint8_t* __restrict__ page, uint8_t* __restrict__ work, const XLane& ln,
                                     int par, int L, int last_ok, int tok0, float scale_log2, int unit_id,
                                     const bf16x8 (&qf)[X1Layout::kRegChunks], float& m_run, float& l_run,
                                     uint32_t tokmask) {
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
  // the attend bits of this lane's 8 tokens (4 q4 + i, 16 + 4 q4 + i), taken here so that the
  // shifts are not spread over the MFMA phase above
  uint32_t m8 = 0xFFu;
  if constexpr (SPARSE) {
    m8 = ((tokmask >> (4 * q4)) & 0xFu) | (((tokmask >> (16 + 4 * q4)) & 0xFu) << 4);
    asm volatile("" : "+v"(m8));
  }
  float mx = kNegInf;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool allowed = (16 * tt + i <= lim) && (!SPARSE || ((m8 >> (4 * tt + i)) & 1u));
      const float v = allowed ? s[tt][i] * scale_log2 : kNegInf;
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

// ----------------------------------------------------------------------------
// 128-row tiles, FP8 pages: the same one-barrier pipeline, without a
// conversion pass.
//
// S phase: the e4m3 codes of K multiply Q on the scaled FP8 MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4). Q (bf16) is split exactly into two
// e4m3 parts per row: hi = rne(q 2^-s) and lo = (q 2^-s - hi) 16, both with
// E8M0 block scales (2^s and 2^(s-4)) that the MFMA applies; for every element
// whose hi part is a normal e4m3 value, hi 2^s + lo 2^(s-4) = q exactly (the
// residual of rounding an 8-bit significand to 4 bits has at most 4 bits), so
// the products are those of the exact codes and q, as in bf16. Two FP8 MFMAs
// per 128 dims take the time of four bf16 ones: the S phase costs what it
// costs on bf16 pages and no code is converted. The fp32 scales of the 4
// latent groups multiply the per-group partial logits; RoPE runs on bf16 MFMA.
// PV phase: V^T comes straight from the codes with the transposing byte read
// (ds_read_b64_tr_b8), each code converted exactly and multiplied by its
// token's scale of the wave's value group, then rounded to bf16 for the MFMA.
//
// MFMA 16x16x128 operand layout (measured on gfx950): lane 16 g + i holds, for
// row i, the k-slots 16 g .. 16 g + 15 in bytes 0 .. 15 and 64 + 16 g .. + 15 in
// bytes 16 .. 31; the E8M0 scale of row i and k-block kb (k-slots 32 kb ..
// 32 kb + 31) is the scale operand of lane 16 kb + i. A (K codes) and B (Q
// codes) share the layout, so lane (r16, q4) carries dims 128 g + 16 q4 + 0..15
// and 128 g + 64 + 16 q4 + 0..15 of latent group g in both.
// ds_read_b64_tr_b8 (measured): within each 16-lane group, lane i receives as
// byte j the byte i % 8 of the 8 bytes lane 2 j + i / 8 addressed.
// ----------------------------------------------------------------------------

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(2))) int i32x2;

struct F8Layout {
  static constexpr int kRows = 128;
  // one unit of 32 raw records, rearranged by the direct loads: the latent
  // codes chunk-group major (code chunk c of token t at xk_off(t, c), 16 KB),
  // the RoPE chunks the same way (4 KB), then the fp32 scales group major
  // ([4 groups][32 tokens], 512 B: two 4-byte-per-lane loads)
  static constexpr int kCodes = 0;
  static constexpr int kRope = 16384;
  static constexpr int kScales = 20480;
  static constexpr int kSlot = kScales + 4 * kXHalf * 4;     // 20992
  static constexpr int kSlots = 3;
  static constexpr int kLoads = 22;
  static constexpr int kRing = 0;
  static constexpr int kP = kRing + kSlots * kSlot;
  static constexpr int kPBytes = kRows * kXHalf * 2;          // one P^T buffer: 8 KB
  static constexpr int kAlpha = kP + 2 * kPBytes;             // [2][128] fp32
  static constexpr int kFlag = kAlpha + 2 * kRows * 4;        // [2] flag words (64 B reserved)
  static constexpr int kQlo = kFlag + 64;                     // lo codes of Q: [128 rows][512 B]
  static constexpr int kQrope = kQlo + kRows * 512;           // RoPE dims of Q (bf16): [128 rows][128 B]
  static constexpr int kTotal = kQrope + kRows * 128;
};
static_assert(F8Layout::kTotal <= 163840, "LDS budget");

constexpr int kE8M0One = 127;                                 // E8M0 code of 1.0

// Byte offset of Q lo chunk c (16 codes; c = 8 g + 4 h + q4) of tile row R:
// 16-chunk groups XOR-swizzled by R % 16, so the 16 rows a read covers fall
// on 16 distinct 16-byte bank slots.
__device__ __forceinline__ int qlo_off(int R, int c) { return R * 512 + 16 * ((c & 16) | ((c & 15) ^ (R & 15))); }

// Direct loads of one FP8 unit (all 8 waves; load k = wave + 8 j): loads
// 0..15 the latent codes (group k / 4, tokens 8 (k % 4) .. + 7, 16 bytes per
// lane), 16..19 RoPE, 20 and 21 the scales (4 bytes per lane: load 20 + m,
// lane l holds scale 2 m + l / 32 of token l % 32). The buffer ends after the
// unit's `valid` tokens: rows past them read zeros. lane_off:
// (l / 8) st + 16 ((l % 8) ^ (l / 8)); scale_off: (l % 32) st + 512 + 4 (l / 32).
__device__ __forceinline__ void f8_issue(const uint8_t* src, int valid, uint8_t* dst, int wave, uint32_t lane_off,
                                         uint32_t scale_off, int st) {
  using X = F8Layout;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), 0, valid * st, kRawBufferWord3);
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int k = wave + kWW * j;
    if (k < 16) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, dst + 1024 * k), 16, lane_off,
                                               8 * (k & 3) * st + 128 * (k >> 2), 0, kPageLoadPolicy);
    } else if (k < 20) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, dst + 1024 * k), 16, lane_off,
                                               8 * (k & 3) * st + 528, 0, kPageLoadPolicy);
    } else if (k < X::kLoads) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, dst + X::kScales + 256 * (k - 20)), 4, scale_off,
                                               8 * (k - 20), 0, kPageLoadPolicy);
    }
  }
}

// Q of one sequence for this lane's row, in the operand forms of the S phase.
struct F8Q {
  i32x8 hi[4];          // hi codes of latent group g (MFMA 16x16x128 B operand)
  int scale_hi, scale_lo;   // E8M0 scale operands of the hi and lo MFMAs
};

// Byte offset of RoPE chunk c (8 dims: 512 + 32 (c / 4) + 8 (c % 4) ..) of tile row R in the
// Q RoPE region: 8 chunks per row, XOR-swizzled by R % 8.
__device__ __forceinline__ int qrope_off(int R, int c) { return R * 128 + 16 * (c ^ (R & 7)); }

// Split this lane's Q values (row srow, 0 when !row_ok) into hi / lo codes; the
// lo codes go to LDS (row R of the tile), the rest to q.
__device__ __forceinline__ void f8_qsetup(const uint16_t* qrow, bool row_ok, int R, int q4, uint8_t* lds, F8Q& q) {
  using X = F8Layout;
  // 16 chunks of 8 bf16: index 4 g + 2 h + k holds dims 128 g + 64 h + 16 q4 + 8 k .. + 7
  u32x4 raw[16];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int k = 0; k < 2; ++k)
        raw[4 * g + 2 * h + k] = row_ok ? *reinterpret_cast<const u32x4*>(qrow + 128 * g + 64 * h + 16 * q4 + 8 * k)
                                        : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const u32x4 v = row_ok ? *reinterpret_cast<const u32x4*>(qrow + 512 + 32 * c + 8 * q4) : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(lds + F8Layout::kQrope + qrope_off(R, 4 * c + q4)) = v;
  }
  auto lo16 = [](uint32_t w) { return __uint_as_float(w << 16); };
  auto hi16 = [](uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); };
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fmaxf(finite_abs(lo16(raw[i][e])), finite_abs(hi16(raw[i][e]))));
  mx = max4lanes(mx);
  // the row's values scaled by 2^-s stay below 2^8 (<= 448); the lo part's scale is 2^(s - 4)
  int e = __builtin_amdgcn_frexp_expf(mx);
  e = e < -100 ? -100 : e;
  const int s = e - 8;
  q.scale_hi = kE8M0One + s;
  q.scale_lo = kE8M0One + s - 4;
  const float inv = __builtin_amdgcn_ldexpf(1.f, -s);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 lo_chunk;
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {     // 4 code words of 4 codes: dims 8 k + 4 (w4 % 2) .. of chunk k = w4 / 2
        const uint32_t a = raw[4 * g + 2 * h + (w4 >> 1)][2 * (w4 & 1)];
        const uint32_t b = raw[4 * g + 2 * h + (w4 >> 1)][2 * (w4 & 1) + 1];
        const float x0 = lo16(a) * inv, x1 = hi16(a) * inv, x2 = lo16(b) * inv, x3 = hi16(b) * inv;
        int hw = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
        hw = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, hw, true);
        const auto d01 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);    // exact decode of the hi codes
        const auto d23 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
        int lw = __builtin_amdgcn_cvt_pk_fp8_f32((x0 - d01[0]) * 16.f, (x1 - d01[1]) * 16.f, 0, false);
        lw = __builtin_amdgcn_cvt_pk_fp8_f32((x2 - d23[0]) * 16.f, (x3 - d23[1]) * 16.f, lw, true);
        q.hi[g][4 * h + w4] = hw;
        lo_chunk[w4] = static_cast<uint32_t>(lw);
      }
      *reinterpret_cast<u32x4*>(lds + X::kQlo + qlo_off(R, 8 * g + 4 * h + q4)) = lo_chunk;
    }
  }
}

// S phase and softmax of one FP8 unit for this wave's 16 rows (as x1_s); also
// returns, for the PV phase, the scales of the lane's 8 tokens (k-slot order of
// P^T) in the wave's value group.
template <bool SPARSE>
__device__ __forceinline__ void f8_s(const uint8_t* __restrict__ page, uint8_t* __restrict__ work, const XLane& ln,
                                     int par, int L, int last_ok, int tok0, float scale_log2, int unit_id,
                                     const F8Q& q, float& m_run, float& l_run, uint32_t tokmask) {
  using X = F8Layout;
  const int wave = ln.wave, r16 = ln.r16, q4 = ln.q4;
  uint8_t* const lds = work - X::kP;
  const int R = 16 * wave + r16;
  const uint8_t* qlo = lds + X::kQlo;
  // K codes of token 16 tt + r16, latent group g: chunks 8 g + q4 and 8 g + 4 + q4
  auto kcodes = [&](int g, int tt) -> i32x8 {
    const u32x4 a = *reinterpret_cast<const u32x4*>(page + X::kCodes + ln.k_off[0] + 2048 * tt + 4096 * g);
    const u32x4 b = *reinterpret_cast<const u32x4*>(page + X::kCodes + ln.k_off[1] + 2048 * tt + 4096 * g);
    return i32x8{static_cast<int>(a[0]), static_cast<int>(a[1]), static_cast<int>(a[2]), static_cast<int>(a[3]),
                 static_cast<int>(b[0]), static_cast<int>(b[1]), static_cast<int>(b[2]), static_cast<int>(b[3])};
  };
  auto qlo_op = [&](int g) -> i32x8 {
    const u32x4 a = *reinterpret_cast<const u32x4*>(qlo + qlo_off(R, 8 * g + q4));
    const u32x4 b = *reinterpret_cast<const u32x4*>(qlo + qlo_off(R, 8 * g + 4 + q4));
    return i32x8{static_cast<int>(a[0]), static_cast<int>(a[1]), static_cast<int>(a[2]), static_cast<int>(a[3]),
                 static_cast<int>(b[0]), static_cast<int>(b[1]), static_cast<int>(b[2]), static_cast<int>(b[3])};
  };
  // RoPE part (bf16 MFMA): K dims 512 + 32 c + 8 q4 .. = RoPE chunk 4 c + q4.
  // Its operands and those of the first latent step are read up front; the
  // latent part then runs in 8 steps (group g, token tile tt), each step's
  // MFMAs covering the reads of the next step's K codes (and, before a group's
  // first step, of the group's lo codes of Q), so that a wait for one step's
  // operands leaves the next step's reads in flight.
  bf16x8 qr[2], kr[2][2];
#pragma unroll
  for (int c = 0; c < 2; ++c) qr[c] = *reinterpret_cast<const bf16x8*>(lds + X::kQrope + qrope_off(R, 4 * c + q4));
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int c = 0; c < 2; ++c) kr[tt][c] = *reinterpret_cast<const bf16x8*>(page + X::kRope + ln.k_off[c] + 2048 * tt);
  i32x8 kc[2], ql[2];
  kc[0] = kcodes(0, 0);
  ql[0] = qlo_op(0);
  f32x4 s[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 2; ++c) s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[tt][c], qr[c], s[tt], 0, 0, 0);
  }
  // latent groups: hi and lo MFMAs into one partial per token tile, then the
  // group's fp32 scales of tokens 16 tt + 4 q4 + i (scales are [group][token];
  // read at the group's second step, before that step's operand reads)
  auto scales4 = [&](int g, int tt) -> f32x4 {
    return *reinterpret_cast<const f32x4*>(page + X::kScales + 4 * (kXHalf * g + 16 * tt + 4 * q4));
  };
  f32x4 part[2], sg[2];
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    const int g = st >> 1, tt = st & 1;
    if (tt == 1) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) sg[t2] = scales4(g, t2);
    }
    if (st + 1 < 8) {
      kc[(st + 1) & 1] = kcodes((st + 1) >> 1, (st + 1) & 1);
      if (tt == 1) ql[(g + 1) & 1] = qlo_op(g + 1);
    }
    part[tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kc[st & 1], q.hi[g], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                                0, kE8M0One, 0, q.scale_hi);
    part[tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kc[st & 1], ql[g & 1], part[tt], 0, 0, 0, kE8M0One, 0,
                                                                q.scale_lo);
    if (tt == 1) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[t2][i] += sg[t2][i] * part[t2][i];
    }
  }

  const int lim = min(L - 1, last_ok) - tok0 - 4 * q4;
  // the attend bits of this lane's 8 tokens (4 q4 + i, 16 + 4 q4 + i), taken here so that the
  // shifts are not spread over the MFMA phase above
  uint32_t m8 = 0xFFu;
  if constexpr (SPARSE) {
    m8 = ((tokmask >> (4 * q4)) & 0xFu) | (((tokmask >> (16 + 4 * q4)) & 0xFu) << 4);
    asm volatile("" : "+v"(m8));
  }
  float mx = kNegInf;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool allowed = (16 * tt + i <= lim) && (!SPARSE || ((m8 >> (4 * tt + i)) & 1u));
      const float v = allowed ? s[tt][i] * scale_log2 : kNegInf;
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
  *reinterpret_cast<bf16x8*>(lds + X::kP + par * X::kPBytes + xrow_off(R, q4)) = pv;
  if (q4 == 0) reinterpret_cast<float*>(lds + X::kAlpha)[par * X::kRows + R] = alpha;
  if (ln.lane == 0 && __builtin_amdgcn_ballot_w64(rescaled) != 0)
    reinterpret_cast<int*>(lds + X::kFlag)[par] = unit_id;
}

// PV phase of one FP8 unit: O^T[dims 64 w + 16 dd + 4 q4 + i][rows 16 rr + r16] += V^T P^T,
// V^T from the codes (tr8 read, exact conversion, times the token's scale, bf16).
__device__ __forceinline__ void f8_pv(const uint8_t* __restrict__ page, uint8_t* __restrict__ work, const XLane& ln,
                                      int par, int unit_id, f32x4 (&acc)[4][8]) {
  using X = F8Layout;
  const int wave = ln.wave, r16 = ln.r16, q4 = ln.q4;
  uint8_t* const lds = work - X::kP;
  // scales of the lane's 8 P^T tokens (4 q4 + i, 16 + 4 q4 + i) in the wave's value group w / 2
  float pv_scale[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const f32x4 sg = *reinterpret_cast<const f32x4*>(page + X::kScales + 4 * (kXHalf * (wave >> 1) + 16 * tt + 4 * q4));
#pragma unroll
    for (int i = 0; i < 4; ++i) pv_scale[4 * tt + i] = sg[i];
  }
  {
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
  // Source lane 2 jj + h of 16-lane group q4 addresses token T(q4, jj) (the
  // token of P^T k-slot 8 q4 + jj: 4 q4 + jj, or 16 + 4 q4 + jj - 4 for
  // jj >= 4), dims D + 8 h .. + 7; after the transposing read, lane i holds
  // dim D + i of tokens T(q4, 0..7) in bytes 0..7 -- the k-slot order of its
  // P^T operand -- so byte j takes this lane's pv_scale[j].
  const int jj = r16 >> 1, hsel = r16 & 1;
  const int tok = (jj < 4) ? 4 * q4 + jj : 16 + 4 * q4 + (jj - 4);
  // all four transposing reads are issued before the first conversion waits
  i32x2 w[4];
#pragma unroll
  for (int dd = 0; dd < 4; ++dd) {
    const int c = 4 * wave + dd;                    // 16-dim code chunk of dims 64 w + 16 dd
    const uint8_t* a0 = page + X::kCodes + xk_off(tok, c) + 8 * hsel;
    w[dd] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i32x2, a0));
  }
  bf16x8 va[4];
#pragma unroll
  for (int dd = 0; dd < 4; ++dd) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(w[dd][h2], false);
      const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8(w[dd][h2], true);
      va[dd][4 * h2 + 0] = static_cast<__bf16>(f01[0] * pv_scale[4 * h2 + 0]);
      va[dd][4 * h2 + 1] = static_cast<__bf16>(f01[1] * pv_scale[4 * h2 + 1]);
      va[dd][4 * h2 + 2] = static_cast<__bf16>(f23[0] * pv_scale[4 * h2 + 2]);
      va[dd][4 * h2 + 3] = static_cast<__bf16>(f23[1] * pv_scale[4 * h2 + 3]);
    }
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


// ----------------------------------------------------------------------------
// Token-level sparse decode on the same pipeline. A unit is 32 consecutive
// entries of a (sequence, query token) pair's index list; lane j < 32 of every
// wave resolves entry j in three steps, one per pipeline iteration so that
// each memory round trip has an iteration to land: (A) load the index,
// (B) check it and load its block-table entry, (C) turn it into the byte
// offset of the token's row within the KV head's pool (kNoToken when the entry
// is padding, is dropped by the causal mask, or is invalid) and the unit's
// attend mask (bit j: entry j is attended). An invalid entry -- outside
// [-1, L_b), or a block-table entry outside the pool -- makes the pair's
// outputs NaN. The unit's loads then gather the rows from the pool (the buffer
// is the whole pool, so kNoToken reads zeros) into the same LDS layout as a
// dense unit, and the softmax masks with the attend mask.
// ----------------------------------------------------------------------------

constexpr uint32_t kNoToken = 0x80000000u;        // past any pool the sparse path accepts (< 2^31 bytes)

struct SparseTok {
  int t = -1;                // the index (step A), then -1 unless attended (step B)
  int page = -1;             // its block-table entry (step B)
  bool bad = false;          // the unit holds an invalid entry (uniform)
};

// The three steps keep their loads unconditional and apply each lane's validity one step
// later: a load under a lane condition is merged with its default value right after it is
// issued, and the wait for that value (vmcnt(0)) also waits for every unit load in flight.

// Step A: lane j < 32 loads entry j of unit u (lanes past the list, or past topk, read entry
// 0 of the list; step B drops them). Nothing past the range.
__device__ __forceinline__ int sparse_load_index(const DecodeParams& p, const Range& r, const XUnit& u, int kvh,
                                                 int lane) {
  if (u.b > r.end_b) return -1;
  const int j = u.pi * kPage + u.hf * kXHalf + lane;
  const bool in_list = lane < kXHalf && j < p.topk;
  const int b = __builtin_amdgcn_readfirstlane(u.b);
  const int br = b / p.sq_real, s = b - br * p.sq_real;
  return p.indices[br * p.idx_sb + s * p.idx_ss + kvh * p.idx_sh + (in_list ? j : 0)];
}

// Step B: validate the (landed) index, drop it unless attended, load its block-table entry
// (lanes that do not attend read entry 0 of the row; step C drops them).
__device__ __forceinline__ SparseTok sparse_load_page(const DecodeParams& p, const Range& r, const XUnit& u, int raw,
                                                      int lane) {
  SparseTok k;
  if (u.b > r.end_b) return k;
  const int b = __builtin_amdgcn_readfirstlane(u.b);
  const int br = b / p.sq_real, s = b - br * p.sq_real;
  const int L = real_len(p, br);
  const int max_len = p.max_blocks * kPage;
  const int j = u.pi * kPage + u.hf * kXHalf + lane;
  const bool in_list = lane < kXHalf && j < p.topk;
  const int idx = in_list ? raw : -1;
  const bool valid = idx == -1 || (idx >= 0 && idx < L && idx < max_len);
  const bool attend = in_list && idx >= 0 && valid && (!p.real_causal || idx <= L - p.sq_real + s);
  k.bad = __builtin_amdgcn_ballot_w64(in_list && !valid) != 0;
  k.t = attend ? idx : -1;
  if (p.kv_rows == 0 && p.max_blocks > 0)     // (contiguous rows: the page is taken in step C)
    k.page = p.block_table[static_cast<int64_t>(br) * p.bt_stride + (attend ? (idx >> 6) : 0)];
  return k;
}

// Step C: the byte offset of the row of the (landed) page entry, the attend mask, validity.
__device__ __forceinline__ uint32_t sparse_offset(const DecodeParams& p, SparseTok& k, uint32_t& mask) {
  const bool attend = k.t >= 0;
  // contiguous rows (kv_rows > 0): page t / 64 of the row array; else the block-table entry
  const int page = attend ? (p.kv_rows > 0 ? (k.t >> 6) : k.page) : -1;
  const bool page_ok = page >= 0 && page < p.num_pages;
  k.bad = k.bad || (__builtin_amdgcn_ballot_w64(attend && !page_ok) != 0);
  mask = static_cast<uint32_t>(__builtin_amdgcn_ballot_w64(attend && page_ok));
  return (attend && page_ok) ? static_cast<uint32_t>(static_cast<int64_t>(page) * p.kv_sp + (k.t & 63) * p.kv_st)
                             : kNoToken;
}

// Gathered loads of one sparse unit into an LDS slot: the layout of a dense unit,
// each token's row at its own offset (lane j of `off` holds token j's). bf16:
// waves 0..3, token 8 w + l / 8, column blocks 0..8; FP8: all waves, load
// k = w + 8 j of f8_issue (token 8 (w % 4) + l / 8; scales: token l % 32).
template <int FMT>
__device__ __forceinline__ void sparse_issue(const uint8_t* kv_head, int64_t pool_bytes, uint32_t off, uint8_t* dst,
                                             int wave, int lane) {
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kv_head), 0,
                                                                        static_cast<int>(pool_bytes), kRawBufferWord3);
  asm volatile("" : "+v"(lane));             // lane-derived offsets computed here, not held (and spilled)
  const uint32_t chunk = 16 * ((lane & 7) ^ (lane >> 3));
  if constexpr (FMT == kFmtFp8) {
    using X = F8Layout;
    const uint32_t tok = static_cast<uint32_t>(__shfl(static_cast<int>(off), 8 * (wave & 3) + (lane >> 3), 64));
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int k = wave + kWW * j;
      if (k < 16) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, dst + 1024 * k), 16, tok + chunk, 128 * (k >> 2),
                                                 0, kPageLoadPolicy);
      } else if (k < 20) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, dst + 1024 * k), 16, tok + chunk, 528, 0,
                                                 kPageLoadPolicy);
      } else if (k < X::kLoads) {
        const uint32_t stok = static_cast<uint32_t>(__shfl(static_cast<int>(off), lane & 31, 64));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, dst + X::kScales + 256 * (k - 20)), 4,
                                                 stok + 512 + 4 * (lane >> 5), 8 * (k - 20), 0, kPageLoadPolicy);
      }
    }
  } else {
    if (wave >= kLoadWaves) return;
    const uint32_t tok = static_cast<uint32_t>(__shfl(static_cast<int>(off), 8 * wave + (lane >> 3), 64));
#pragma unroll
    for (int j = 0; j < 9; ++j) {
      const int k = wave + kLoadWaves * j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, dst + 1024 * k), 16, tok + chunk, 128 * j, 0,
                                               kPageLoadPolicy);
    }
  }
}

template <int FMT, bool SPARSE>
__global__ void __launch_bounds__(kWThreads) splitkv_x1_kernel(DecodeParams p) {
  constexpr bool kFp8 = (FMT == kFmtFp8);
  using X = typename std::conditional<kFp8, F8Layout, X1Layout>::type;
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
  // issue the loads of one unit into a ring slot. The per-lane source offsets are computed
  // here from an opaque copy of the lane index, not held across the unit loop: held, they
  // were spilled, and the reload before the scale loads waited for every load in flight
  // (the unit's own code loads included), which made two waves late at every barrier.
  auto issue = [&](const uint8_t* src, int valid, uint8_t* dst) {
    int lane = ln.lane;
    asm volatile("" : "+v"(lane));
    const uint32_t ld_off = x_load_off(lane, st);
    if constexpr (kFp8) {
      const uint32_t scale_off = static_cast<uint32_t>((lane & 31) * st + 512 + 4 * (lane >> 5));
      f8_issue(src, valid, dst, wave, ld_off, scale_off, st);
    } else if (wave < kLoadWaves) {
      x1_issue(src, valid, dst, wave, ld_off, st);
    }
  };

  // This lane's S-phase row (row 16 wave + r16 of the tile) and its query token and head. They
  // are needed before and after the unit loop, not in it: recomputed from an opaque copy of r16
  // at each use so they are not held (and spilled) across the loop -- a spill reload waits for
  // every memory operation in flight, and the epilogue had several, each a memory round trip.
  struct RowIdx {
    int srow, s_idx, shead;
    bool ok;
  };
  auto row_idx = [&]() -> RowIdx {
    int rr = r16;
    asm volatile("" : "+v"(rr));
    RowIdx x;
    x.srow = mt * M_TILE + 16 * wave + rr;
    x.ok = x.srow < p.rows;
    x.s_idx = x.ok ? x.srow / p.group : 0;
    x.shead = kvh * p.group + (x.ok ? x.srow % p.group : 0);
    return x;
  };

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
  // sparse: units 2 and 3 ahead, their resolution state, and the attend masks of units 0..2
  XUnit uq2{}, uq3{};
  SparseTok tk2;
  int idx3 = -1;
  uint32_t maskq[2] = {0u, 0u};
  auto next_unit = [&](const XUnit& u) { return (u.b <= r.end_b) ? x_next(p, r, u) : u; };
  if constexpr (SPARSE) {
    uq[0] = x_seek(p, r, r.begin_b);
    uq[1] = next_unit(uq[0]);
    uq2 = next_unit(uq[1]);
    uq3 = next_unit(uq2);
    const int i0 = sparse_load_index(p, r, uq[0], kvh, ln.lane), i1 = sparse_load_index(p, r, uq[1], kvh, ln.lane);
    wait_vm_all();
    SparseTok k0 = sparse_load_page(p, r, uq[0], i0, ln.lane), k1 = sparse_load_page(p, r, uq[1], i1, ln.lane);
    const int i2 = sparse_load_index(p, r, uq2, kvh, ln.lane);
    wait_vm_all();
    const uint32_t o0 = sparse_offset(p, k0, maskq[0]), o1 = sparse_offset(p, k1, maskq[1]);
    okq[0] = !k0.bad;
    okq[1] = !k1.bad;
    if (uq[0].b <= r.end_b) sparse_issue<FMT>(kv_head, p.pool_bytes, o0, lds + X::kRing, wave, ln.lane);
    if (uq[1].b <= r.end_b) sparse_issue<FMT>(kv_head, p.pool_bytes, o1, lds + X::kRing + X::kSlot, wave, ln.lane);
    tk2 = sparse_load_page(p, r, uq2, i2, ln.lane);      // lands by the first wait of the unit loop
    idx3 = sparse_load_index(p, r, uq3, kvh, ln.lane);
  } else {
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
      if (okq[i]) issue(src, unit_valid(uq[i]), lds + X::kRing + i * X::kSlot);
    }
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
    const RowIdx ri = row_idx();
    const int last_ok = p.causal ? (L - p.s_q + ri.s_idx) : (L - 1);

    bf16x8 qf[X1Layout::kRegChunks];
    F8Q q8;
    if constexpr (kFp8) {
      // hi codes and scales in registers, lo codes in this wave's rows of the LDS
      const uint16_t* qrow = p.q + b * p.q_sb + ri.s_idx * p.q_ss + ri.shead * p.q_sh;
      f8_qsetup(qrow, ri.ok, 16 * wave + r16, q4, lds, q8);
    } else {
    {
      const uint16_t* qrow = p.q + b * p.q_sb + ri.s_idx * p.q_ss + ri.shead * p.q_sh;
#pragma unroll
      for (int c = 0; c < 18; ++c) {
        if (X1Layout::qslot(c) >= 0) continue;
        const u32x4 v = ri.ok ? *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * q4) : u32x4{0u, 0u, 0u, 0u};
        qf[X1Layout::qreg(c)] = __builtin_bit_cast(bf16x8, v);
      }
    }
    lds_barrier_keep_loads();                 // no wave still reads the previous sequence's Q^T chunks
    {
      const uint16_t* qb = p.q + b * p.q_sb;
      const int q_bytes = 2 * static_cast<int>((p.s_q - 1) * p.q_ss + (p.h_q - 1) * p.q_sh + kDqk);
      const __amdgpu_buffer_rsrc_t qrsrc =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(qb), 0, q_bytes, kRawBufferWord3);
      int lane_q = ln.lane;
      asm volatile("" : "+v"(lane_q));          // offsets computed here, not held across the unit loop
      const int lrow = lane_q >> 2, pslot = lane_q & 3;
#pragma unroll
      for (int j = 0; j < (X1Layout::kQChunks * 8 + kWW - 1) / kWW; ++j) {
        const int k = wave + kWW * j;
        if (k < X1Layout::kQChunks * 8) {
          const int qs = k >> 3, i = k & 7;
          const int row = 16 * i + lrow;
          const int sl = pslot ^ ((row >> 1) & 3);
          const int grow = mt * M_TILE + row;
          uint32_t off = 0xFFFFFFF0u;
          if (grow < p.rows) {
            const int sg = grow / p.group, hg = kvh * p.group + grow % p.group;
            off = static_cast<uint32_t>(2 * (sg * p.q_ss + hg * p.q_sh + 32 * X1Layout::qchunk(qs) + 8 * sl));
          }
          __builtin_amdgcn_raw_ptr_buffer_load_lds(qrsrc, LDS_PTR(void, lds + X1Layout::kQ + qs * X1Layout::kQChunkBytes + 1024 * i),
                                                   16, off, 0, 0, 0);
        }
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
      const uint32_t tokmask = SPARSE ? maskq[0] : ~0u;
      if constexpr (kFp8)
        f8_s<SPARSE>(cur, work, ln, par, L, last_ok, tok0, p.scale_log2, unit_id, q8, m_run, l_run, tokmask);
      else
        x1_s<SPARSE>(cur, work, ln, par, L, last_ok, tok0, p.scale_log2, unit_id, qf, m_run, l_run, tokmask);
      wait_vm_all();                          // this wave's loads of uq[1] landed
      XUnit un;
      bool ok_n = true;
      uint32_t mask_n = 0u, off_n = kNoToken;
      if constexpr (SPARSE) {
        // unit 2 ahead: its block-table entries landed with the wait above
        off_n = sparse_offset(p, tk2, mask_n);
        ok_n = !tk2.bad;
        un = uq2;
      }
      lds_barrier_keep_loads();               // P^T of u and uq[1] visible; every wave is past PV of u - 1
      if constexpr (SPARSE) {
        // the slot of u - 1: its last reader was PV of u - 1, before this barrier
        if (un.b <= r.end_b)
          sparse_issue<FMT>(kv_head, p.pool_bytes, off_n, lds + X::kRing + ((slot + 2) % 3) * X::kSlot, wave,
                            ln.lane);
        tk2 = sparse_load_page(p, r, uq3, idx3, ln.lane);   // step B of unit 3 ahead (its index landed)
        uq2 = uq3;
        uq3 = next_unit(uq3);
        idx3 = sparse_load_index(p, r, uq3, kvh, ln.lane);        // step A of the new unit 3 ahead
      } else {
      un = (uq[1].b <= r.end_b) ? x_next(p, r, uq[1]) : uq[1];
      if (un.b <= r.end_b) {
        const uint8_t* src_n = unit_src(un);
        ok_n = src_n != nullptr;
        // the slot of u - 1: its last reader was PV of u - 1, before this barrier
        if (ok_n) issue(src_n, unit_valid(un), lds + X::kRing + ((slot + 2) % 3) * X::kSlot);
      }
      }
      if constexpr (kFp8)
        f8_pv(cur, work, ln, par, unit_id, acc);
      else
        x1_pv(cur, work, ln, par, unit_id, acc);
      ++unit_id;
      slot = (slot + 1) % 3;
      uq[0] = uq[1];
      okq[0] = okq[1];
      maskq[0] = maskq[1];
      uq[1] = un;
      okq[1] = ok_n;
      maskq[1] = mask_n;
    }

    // ---- epilogue: l of every row through LDS; each wave writes its 64 dims ----
    lds_barrier_keep_loads();                 // every wave's PV is done: the P^T buffers are free
    float* lrow = reinterpret_cast<float*>(lds + X::kP);
    {
      const float l_tot = sum4lanes(l_run);
      const RowIdx re = row_idx();
      if (q4 == 0) lrow[re.srow - mt * M_TILE] = l_tot;
      if (q4 == 0 && re.ok) {
        float lse = (l_tot > 0.f) ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
        if (bad) lse = __builtin_nanf("");
        if (nsplit == 1)
          p.lse[lse_index(p, b, re.shead, re.s_idx)] = lse;
        else if (slot0 + split_idx < p.max_slots && split_idx < nsplit)
          p.part_lse[(static_cast<int64_t>(slot0 + split_idx) * p.h_kv + kvh) * p.rows + re.srow] = lse;
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

// ----------------------------------------------------------------------------
// A separate V cache (the optional vcache of the decode call: bf16 rows
// [pages, 64, h_kv, 512] addressed through the same block table as the keys;
// mmssai.com, "代码解读：flash_api.cpp 核心逻辑").
//
// 64-row tiles on 4 wavefronts: wave w owns rows 16 w .. 16 w + 15 and keeps
// their whole O (512 dims, 128 accumulator registers) and all of Q in
// registers, so P never leaves the wave and no exchange is needed. Units of 32
// tokens stream into a two-slot ring; a slot holds the unit's keys (36 KB in
// the xk_off layout) and its values (32 KB, the same layout over 64 chunks).
// One barrier per unit: after it, the loads of the next unit go out into the
// other slot (free: every wave has finished the unit before) and land while
// this one is computed. More than 64 rows per KV head take several row tiles;
// WIDE (more than 64 rows) writes the fp16 block-scaled partials of the
// 128-row kernels, otherwise fp32 partials, so the workspace and the combine
// are those of the plain decode.
// ----------------------------------------------------------------------------

constexpr int kVcWaves = 4;
constexpr int kVcThreads = 64 * kVcWaves;
constexpr int kVcRows = 16 * kVcWaves;                       // rows per workgroup
constexpr int kVcKBytes = kXHalfBytes;                       // 36864: keys of a unit
constexpr int kVcVBytes = kXHalf * kDv * 2;                  // 32768: values of a unit
constexpr int kVcSlot = kVcKBytes + kVcVBytes;
constexpr int kVcLds = 2 * kVcSlot;                          // 139264
static_assert(kVcLds <= 163840, "LDS budget");

// Direct loads of one unit into a slot: keys (k = wave + 4 j, j < 9: column
// block j, tokens 8 wave .. + 7) and values (j < 8), each buffer ending after
// the unit's `valid` tokens, so rows past them read zeros.
__device__ __forceinline__ void vc_issue(const uint8_t* ksrc, const uint8_t* vsrc, int valid, uint8_t* dst, int wave,
                                         uint32_t koff, uint32_t voff, int kst, int vst) {
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(ksrc), 0, valid * kst, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vsrc), 0, valid * vst, kRawBufferWord3);
#pragma unroll
  for (int j = 0; j < 9; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, LDS_PTR(void, dst + 1024 * (wave + 4 * j)), 16, koff,
                                             8 * wave * kst + 128 * j, 0, kPageLoadPolicy);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, LDS_PTR(void, dst + kVcKBytes + 1024 * (wave + 4 * j)), 16, voff,
                                             8 * wave * vst + 128 * j, 0, kPageLoadPolicy);
}

// S, softmax and PV of one unit for this wave's 16 rows: keys at kpage, values at vpage.
__device__ __forceinline__ void vc_unit(const uint8_t* __restrict__ kpage, const uint8_t* __restrict__ vpage,
                                        const XLane& ln, const bf16x8 (&qf)[18], int L, int last_ok, int tok0,
                                        float scale_log2, float& m_run, float& l_run, f32x4 (&acc)[32]) {
  const int q4 = ln.q4;
  auto kload = [&](int c, int tt) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(kpage + ln.k_off[c & 1] + 16 * tt * 128 + 4096 * (c >> 1));
  };
  f32x4 s[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    bf16x8 kbuf[2][2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) kbuf[0][tt] = kload(0, tt);
#pragma unroll
    for (int c = 0; c < 18; ++c) {
      if (c + 1 < 18) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) kbuf[(c + 1) & 1][tt] = kload(c + 1, tt);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kbuf[c & 1][tt], qf[c], s[tt], 0, 0, 0);
    }
  }
  // mask (sequence end, causal limit) and online softmax; lane (r16, q4) holds tokens
  // 16 tt + 4 q4 + i of row r16
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
  const bool rescale = grow && m_run != kNegInf;
  const float alpha = rescale ? fast_exp2(m_run - mx) : 1.f;
  l_run *= alpha;
  m_run = grow ? mx : m_run;
  if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
    for (int d = 0; d < 32; ++d) acc[d] *= alpha;      // this lane's row only
  }
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
  // O^T[dims 16 d + 4 q4 + i][row r16] += V^T P^T: P^T (k-slots: tokens 4 q4 + j, then 16 + 4 q4 + j)
  // is pv itself; V^T by transposed reads in the same token order
  auto vload = [&](int d) -> bf16x8 {
    const uint8_t* a0 = vpage + ln.v_off[d & 3] + 4096 * (d >> 2);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, a0));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, a0 + 16 * 128));
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
    acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pv, acc[d], 0, 0, 0);
  }
}

template <bool WIDE>
__global__ void __launch_bounds__(kVcThreads) splitkv_vc_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kVcLds];
  XLane ln;
  ln.tid = threadIdx.x;
  ln.lane = ln.tid & 63;
  ln.wave = __builtin_amdgcn_readfirstlane(ln.tid >> 6);
  ln.r16 = ln.lane & 15;
  ln.q4 = ln.lane >> 4;
  ln.k_off[0] = xk_off(ln.r16, ln.q4);
  ln.k_off[1] = xk_off(ln.r16, 4 + ln.q4);
  {
    const int tok = 4 * ln.q4 + (ln.r16 >> 2);
    const int hh = (ln.r16 & 3) >> 1, half8 = ln.r16 & 1;
#pragma unroll
    for (int e = 0; e < 4; ++e) ln.v_off[e] = xk_off(tok, 2 * e + hh) + 8 * half8;
  }
  const int wave = ln.wave, r16 = ln.r16, q4 = ln.q4;

  const int per_xcd = gridDim.x / 8;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= p.grid_wgs) return;
  const int m_tiles = (p.rows + kVcRows - 1) / kVcRows;
  const int mt = logical % m_tiles;
  const int kvh = (logical / m_tiles) % p.h_kv;
  const int part = logical / (m_tiles * p.h_kv);
  Range r;
  if (!read_range(p, part, r)) return;

  const int srow = mt * kVcRows + 16 * wave + r16;
  const bool srow_ok = srow < p.rows;
  const int s_idx = srow_ok ? srow / p.group : 0;
  const int shead = kvh * p.group + (srow_ok ? srow % p.group : 0);
  const int kst = static_cast<int>(p.kv_st), vst = static_cast<int>(p.vc_st);
  const uint32_t koff = x_load_off(ln.lane, kst), voff = x_load_off(ln.lane, vst);
  const uint8_t* const k_head = p.kv + kvh * p.kv_sh;
  const uint8_t* const v_head = p.vcache + kvh * p.vc_sh;

  // loads of unit u into `dst`; false (nothing issued) for a block-table entry outside the pool
  auto issue_unit = [&](const XUnit& u, uint8_t* dst) -> bool {
    const int pg = ld_meta(p.block_table + static_cast<int64_t>(u.b) * p.bt_stride + u.pi);
    if (pg < 0 || pg >= p.num_pages) return false;
    const int valid = min(u.L - (u.pi * kPage + u.hf * kXHalf), kXHalf);
    const uint8_t* ks = k_head + static_cast<int64_t>(pg) * p.kv_sp + static_cast<int64_t>(u.hf * kXHalf) * p.kv_st;
    const uint8_t* vs = v_head + static_cast<int64_t>(pg) * p.vc_sp + static_cast<int64_t>(u.hf * kXHalf) * p.vc_st;
    vc_issue(ks, vs, valid, dst, wave, koff, voff, kst, vst);
    return true;
  };

  XUnit u = x_seek(p, r, r.begin_b);
  bool ok = true;
  int slot = 0;
  if (u.b <= r.end_b) ok = issue_unit(u, lds);

  for (int b = r.begin_b; b <= r.end_b; ++b) {
    int L, pg0, pg1;
    bool len_ok;
    seq_pages(p, r, b, L, pg0, pg1, len_ok);
    const int split_idx = (b == r.begin_b) ? r.split0 : 0;
    const int slot0 = ld_meta(p.num_splits + b);
    const int nsplit = ld_meta(p.num_splits + b + 1) - slot0;
    const int last_ok = p.causal ? (L - p.s_q + s_idx) : (L - 1);

    bf16x8 qf[18];
    {
      const uint16_t* qrow = p.q + b * p.q_sb + s_idx * p.q_ss + shead * p.q_sh;
#pragma unroll
      for (int c = 0; c < 18; ++c) {
        const u32x4 v = srow_ok ? *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * q4) : u32x4{0u, 0u, 0u, 0u};
        qf[c] = __builtin_bit_cast(bf16x8, v);
      }
    }
    float m_run = kNegInf, l_run = 0.f;
    f32x4 acc[32];
#pragma unroll
    for (int d = 0; d < 32; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool bad = r.stale || !len_ok;

    // Invariant at the top: the loads of unit u into `slot` are issued (none if !ok).
    while (u.b == b) {
      const XUnit un = x_next(p, r, u);
      wait_vm_all();                          // this wave's loads of u (and Q) landed
      lds_barrier_keep_loads();               // every wave's loads of u landed; the other slot is free
      bool ok_n = true;
      if (un.b <= r.end_b) ok_n = issue_unit(un, lds + (slot ^ 1) * kVcSlot);
      bad |= !ok;
      const uint8_t* cur = lds + slot * kVcSlot;
      vc_unit(cur, cur + kVcKBytes, ln, qf, L, last_ok, u.pi * kPage + u.hf * kXHalf, p.scale_log2, m_run, l_run,
              acc);
      slot ^= 1;
      u = un;
      ok = ok_n;
    }

    // ---- epilogue: this lane's row, dims 16 d + 4 q4 .. + 3 ----
    const float l_tot = sum4lanes(l_run);
    float lse = (l_tot > 0.f) ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
    if (bad) lse = __builtin_nanf("");
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int d = 0; d < 32; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[d][i] = bad ? nan : acc[d][i] * inv;
    if (nsplit == 1) {
      if (srow_ok) {
        if (q4 == 0) p.lse[lse_index(p, b, shead, s_idx)] = lse;
        uint16_t* orow = p.o + ((static_cast<int64_t>(b) * p.s_q + s_idx) * p.h_q + shead) * kDv + 4 * q4;
#pragma unroll
        for (int d = 0; d < 32; ++d) {
          u32x2 w;
          w[0] = static_cast<uint32_t>(f32_to_bf16(acc[d][0])) | (static_cast<uint32_t>(f32_to_bf16(acc[d][1])) << 16);
          w[1] = static_cast<uint32_t>(f32_to_bf16(acc[d][2])) | (static_cast<uint32_t>(f32_to_bf16(acc[d][3])) << 16);
          *reinterpret_cast<u32x2*>(orow + 16 * d) = w;
        }
      }
    } else {
      const int pslot = slot0 + split_idx;
      const bool slot_ok = pslot >= 0 && pslot < p.max_slots && split_idx < nsplit;
      const int64_t prow = (static_cast<int64_t>(pslot) * p.h_kv + kvh) * p.rows + srow;
      if constexpr (WIDE) {
        // fp16 with a power-of-two scale per 64-dim block (block g: d = 4 g .. 4 g + 3)
#pragma unroll
        for (int g = 0; g < kPartBlocks; ++g) {
          float mx = 0.f;
#pragma unroll
          for (int dd = 0; dd < 4; ++dd)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, finite_abs(acc[4 * g + dd][i]));
          float scl, bi;
          part_block_scale(max4lanes(mx), scl, bi);
          u32x4 w[2];
          int off[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const f32x4& x = acc[4 * g + 2 * h];
            const f32x4& y = acc[4 * g + 2 * h + 1];
            u32x2 a, c;
            a[0] = pack_f16x2(x[0] * bi, x[1] * bi);
            a[1] = pack_f16x2(x[2] * bi, x[3] * bi);
            c[0] = pack_f16x2(y[0] * bi, y[1] * bi);
            c[1] = pack_f16x2(y[2] * bi, y[3] * bi);
            w[h] = span_f16x8(a, c, q4, &off[h]);
          }
          if (srow_ok && slot_ok) {
            uint16_t* const po = p.part_o16 + prow * kDv + 64 * g;
#pragma unroll
            for (int h = 0; h < 2; ++h) *reinterpret_cast<u32x4*>(po + 32 * h + off[h]) = w[h];
            if (q4 == 0) p.part_scale[prow * kPartBlocks + g] = scl;
          }
        }
      } else {
        if (srow_ok && slot_ok) {
          float* const po = p.part_o32 + prow * kDv + 4 * q4;
#pragma unroll
          for (int d = 0; d < 32; ++d) *reinterpret_cast<f32x4*>(po + 16 * d) = acc[d];
        }
      }
      if (srow_ok && slot_ok && q4 == 0) p.part_lse[prow] = lse;
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
    hipExtLaunchKernelGGL((splitkv_x1_kernel<kFmtFp8, false>), g, blk, 0, stream, ev_start, ev_stop, 0, p);
  else
    hipExtLaunchKernelGGL((splitkv_x1_kernel<kFmtBf16, false>), g, blk, 0, stream, ev_start, ev_stop, 0, p);
  return hipGetLastError();
}

hipError_t launch_split_vc(const DecodeParams& p, int grid, hipStream_t stream, hipEvent_t ev_start,
                           hipEvent_t ev_stop) {
  const dim3 g(grid), blk(kVcThreads);
  if (p.part_o16 != nullptr)
    hipExtLaunchKernelGGL((splitkv_vc_kernel<true>), g, blk, 0, stream, ev_start, ev_stop, 0, p);
  else
    hipExtLaunchKernelGGL((splitkv_vc_kernel<false>), g, blk, 0, stream, ev_start, ev_stop, 0, p);
  return hipGetLastError();
}

hipError_t launch_split_x_sparse(const DecodeParams& p, int kv_format, int grid, hipStream_t stream,
                                 hipEvent_t ev_start, hipEvent_t ev_stop) {
  const dim3 g(grid), blk(kWThreads);
  if (kv_format == kFmtFp8)
    hipExtLaunchKernelGGL((splitkv_x1_kernel<kFmtFp8, true>), g, blk, 0, stream, ev_start, ev_stop, 0, p);
  else
    hipExtLaunchKernelGGL((splitkv_x1_kernel<kFmtBf16, true>), g, blk, 0, stream, ev_start, ev_stop, 0, p);
  return hipGetLastError();
}

}  // namespace mla
