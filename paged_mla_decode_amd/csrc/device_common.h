// device_common.h -- device helpers shared by the split-KV kernels: vector
// types, the swizzled LDS row layout, FP8 code conversion, lane reductions,
// iteration over a KV range, and the LDS-only barrier.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace mla {
namespace dev {


typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))
#define GLOBAL_PTR(p) ((const __attribute__((address_space(1))) void*)(p))

constexpr int kRowBytes = kDqk * 2;                  // 1152: one bf16 token row
constexpr int kPageBytes = kPage * kRowBytes;        // 73728 = 72 x 1 KB
constexpr int kRawPageBytes = kPage * kFp8Record;    // 41984 = 41 x 1 KB
constexpr int kBf16Loads = kPageBytes / 1024;        // 72 direct-load instructions per page
constexpr int kFp8Loads = kRawPageBytes / 1024;      // 41
constexpr int kFmtFp8 = 1;
constexpr int kFmtBf16 = 0;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;

// LDS budget (bytes): bf16 -- two page slots; fp8 -- two raw slots, one bf16
// page, per-token scales.
constexpr int kLdsBf16 = 2 * kPageBytes;                                   // 147456
constexpr int kLdsFp8 = 2 * kRawPageBytes + kPageBytes + kPage * 4 * 4;    // 158720

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));   // round to nearest even
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Partial O of a piece in the workspace: fp16 values, each 64-dim block of a
// row divided by 2^(e - 15), where 2^e exceeds the largest finite magnitude in
// the block. The values then stay below 2^15 (fp16 keeps 11 significant bits
// of each), the power-of-two scale is exact both ways, and the combine
// multiplies it back. Infinities and NaN pass through unchanged.
constexpr int kPartBlocks = 8;                     // 64-dim blocks per row of 512

__device__ __forceinline__ float finite_abs(float v) {
  const float a = __builtin_fabsf(v);
  return a < __builtin_inff() ? a : 0.f;          // NaN compares false: 0
}

// scale (the combine multiplies by it) and inv (the writer multiplies by it)
// for a block whose largest finite magnitude is mx
__device__ __forceinline__ void part_block_scale(float mx, float& scale, float& inv) {
  int e = __builtin_amdgcn_frexp_expf(mx);         // mx < 2^e; 0 for mx = 0
  e = e < -110 ? -110 : e;
  scale = __builtin_amdgcn_ldexpf(1.f, e - 15);
  inv = __builtin_amdgcn_ldexpf(1.f, 15 - e);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(a))) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(b))) << 16);
}

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w)));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// One 32-dim span of a row's partial O, held as the MFMA output leaves it: lane
// (r16, q4) has dims 4 q4 .. + 3 (a, fp16 x 4) and 16 + 4 q4 .. + 3 (b) of row
// r16. Lanes q4 and q4 ^ 1 trade halves (v_permlane16_swap) so that each lane
// holds 8 consecutive dims: q4 even the dims of a of lanes q4, q4 + 1 (from
// 4 q4), q4 odd the dims of b of lanes q4 - 1, q4 (from 4 q4 + 12). The 4 lanes
// of a row then store 64 contiguous bytes. Returns the 16 bytes; *off = the
// lane's first dim within the span.
__device__ __forceinline__ u32x4 span_f16x8(const u32x2& a, const u32x2& b, int q4, int* off) {
  const auto a0 = __builtin_amdgcn_permlane16_swap(a[0], a[0], false, false);
  const auto a1 = __builtin_amdgcn_permlane16_swap(a[1], a[1], false, false);
  const auto b0 = __builtin_amdgcn_permlane16_swap(b[0], b[0], false, false);
  const auto b1 = __builtin_amdgcn_permlane16_swap(b[1], b[1], false, false);
  // element 0 of a swap result: the value of the even lane of the pair, 1: the odd one
  const bool odd = (q4 & 1) != 0;
  *off = 4 * q4 + (odd ? 12 : 0);
  return odd ? u32x4{b0[0], b1[0], b0[1], b1[1]} : u32x4{a0[0], a1[0], a0[1], a1[1]};
}

// Swizzle of the 16-byte chunk index inside a token row: chunk j of token t is
// stored at j ^ (t & 7), inside its aligned group of 8 chunks. Chosen by
// measurement on gfx950 (a 1152-byte row puts consecutive tokens half a bank
// window apart): with it both the K reads (ds_read_b128, 16 consecutive
// tokens x one chunk) and the transposed V reads (ds_read_b64_tr_b16, 4
// tokens x 2 chunks per 16 lanes) run at the full LDS rate (~286 and ~266
// B/clk/CU with 16 waves); the XOR patterns tried before reached 157-163.
__device__ __forceinline__ int swz(int token) { return token & 7; }

__device__ __forceinline__ int chunk_off(int token, int chunk) { return token * kRowBytes + 16 * (chunk ^ swz(token)); }

// Four OCP E4M3FN codes (the bytes of w, lowest first) -> four bf16 values
// (two per 32-bit word, lowest first), exactly: an e4m3 value has at most 4
// significant bits, so bf16 holds it without rounding. v_cvt_scalef32_pk_bf16_fp8
// with scale 1.0 converts two codes per instruction; checked against the OCP
// definition for all 256 codes (subnormals m * 2^-9, 0x7F / 0xFF -> NaN).
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, true));
}

// Cache-policy operand of the page loads: non-temporal (the "nt" bit of the
// gfx940-family cache policy; bit 1 of the builtin's aux operand). Each page
// is read once per workgroup, and streaming it with this hint raised the
// measured rate of the direct-to-LDS page ring from 6.2 to 7.1 TB/s.
constexpr int kPageLoadPolicy = 2;

// s_waitcnt vmcnt(0) as a builtin (expcnt and lgkmcnt fields left at "no wait"),
// so the compiler's own wait-count tracking sees it.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N vector-memory operations of this wave are outstanding
// (vmcnt, 6 bits on gfx950: low 4 in bits 3:0, high 2 in bits 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Lane l and lane l ^ 32 (v_permlane32_swap: the pair it returns holds, in
// every lane, the value of that lane and of its partner across the halves).
__device__ __forceinline__ void pair32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Lane l and lane l ^ 16 (v_permlane16_swap, the same within each 32-lane half).
__device__ __forceinline__ void pair16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Over the 4 lanes sharing lane % 16 (VALU lane swaps, no LDS round trip).
__device__ __forceinline__ float max4lanes(float v) {
  float a, b;
  pair16(v, a, b);
  v = fmaxf(a, b);
  pair32(v, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float sum4lanes(float v) {
  float a, b;
  pair16(v, a, b);
  v = a + b;
  pair32(v, a, b);
  return a + b;
}

// ----------------------------------------------------------------------------
// Page iteration over one KV range: sequences begin_b..end_b, pages [pg0, pg1)
// of each, in order. Zero-page sequences still get their epilogue.
// ----------------------------------------------------------------------------
// Read of launch-invariant metadata (sequence lengths, block table, ranges,
// piece counts) through the constant address space: with a wave-uniform index
// this becomes a scalar load, waited on with lgkmcnt, so it never waits for
// the page loads in flight (a vector load would need vmcnt(0)).
__device__ __forceinline__ int ld_meta(const int32_t* ptr) {
  return *(const __attribute__((address_space(4))) int32_t*)(ptr);
}

struct Range {
  int begin_b, begin_page, end_b, end_page, split0;
  bool stale;             // the metadata was built for other page counts: outputs become NaN
};

// Length of (virtual) sequence b: its cache length, or topk for sparse decode.
__device__ __forceinline__ int seq_len(const DecodeParams& p, int b) {
  return p.topk > 0 ? p.topk : ld_meta(p.seqlens + b);
}

// Real cache length of sequence b_real (sparse paths): kv_rows for sparse prefill.
__device__ __forceinline__ int real_len(const DecodeParams& p, int b_real) {
  return p.kv_rows > 0 ? p.kv_rows : ld_meta(p.seqlens + b_real);
}

// Index of (sequence b, head, query token s_idx) in lse [batch, h_q, s_q]; for
// sparse decode b is the virtual sequence b_real * sq_real + s.
__device__ __forceinline__ int64_t lse_index(const DecodeParams& p, int b, int head, int s_idx) {
  if (p.topk > 0) {
    const int br = b / p.sq_real, s = b - br * p.sq_real;
    return (static_cast<int64_t>(br) * p.h_q + head) * p.sq_real + s;
  }
  return (static_cast<int64_t>(b) * p.h_q + head) * p.s_q + s_idx;
}

// Row `part` of the tile metadata. Returns false for an empty range. Sets
// r.stale when the range's checksum of page counts (field 5) or the batch
// (field 6) differs from what this call's lengths give (plan.h, chk_step).
__device__ __forceinline__ bool read_range(const DecodeParams& p, int part, Range& r) {
  const int32_t* meta = p.meta + part * kMetaInts;
  r.begin_b = ld_meta(meta + 0);
  r.begin_page = ld_meta(meta + 1);
  r.end_b = min(ld_meta(meta + 2), p.batch - 1);
  r.end_page = ld_meta(meta + 3);
  r.split0 = ld_meta(meta + 4);
  if (r.begin_b < 0 || r.begin_b >= p.batch || r.end_b < r.begin_b) return false;
  uint32_t chk = kChkSeed;
  for (int b = r.begin_b; b <= r.end_b; ++b) chk = chk_step(chk, seq_npages(seq_len(p, b)));
  r.stale = static_cast<int32_t>(chk) != ld_meta(meta + 5) || ld_meta(meta + 6) != p.batch ||
            ld_meta(meta + 2) != r.end_b;
  return true;
}

// Length and page span of sequence b inside range r. A length outside
// [0, 64 * max_blocks] is clamped into it (no block-table read past the row)
// and reported through len_ok; its outputs become NaN.
__device__ __forceinline__ void seq_pages(const DecodeParams& p, const Range& r, int b, int& L, int& pg0, int& pg1,
                                          bool& len_ok) {
  const int max_len = p.max_blocks * kPage;
  int len;
  if (p.topk > 0) {                       // sparse: topk entries; the real length is checked
    const int real = real_len(p, b / p.sq_real);
    len_ok = real >= 0 && real <= max_len;
    len = p.topk;
  } else {
    len = ld_meta(p.seqlens + b);
    len_ok = len >= 0 && len <= max_len;
    len = len < 0 ? 0 : (len > max_len ? max_len : len);
  }
  L = len;
  const int np = (len + kPage - 1) / kPage;
  pg0 = (b == r.begin_b) ? max(r.begin_page, 0) : 0;
  pg1 = (b == r.end_b) ? min(r.end_page, np) : np;
  if (pg0 > pg1) pg0 = pg1;
}

__device__ __forceinline__ void seq_pages(const DecodeParams& p, const Range& r, int b, int& L, int& pg0, int& pg1) {
  bool len_ok;
  seq_pages(p, r, b, L, pg0, pg1, len_ok);
}

// First (sequence, page) at or after sequence b that has a page in the range; nb = end_b + 1 if none.
__device__ __forceinline__ void next_with_pages(const DecodeParams& p, const Range& r, int b, int& nb, int& npg) {
  for (; b <= r.end_b; ++b) {
    int L, pg0, pg1;
    seq_pages(p, r, b, L, pg0, pg1);
    if (pg0 < pg1) {
      nb = b;
      npg = pg0;
      return;
    }
  }
  nb = r.end_b + 1;
  npg = 0;
}

// Barrier that orders LDS only: unlike __syncthreads it does not wait for the
// page loads still in flight into the other ring slot.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup barrier for LDS exchanges made while direct page loads are in
// flight. A release fence on LDS also waits for those loads (they write LDS),
// so this one waits for this wave's own LDS accesses only (lgkmcnt(0);
// vmcnt and expcnt fields at their no-wait maxima); the asm memory clobber
// keeps the compiler from moving memory accesses across it. The caller
// orders the direct loads itself (s_waitcnt vmcnt before the barrier that
// publishes them).
// 16-byte LDS store in inline asm, for LDS regions that the compiler cannot tell
// apart from direct loads in flight (a plain store would wait for all of them).
// Completion is ordered by lgkmcnt (lds_barrier_keep_loads waits for it).
__device__ __forceinline__ uint32_t lds_addr(const void* ptr) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ptr));
}
__device__ __forceinline__ void lds_store16(uint32_t addr, const f32x4& v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

// N 16-byte LDS reads in one inline-asm block, waited inside it (lgkmcnt(0)), for
// reads the compiler would otherwise hold back behind every direct load in flight.
// Outputs are early-clobber: no address register is reused while a read is in flight.
template <int N>
__device__ __forceinline__ void lds_read16_block(const uint32_t (&a)[N], bf16x8 (&v)[N]);
template <>
__device__ __forceinline__ void lds_read16_block<3>(const uint32_t (&a)[3], bf16x8 (&v)[3]) {
  asm volatile(
      "ds_read_b128 %0, %3\n\tds_read_b128 %1, %4\n\tds_read_b128 %2, %5\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2])
      : "v"(a[0]), "v"(a[1]), "v"(a[2])
      : "memory");
}
template <>
__device__ __forceinline__ void lds_read16_block<6>(const uint32_t (&a)[6], bf16x8 (&v)[6]) {
  asm volatile(
      "ds_read_b128 %0, %6\n\tds_read_b128 %1, %7\n\tds_read_b128 %2, %8\n\t"
      "ds_read_b128 %3, %9\n\tds_read_b128 %4, %10\n\tds_read_b128 %5, %11\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5])
      : "memory");
}
template <>
__device__ __forceinline__ void lds_read16_block<8>(const uint32_t (&a)[8], bf16x8 (&v)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\tds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\tds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// 8 transposed 8-byte LDS reads (ds_read_b64_tr_b16) in one asm block, waited inside it.
__device__ __forceinline__ void lds_read_tr8_block(const uint32_t (&a)[8], u32x2 (&v)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %9\n\tds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\tds_read_b64_tr_b16 %4, %12\n\tds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\tds_read_b64_tr_b16 %7, %15\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

__device__ __forceinline__ void lds_barrier_keep_loads() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("s_barrier" ::: "memory");
}

// Lane-constant indices of one wavefront.
struct Lane {
  int tid, lane, wave, tg, r16, q4;
  int sw_k;              // swizzle of K rows read by this lane (token 16*tile + r16)
  int tr_tok, sw_v;      // V^T transposed reads: token tb + tr_tok (+16), its swizzle
  int tr_half, tr_hh;    // 8-byte half and chunk parity of the transposed read
};

// Exact online-softmax rescale is deferred until the running max grows by
// more than this (log2 units): P stays <= 2^8, far from fp32/bf16 limits, and
// O / l and LSE = m + log2 l are unchanged.
constexpr float kRescaleSlack = 8.f;

}  // namespace dev
}  // namespace mla
