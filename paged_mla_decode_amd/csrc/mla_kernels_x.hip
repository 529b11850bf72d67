// mla_kernels_x.hip -- split-KV MLA decode kernel for more than 64 query rows
// per KV head on gfx950 (MI355X): 128-row tiles.
//
// Same computation as the 64-row kernel in mla_kernels.hip (softmax attention
// of query rows over a sequence's cached latent rows, V = their first 512
// dims; pieces of a sequence leave partial O / LSE for the combine kernel:
// wmrh.cn FlashMLA深度解析, "计算流水线设计"), organised so that V is read from
// LDS once per workgroup instead of once per wave.
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
// Each workgroup covers 128 query rows. Work advances in units of 32 tokens
// (half a page) through a three-slot LDS ring, so two units are in flight
// while one is computed, and LDS keeps room for the exchange buffers:
//   S phase  -- wave w owns rows 32w .. 32w + 31 as two 16-row blocks that
//               share every K operand read: S^T = K Q^T on MFMA 16x16x32 bf16
//               (A = 16 tokens x 32 dims of K from LDS, B = Q^T); 13 of the
//               18 32-dim Q chunks stay in VGPRs, 5 in LDS (O alone takes 256
//               of the 512 registers a lane has).
//   exchange -- each wave writes bf16 P^T of its rows, its rescale factors
//               and a flag; one barrier.
//   PV phase -- wave w accumulates O^T for value dims 128w .. 128w + 127 of
//               all 128 rows: it reads only its quarter of V (transposed) and
//               every wave's P^T.
// Per page this reads K four times (288 KB) but V once (64 KB), against four
// times each when every wave owns whole rows.
// Built for bf16 pages; FP8 pages use the 64-row kernel.
// ----------------------------------------------------------------------------

constexpr int kXHalf = 32;                                  // tokens per unit
constexpr int kXHalfBytes = kXHalf * kRowBytes;             // 36864 = 36 x 1 KB
constexpr int kXHalfLoads = kXHalfBytes / 1024;             // 36
constexpr int kXSlots = 3;
constexpr int kXPBytes = 128 * kXHalf * 2;                  // 8192: P^T [128 rows][32 tokens] bf16
constexpr int kXQChunkBytes = 128 * 64;                     // one 32-dim Q^T chunk of 128 rows
// LDS layout (bytes): the ring, P^T, rescale factors, flags, and the Q^T
// chunks {0, 1, 2, 16, 17} of the 128 rows; the other 13 chunks of each row
// stay in VGPRs.
struct XLayout {
  static constexpr int kSlot = kXHalfBytes;
  static constexpr int kRing = 0;
  static constexpr int kP = kRing + kXSlots * kSlot;        // 110592
  static constexpr int kAlpha = kP + kXPBytes;              // [128] fp32
  static constexpr int kFlag = kAlpha + 128 * 4;            // [4] int32 (64 B)
  static constexpr int kQ = kFlag + 64;
  static constexpr int kQChunks = 5;
  static constexpr int kTotal = kQ + kQChunks * kXQChunkBytes;   // 160320
  static constexpr int kLoads = kXHalfLoads;
  static constexpr int kLoadsPerWave = kLoads / kWaves;          // 9
  // LDS slot of Q^T chunk c, or -1 when it lives in VGPRs
  static constexpr int qslot(int c) { return c < 3 ? c : (c == 16 ? 3 : (c == 17 ? 4 : -1)); }
  static constexpr int kRegChunks = 18 - kQChunks;
  // register index of chunk c (chunks 3 .. 15)
  static constexpr int qreg(int c) { return c - 3; }
  // LDS chunk index qs -> Q chunk
  static constexpr int qchunk(int qs) { return qs < 3 ? qs : 13 + qs; }
};
static_assert(XLayout::kTotal <= 163840, "LDS budget");
static_assert(XLayout::kLoads % kWaves == 0, "equal direct-load counts per wave");

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

// Source offset of the 16 bytes that lane `lane` of direct load k brings into
// LDS byte 1024 k + 16 lane: token t, LDS chunk j holds global chunk j ^ swz(t).
__device__ __forceinline__ uint32_t x_load_off(int k, int lane, int st) {
  const int pc = 64 * k + lane;
  const int t = pc / 72;
  return static_cast<uint32_t>(t * st + 16 * ((pc - 72 * t) ^ swz(t)));
}

// Buffer resource word 3 for raw (unformatted, stride 0) buffer access on gfx9-family GPUs.
constexpr int kRawBufferWord3 = 0x00020000;

// Issue the direct loads of one unit (32 tokens starting at `src`, token stride
// `st`) into `dst`: MUBUF loads to LDS (buffer_load_dwordx4 ... lds), 16 bytes
// per lane, with the unit as the buffer (offsets past its 32 rows read zeros).
// The buffer form keeps the LDS read waits of the compute phases partial
// (the FLAT form makes every LDS wait a full drain while a load is in flight).
__device__ __forceinline__ void x_issue(const uint8_t* src, uint8_t* dst, int wave, const uint32_t (&off)[9], int st) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), 0, kXHalf * st, kRawBufferWord3);
#pragma unroll
  for (int j = 0; j < XLayout::kLoadsPerWave; ++j) {
    const int k = wave + kWaves * j;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, dst + 1024 * k), 16, off[j], 0, 0, 0);
  }
}

// s_waitcnt vmcnt(9): one unit's direct loads may stay in flight.
// (vmcnt: bits 3:0 and 15:14; expcnt 6:4 = 7 and lgkmcnt 11:8 = 15 mean no wait.)
__device__ __forceinline__ void wait_vm_one_unit() { __builtin_amdgcn_s_waitcnt(0x0F70 | XLayout::kLoadsPerWave); }
static_assert(XLayout::kLoadsPerWave < 16 && XLayout::kLoadsPerWave == 9, "vmcnt low field; load offsets per lane");

// Lane-constant indices. MFMA 16x16x32: lane l supplies A[i = l % 16][k-slots
// 8 (l / 16) .. + 7] and B[the same k-slots][j = l % 16]; D register i of lane
// l is D[4 (l / 16) + i][l % 16].
struct XLane {
  int tid, lane, wave;
  int r16, q4;          // lane % 16, lane / 16
  int k_off[2];         // S phase: K row r16, logical chunks q4 and 4 + q4 (swizzled), bytes
  int v_off[4];         // PV phase: transposed V read offsets, by 16-dim block d & 3
  uint32_t ld_off[9];   // direct loads: source offset of this lane's 16 bytes in load wave + 4 j
};

// One unit of the pipeline. `cur` holds the unit (32 bf16 rows), `nxt`
// receives the unit two ahead, `work` is the LDS after the ring (P^T, rescale
// factors, flags, Q^T chunks). The regions are disjoint; the restrict
// qualifiers let the compiler see that the LDS reads of this unit never touch
// the direct loads in flight into `nxt`.
__device__ __forceinline__ void x_step(uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt,
                                       uint8_t* __restrict__ work, const uint8_t* next_src, int st, const XLane& ln,
                                       int L, const int (&last_ok)[2], int tok0, int valid, bool this_ok,
                                       float scale_log2, int unit_id, const bf16x8 (&qf)[XLayout::kRegChunks][2],
                                       f32x4 (&acc)[8][8], float (&m_run)[2], float (&l_run)[2]) {
  using X = XLayout;
  const int tid = ln.tid, wave = ln.wave, r16 = ln.r16, q4 = ln.q4;
  uint8_t* const lds = work - X::kP;

  // ---- zero the rows past the sequence end (or the whole unit of a bad page) --------
  if (valid < kXHalf || !this_ok) {
    const int z0 = this_ok ? valid : 0;
    for (int x = z0 * kRowBytes + 16 * tid; x < kXHalfBytes; x += 16 * kThreads)
      *reinterpret_cast<u32x4*>(cur + x) = u32x4{0u, 0u, 0u, 0u};
    lds_barrier_keep_loads();
  }

  // ---- the unit two ahead -> nxt ----------------------------------------------------
  if (next_src != nullptr) x_issue(next_src, nxt, wave, ln.ld_off, st);

  // ---- S phase: S^T[token 16 tt + 4 q4 + i][row 32 w + 16 rb + r16] -------------------
  const uint8_t* qlds = lds + X::kQ;
  auto qop = [&](int c, int rb) -> bf16x8 {
    const int qs = X::qslot(c);
    if (qs >= 0)
      return *reinterpret_cast<const bf16x8*>(qlds + qs * kXQChunkBytes + xrow_off(32 * wave + 16 * rb + r16, q4));
    return qf[X::qreg(c)][rb];
  };
  // K: token 16 tt + r16, dims 32 c + 8 q4 .. + 7 = logical chunk 8 (c / 2) + 4 (c & 1) + q4
  auto kload = [&](int c, int tt) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(cur + ln.k_off[c & 1] + 16 * tt * kRowBytes + 128 * (c >> 1));
  };
  f32x4 s[2][2];                                  // [token tile][row block]
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) s[tt][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 kbuf[2][2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) kbuf[0][tt] = kload(0, tt);
#pragma unroll
  for (int c = 0; c < 18; ++c) {
    if (c + 1 < 18) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) kbuf[(c + 1) & 1][tt] = kload(c + 1, tt);
    }
    const bf16x8 q0 = qop(c, 0), q1 = qop(c, 1);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      s[tt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kbuf[c & 1][tt], q0, s[tt][0], 0, 0, 0);
      s[tt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kbuf[c & 1][tt], q1, s[tt][1], 0, 0, 0);
    }
  }

  // ---- softmax of this wave's rows; P^T, rescale factors and a flag -> LDS ---------------
  uint8_t* pbuf = lds + X::kP;
  float* alpha_buf = reinterpret_cast<float*>(lds + X::kAlpha);
  int* flags = reinterpret_cast<int*>(lds + X::kFlag);
  // Both 16-row blocks are handled side by side without branches, so their
  // dependent VALU chains interleave.
  float mx[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    // token tok0 + 16 tt + 4 q4 + i is allowed iff 16 tt + i <= lim
    const int lim = min(L - 1, last_ok[rb]) - tok0 - 4 * q4;
    mx[rb] = kNegInf;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = (16 * tt + i <= lim) ? s[tt][rb][i] * scale_log2 : kNegInf;
        s[tt][rb][i] = v;
        mx[rb] = fmaxf(mx[rb], v);
      }
  }
  mx[0] = max4lanes(mx[0]);
  mx[1] = max4lanes(mx[1]);
  bool rescaled = false;
  float alpha[2], m_use[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    // the running max moves only when it grows by more than the slack; a row's
    // first allowed tokens need no rescale (its O and l are still 0)
    const bool grow = mx[rb] > m_run[rb] + kRescaleSlack;
    const bool had = m_run[rb] != kNegInf;
    alpha[rb] = (grow && had) ? fast_exp2(m_run[rb] - mx[rb]) : 1.f;
    rescaled |= grow && had;
    l_run[rb] *= alpha[rb];
    m_run[rb] = grow ? mx[rb] : m_run[rb];
    m_use[rb] = (m_run[rb] == kNegInf) ? 0.f : m_run[rb];
  }
  bf16x8 pv[2];
  float psum[2] = {0.f, 0.f};
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float e = fast_exp2(s[tt][rb][i] - m_use[rb]);
        psum[rb] += e;
        pv[rb][4 * tt + i] = static_cast<__bf16>(e);
      }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    l_run[rb] += psum[rb];
    const int row = 32 * wave + 16 * rb + r16;
    // slot q4 of the row holds tokens 4 q4 .. 4 q4 + 3 and 16 + 4 q4 .. 16 + 4 q4 + 3
    *reinterpret_cast<bf16x8*>(pbuf + xrow_off(row, q4)) = pv[rb];
    if (q4 == 0) alpha_buf[row] = alpha[rb];
  }
  if (ln.lane == 0 && __builtin_amdgcn_ballot_w64(rescaled) != 0) flags[wave] = unit_id;
  lds_barrier_keep_loads();

  // ---- PV phase: O^T[dim 128 w + 16 dd + 4 q4 + i][row 16 rr + r16] += V^T P^T -------------
  if (flags[0] == unit_id || flags[1] == unit_id || flags[2] == unit_id || flags[3] == unit_id) {
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const float a = alpha_buf[16 * rr + r16];
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) acc[dd][rr] *= a;
    }
  }
  // transposed V reads: k-slots 0..3 = tokens 4 q4 + 0..3, 4..7 = the same + 16,
  // the token order of P^T slot q4
  auto vload = [&](int dd) -> bf16x8 {
    const int d = 8 * wave + dd;                  // 16-dim block of V
    const uint8_t* a0 = cur + ln.v_off[d & 3] + 128 * (d >> 2);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, a0));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, a0 + 16 * kRowBytes));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  bf16x8 pb[8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) pb[rr] = *reinterpret_cast<const bf16x8*>(pbuf + xrow_off(16 * rr + r16, q4));
  bf16x8 va[2];
  va[0] = vload(0);
#pragma unroll
  for (int dd = 0; dd < 8; ++dd) {
    if (dd + 1 < 8) va[(dd + 1) & 1] = vload(dd + 1);
#pragma unroll
    for (int rr = 0; rr < 8; ++rr)
      acc[dd][rr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dd & 1], pb[rr], acc[dd][rr], 0, 0, 0);
  }
}

__global__ void __launch_bounds__(kThreads) splitkv_x_kernel(DecodeParams p) {
  using X = XLayout;
  constexpr int M_TILE = 128;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[X::kTotal];

  XLane ln;
  ln.tid = threadIdx.x;
  ln.lane = ln.tid & 63;
  ln.wave = __builtin_amdgcn_readfirstlane(ln.tid >> 6);
  ln.r16 = ln.lane & 15;
  ln.q4 = ln.lane >> 4;
  {
    const int sw_k = swz(ln.r16);     // = swz(r16 + 16)
    ln.k_off[0] = ln.r16 * kRowBytes + 16 * (ln.q4 ^ sw_k);
    ln.k_off[1] = ln.r16 * kRowBytes + 16 * ((4 + ln.q4) ^ sw_k);
    // transposed V reads: lane i of a 16-lane group addresses token 4 q4 + i / 4
    // (+16) and dims 4 (i % 4) .. + 3 of each 16-dim block
    const int tok = 4 * ln.q4 + (ln.r16 >> 2);
    const int sw_v = swz(tok);        // = swz(tok + 16)
    const int hh = (ln.r16 & 3) >> 1, half8 = ln.r16 & 1;
#pragma unroll
    for (int e = 0; e < 4; ++e) ln.v_off[e] = tok * kRowBytes + 16 * ((2 * e + hh) ^ sw_v) + 8 * half8;
  }
  const int tid = ln.tid, wave = ln.wave, r16 = ln.r16, q4 = ln.q4;
  const int st = static_cast<int>(p.kv_st);
#pragma unroll
  for (int j = 0; j < X::kLoadsPerWave; ++j) ln.ld_off[j] = x_load_off(wave + kWaves * j, ln.lane, st);

  // XCD-aware order: consecutive logical workgroups share an XCD (and its L2)
  const int per_xcd = gridDim.x / 8;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= p.grid_wgs) return;
  const int m_tiles = (p.rows + M_TILE - 1) / M_TILE;
  const int mt = logical % m_tiles;
  const int kvh = (logical / m_tiles) % p.h_kv;
  const int part = logical / (m_tiles * p.h_kv);

  Range r;
  {
    const int32_t* meta = p.meta + part * kMetaInts;
    r.begin_b = ld_meta(meta + 0);
    r.begin_page = ld_meta(meta + 1);
    r.end_b = min(ld_meta(meta + 2), p.batch - 1);
    r.end_page = ld_meta(meta + 3);
    r.split0 = ld_meta(meta + 4);
  }
  if (r.begin_b < 0 || r.begin_b >= p.batch || r.end_b < r.begin_b) return;

  if (tid < 4) reinterpret_cast<int*>(lds + X::kFlag)[tid] = -1;

  // S-phase rows of this lane
  int srow[2], s_idx[2], shead[2];
  bool srow_ok[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    srow[rb] = mt * M_TILE + 32 * wave + 16 * rb + r16;
    srow_ok[rb] = srow[rb] < p.rows;
    s_idx[rb] = srow_ok[rb] ? srow[rb] / p.group : 0;
    shead[rb] = kvh * p.group + (srow_ok[rb] ? srow[rb] % p.group : 0);
  }

  const uint8_t* const kv_head = p.kv + kvh * p.kv_sh;
  // Block-table window: lane i holds entry win_pi + i of sequence win_b's row
  // (-1 past the row). Refilled with one vector load when a unit falls outside
  // it (a new sequence, or every 64 pages), so units need no scalar load each.
  int bt_win = -1, win_b = -1, win_pi = 0;
  // global address of a unit (nullptr: block-table entry outside the pool)
  auto unit_src = [&](const XUnit& u) -> const uint8_t* {
    if (u.b != win_b || u.pi < win_pi || u.pi >= win_pi + 64) {
      win_b = u.b;
      win_pi = u.pi;
      const int e = u.pi + ln.lane;
      bt_win = e < p.max_blocks ? p.block_table[static_cast<int64_t>(u.b) * p.bt_stride + e] : -1;
      wait_vm_all();
    }
    const int pg = __builtin_amdgcn_readlane(bt_win, u.pi - win_pi);
    if (pg < 0 || pg >= p.num_pages) return nullptr;
    return kv_head + static_cast<int64_t>(pg) * p.kv_sp + static_cast<int64_t>(u.hf) * kXHalf * st;
  };

  // ---- prime the ring: the first two units ----------------------------------------------
  // u1 is in flight into `slot`, u2 into the next slot; ok = its page is valid
  // (a unit is issued iff it is inside the range and ok).
  XUnit u1 = x_seek(p, r, r.begin_b), u2;
  bool ok1 = true, ok2 = true;
  if (u1.b <= r.end_b) {
    const uint8_t* src = unit_src(u1);
    ok1 = src != nullptr;
    if (ok1) x_issue(src, lds + X::kRing, wave, ln.ld_off, st);
    u2 = x_next(p, r, u1);
  } else {
    u2 = u1;
  }
  if (u2.b <= r.end_b) {
    const uint8_t* src = unit_src(u2);
    ok2 = src != nullptr;
    if (ok2) x_issue(src, lds + X::kRing + X::kSlot, wave, ln.ld_off, st);
  }
  int slot = 0;
  int unit_id = 0;

  for (int b = r.begin_b; b <= r.end_b; ++b) {
    int L, pg0, pg1;
    seq_pages(p, r, b, L, pg0, pg1);
    const int split_idx = (b == r.begin_b) ? r.split0 : 0;
    const int slot0 = ld_meta(p.num_splits + b);
    const int nsplit = ld_meta(p.num_splits + b + 1) - slot0;
    int last_ok[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) last_ok[rb] = p.causal ? (L - p.s_q + s_idx[rb]) : (L - 1);

    // Q^T of this sequence: chunks 3..15 of the lane's rows in VGPRs, chunks
    // 0, 1, 2, 16, 17 of all 128 rows in LDS
    bf16x8 qf[X::kRegChunks][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const uint16_t* qrow = p.q + b * p.q_sb + s_idx[rb] * p.q_ss + shead[rb] * p.q_sh;
#pragma unroll
      for (int c = 0; c < 18; ++c) {
        if (X::qslot(c) >= 0) continue;
        const u32x4 v = srow_ok[rb] ? *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * q4) : u32x4{0u, 0u, 0u, 0u};
        qf[X::qreg(c)][rb] = __builtin_bit_cast(bf16x8, v);
      }
    }
    lds_barrier_keep_loads();                 // no wave still reads the previous sequence's Q^T chunks
    for (int item = tid; item < X::kQChunks * 128 * 4; item += kThreads) {
      const int qs = item / 512, row = (item >> 2) & 127, sl = item & 3;
      const int c = X::qchunk(qs);
      const int grow = mt * M_TILE + row;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (grow < p.rows) {
        const int sg = grow / p.group, hg = kvh * p.group + grow % p.group;
        v = *reinterpret_cast<const u32x4*>(p.q + b * p.q_sb + sg * p.q_ss + hg * p.q_sh + 32 * c + 8 * sl);
      }
      *reinterpret_cast<u32x4*>(lds + X::kQ + qs * kXQChunkBytes + xrow_off(row, sl)) = v;
    }
    wait_vm_all();
    lds_barrier();

    float m_run[2] = {kNegInf, kNegInf}, l_run[2] = {0.f, 0.f};
    f32x4 acc[8][8];                          // [16-dim block][16-row block]
#pragma unroll
    for (int dd = 0; dd < 8; ++dd)
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) acc[dd][rr] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool bad = false;

    while (u1.b == b) {
      const XUnit u = u1;
      const bool this_ok = ok1;
      bad |= !this_ok;
      const bool u2_issued = u2.b <= r.end_b && ok2;
      if (u2_issued) wait_vm_one_unit(); else wait_vm_all();
      lds_barrier_keep_loads();               // every wave's loads of u landed; unit u - 1 is done everywhere
      const XUnit u3 = (u2.b <= r.end_b) ? x_next(p, r, u2) : u2;
      const uint8_t* src3 = nullptr;
      bool ok3 = true;
      if (u3.b <= r.end_b) {
        src3 = unit_src(u3);
        ok3 = src3 != nullptr;
      }
      const int tok0 = u.pi * kPage + u.hf * kXHalf;
      const int valid = min(L - tok0, kXHalf);
      const int slot3 = (slot + 2) % kXSlots;  // held unit u - 1, free now
      x_step(lds + X::kRing + slot * X::kSlot, lds + X::kRing + slot3 * X::kSlot, lds + X::kP, src3, st, ln, L,
             last_ok, tok0, valid, this_ok, p.scale_log2, unit_id, qf, acc, m_run, l_run);
      ++unit_id;
      slot = (slot + 1) % kXSlots;
      u1 = u2;
      ok1 = ok2;
      u2 = u3;
      ok2 = ok3;
    }

    // ---- epilogue: l of every row through LDS; each wave writes its 128 dims ----
    lds_barrier_keep_loads();                 // the P^T buffer is free
    float* lrow = reinterpret_cast<float*>(lds + X::kP);   // [128] l
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float l_tot = sum4lanes(l_run[rb]);
      if (q4 == 0) lrow[32 * wave + 16 * rb + r16] = l_tot;
      if (q4 == 0 && srow_ok[rb]) {
        float lse = (l_tot > 0.f) ? (m_run[rb] + __log2f(l_tot)) * kLn2 : kNegInf;
        if (bad) lse = __builtin_nanf("");
        if (nsplit == 1)
          p.lse[(static_cast<int64_t>(b) * p.h_q + shead[rb]) * p.s_q + s_idx[rb]] = lse;
        else if (slot0 + split_idx < p.max_slots && split_idx < nsplit)
          p.part_lse[(static_cast<int64_t>(slot0 + split_idx) * p.h_kv + kvh) * p.rows + srow[rb]] = lse;
      }
    }
    lds_barrier_keep_loads();
    // lane l holds, per (dd, rr), row 16 rr + r16 and dims 128 w + 16 dd + 4 q4 + 0..3
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int row = mt * M_TILE + 16 * rr + r16;
      if (row >= p.rows) continue;
      const float l_row = lrow[16 * rr + r16];
      const float inv = (l_row > 0.f) ? 1.f / l_row : 0.f;
      const int si = row / p.group, hh = kvh * p.group + row % p.group;
      if (nsplit == 1) {
        uint16_t* orow = p.o + ((static_cast<int64_t>(b) * p.s_q + si) * p.h_q + hh) * kDv + 128 * wave + 4 * q4;
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
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
          float* prow = p.part_o + ((static_cast<int64_t>(pslot) * p.h_kv + kvh) * p.rows + row) * kDv +
                        128 * wave + 4 * q4;
#pragma unroll
          for (int dd = 0; dd < 8; ++dd) {
            f32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = bad ? nan : acc[dd][rr][i] * inv;
            *reinterpret_cast<f32x4*>(prow + 16 * dd) = v;
          }
        }
      }
    }
  }
  wait_vm_all();
}

}  // namespace

hipError_t launch_split_x(const DecodeParams& p, int grid, hipStream_t stream, hipEvent_t ev_start,
                          hipEvent_t ev_stop) {
  hipExtLaunchKernelGGL(splitkv_x_kernel, dim3(grid), dim3(kThreads), 0, stream, ev_start, ev_stop, 0, p);
  return hipGetLastError();
}

}  // namespace mla
