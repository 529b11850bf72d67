// plan.h -- launch plan shared by the host scheduler and the kernel launcher.
//
// The split-KV kernels run 4 wavefronts per workgroup over the query rows of
// one KV head (rows = s_q * h_q / h_kv, the head fold of the
// deepseekonline.chat day-1 post, "Dynamische Sequenzoptimierung").
// Up to 64 rows: each wavefront owns a block of 16 rows and a
// group of the 64 tokens of every page it visits:
//   rb = 16-row blocks per workgroup, tg = token groups per page, rb * tg = 4.
// Few rows (memory-bound decode) split each page's tokens over the waves; 64
// rows give each wave 16 rows and the whole page.
// More than 64 rows: 128-row tiles (wide = 1, rb = 8) on 8 wavefronts, the S
// phase split by rows and the PV phase by value dims.
#pragma once

#include <cstdint>

namespace mla {

constexpr int kPage = 64;
constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kFp8Record = 656;
constexpr int kMetaInts = 8;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kFmtSparsePlan = 0;   // make_plan ignores the format

struct Plan {
  int wide;        // 1: 128-row tiles (more than 64 rows)
  int rb;          // 16-row blocks per workgroup
  int tg;          // token groups per page (rb * tg == kWaves unless wide)
  int m_tile;      // rows per workgroup
  int m_tiles;     // workgroups per (range, KV head) along the rows
  int wgs_per_cu;  // resident workgroups per CU the part count assumes
  int split_cost;  // scheduler: fixed cost of one piece of a sequence, in pages
  int min_pages;   // scheduler: smallest piece worth cutting off a sequence
};

inline Plan make_plan(int heads_per_kv, int kv_format) {
  (void)kv_format;
  Plan p{};
  if (heads_per_kv <= 16) {
    p.rb = 1; p.tg = 4;
  } else if (heads_per_kv <= 32) {
    p.rb = 2; p.tg = 2;
  } else if (heads_per_kv <= 64) {
    p.rb = 4; p.tg = 1;
  } else {
    p.wide = 1; p.rb = 8; p.tg = 1;   // more than 64 rows: 128-row tiles
  }
  p.m_tile = 16 * p.rb;
  p.m_tiles = (heads_per_kv + p.m_tile - 1) / p.m_tile;
  p.wgs_per_cu = 1;      // the two-page LDS ring (144-155 KB) leaves room for one workgroup per CU
  // per-piece fixed work in pages of KV: a 128-row piece loads 147 KB of Q,
  // writes 256 KB of partial O and the combine reads it back (about 9 pages of
  // KV bytes); a piece of up to 64 rows carries 1/8 of that plus the merge of
  // the token groups. Measured with the scheduler's searched budget: 8 and 3
  // (compute_heavy, ragged; the other workloads move by 1 % or less).
  p.split_cost = p.wide ? 8 : 3;
  p.min_pages = 1;
  return p;
}

// Token-level sparse decode: every (sequence, query token) pair is its own
// virtual sequence of topk entries with h_q / h_kv rows, always on the
// 128-row kernel (a smaller group leaves rows of the tile idle).
inline Plan make_plan_sparse(int group) {
  Plan p = make_plan(65, kFmtSparsePlan);
  p.m_tiles = (group + p.m_tile - 1) / p.m_tile;
  return p;
}

// Ranges the scheduler makes by default: enough workgroups to fill every CU
// `wgs_per_cu` deep once the row tiles and KV heads are counted.
inline int default_parts(const Plan& p, int h_kv, int num_cus) {
  long slots = static_cast<long>(num_cus) * p.wgs_per_cu;
  long per_range = static_cast<long>(p.m_tiles) * h_kv;
  long parts = slots / (per_range > 0 ? per_range : 1);
  if (parts < 1) parts = 1;
  if (parts > (1 << 20)) parts = 1 << 20;
  return static_cast<int>(parts);
}

// Pages of a sequence of length len (>= 0); -1 for a negative length.
constexpr int32_t seq_npages(int32_t len) { return len < 0 ? -1 : (len >> 6) + ((len & 63) != 0 ? 1 : 0); }

// Checksum of the page counts of the sequences a range covers (tile_metadata
// field 5), folded in sequence order: each step is a bijection of the running
// value for a fixed page count, so a change in the page count of any one
// sequence always changes the result. The decode recomputes it from the
// device lengths and poisons the range's sequences (NaN) when it differs:
// the metadata was built for other lengths.
constexpr uint32_t kChkSeed = 0x6D6C6131u;
constexpr uint32_t chk_step(uint32_t h, int32_t npages) {
  return (h ^ static_cast<uint32_t>(npages)) * 0x9E3779B1u + 0x7F4A7C15u;
}

// Host scheduler (scheduler.cpp). Lengths must be >= 0; num_parts >= 1.
// Returns the total number of pieces (num_splits[batch]).
int schedule(const int32_t* seqlens, int batch, int num_parts, int split_cost, int min_pages,
             int32_t* meta, int32_t* num_splits);

}  // namespace mla
