// scheduler_device.hip -- the tile scheduler of scheduler.cpp as one HIP
// workgroup, for lengths that live on the device (no host round trip). Its
// output is bit-identical to the host scheduler's for the same lengths, plan
// and number of ranges.
//
// The host's greedy fill with budget Bd, seen on a cost line: sequence b
// occupies [S_b, S_b+1) with S_b+1 - S_b = split_cost + pages_b (its fixed
// cost first, then its pages). A range whose work starts at line position V
// (a sequence start S_b, or page i of sequence b: V = S_b + i, the range then
// paying split_cost for its first piece) ends where its budget does,
// E = V + Bd, and the next range starts at f(E): the start S_e of the sequence
// e holding E when E - S_e <= split_cost (the cut would leave no page: the
// range stops before e), else E - split_cost (e is cut after page
// E - S_e - split_cost). f is non-decreasing, so the number of ranges a budget
// needs never grows with it, and each range advances at least Bd - split_cost:
// the smallest budget that places all the work in P ranges -- what the host's
// binary search finds -- lies in [ceil(W / P), ceil(W / P) + split_cost],
// W = S_batch. One wavefront per candidate walks the ranges (the sequence
// holding E found by a ballot over the prefix sums); the rows, their first
// piece indices, the piece counts and the checksums then follow from the range
// starts in parallel. (The tile scheduler of the wmrh.cn FlashMLA深度解析
// page, "计算流水线设计", spreads requests and blocks over the SMs; this
// cost model and layout are this library's own.)
#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.h"

namespace mla {
namespace {

constexpr int kSchedThreads = 1024;                 // 16 wavefronts
constexpr int kSchedWaves = kSchedThreads / 64;
constexpr int kSchedMaxBatch = 1023;                // prefix sums S[0..batch] in 16 chunks of 64 lanes
constexpr int kSchedMaxParts = 1024;
constexpr int kSchedChunks = (kSchedMaxBatch + 1) / 64;
constexpr int kSchedMaxPages = 1 << 20;             // per sequence

constexpr int kSnapTable = 1 << 16;                 // cost-line positions the snap table covers

struct SchedShared {
  uint8_t snap[kSnapTable];                         // x - S_b if x in [S_b, S_b + split_cost] (b holding x), else 255
  int32_t npages[kSchedMaxBatch];
  int32_t S[kSchedMaxBatch + 1];                    // cost-line start of each sequence; S[batch] = W
  int32_t V[kSchedWaves][kSchedMaxParts + 1];       // range starts of each candidate budget, then W
  int32_t scan[kSchedThreads];
  int32_t ok[kSchedWaves];
  int32_t nranges[kSchedWaves];
};

// Inclusive scan of one value per thread (every thread of the workgroup calls
// it): within each wavefront by lane shuffles, then the 16 wavefront totals.
__device__ __forceinline__ int block_scan(int32_t* buf, int x) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) buf[wave] = x;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += buf[w];
  const int total = [&] {
    int t = 0;
    for (int w = 0; w < kSchedWaves; ++w) t += buf[w];
    return t;
  }();
  __syncthreads();
  if (tid == kSchedThreads - 1) buf[kSchedThreads - 1] = total;   // the grand total, read after a barrier
  __syncthreads();
  return before + x;
}

// The same walk with the snap table (cost lines of up to kSnapTable
// positions), one candidate budget per lane of wavefront 0: lane c walks
// budget lo + c with its own LDS byte reads, so all candidates advance
// together and a step is one LDS read and a few vector instructions.
__device__ __forceinline__ void walk_candidates_table(SchedShared& sh, int W, int lo, int split_cost, int num_parts) {
  const int lane = threadIdx.x & 63;
  if (lane > split_cost) return;
  const int bd = lo + lane;
  int32_t* vout = sh.V[lane];
  int v = 0, p = 0;
  bool ok = bd > split_cost;
  while (ok && v < W) {
    if (p == num_parts) {
      ok = false;
      break;
    }
    const int E = v + bd;
    const int d = sh.snap[E < W ? E : 0];           // issued before the store below: they overlap
    vout[p] = v;
    const int nv = E >= W ? W : (d <= split_cost ? E - d : E - split_cost);
    if (nv <= v) {
      ok = false;
      break;
    }
    v = nv;
    ++p;
  }
  sh.ok[lane] = ok ? 1 : 0;
  sh.nranges[lane] = p;
  vout[p] = W;
}

template <int NC>
__device__ __forceinline__ void walk_candidate(SchedShared& sh, int batch, int W, int bd, int split_cost,
                                               int num_parts) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int32_t sreg[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = 64 * c + lane;
    sreg[c] = i <= batch ? sh.S[i] : 0x7FFFFFFF;
  }
  bd = __builtin_amdgcn_readfirstlane(bd);
  int32_t* vout = sh.V[wave];
  int v = 0, p = 0;
  bool ok = bd > split_cost;
  while (ok && v < W) {
    if (p == num_parts) {
      ok = false;
      break;
    }
    if (lane == 0) vout[p] = v;
    const int E = v + bd;
    int nv = E - split_cost;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(sreg[c] >= E - split_cost && sreg[c] <= E);
      const int idx = __builtin_amdgcn_readfirstlane(63 - __builtin_clzll(m | 1));
      const int sv = __builtin_amdgcn_readlane(sreg[c], idx);
      nv = m != 0 ? sv : nv;
    }
    nv = __builtin_amdgcn_readfirstlane(E >= W ? W : nv);
    if (nv <= v) {                                // no progress (cannot happen when bd > split_cost)
      ok = false;
      break;
    }
    v = nv;
    ++p;
  }
  if (lane == 0) {
    sh.ok[wave] = ok ? 1 : 0;
    sh.nranges[wave] = p;
    vout[p] = W;
  }
}

__global__ void __launch_bounds__(kSchedThreads) schedule_kernel(const int32_t* __restrict__ seqlens, int batch,
                                                                 int num_parts, int split_cost,
                                                                 int32_t* __restrict__ meta,
                                                                 int32_t* __restrict__ num_splits) {
  __shared__ SchedShared sh;
  const int tid = threadIdx.x, wave = tid >> 6;

  // ---- page counts and the exclusive prefix sums of (split_cost + pages) -------------------
  int cost = 0;
  int np = 0;
  if (tid < batch) {
    const int n = seq_npages(seqlens[tid]);
    np = n < 0 ? 0 : n;                             // a negative length is scheduled as empty
    sh.npages[tid] = np;
    cost = np > kSchedMaxPages ? 0 : split_cost + np;
  }
  // a sequence of more than 2^20 pages (67 million tokens): every range empty and no pieces,
  // so the decode reports every sequence as NaN; below that the cost line stays under 2^31
  const bool huge = np > kSchedMaxPages;
  block_scan(sh.scan, huge ? 1 : 0);
  const bool overflow = sh.scan[kSchedThreads - 1] != 0;
  __syncthreads();
  const int incl = block_scan(sh.scan, static_cast<int>(cost));
  if (tid < batch) sh.S[tid] = incl - static_cast<int>(cost);
  if (tid == 0) sh.S[batch] = sh.scan[kSchedThreads - 1];
  __syncthreads();
  if (overflow) {
    for (int p = tid; p < num_parts; p += kSchedThreads) {
      int32_t* m = meta + static_cast<int64_t>(p) * kMetaInts;
      m[0] = -1; m[1] = 0; m[2] = -2; m[3] = 0; m[4] = 0; m[5] = 0; m[6] = batch; m[7] = 0;
    }
    for (int b = tid; b <= batch; b += kSchedThreads) num_splits[b] = 0;
    return;
  }
  const int W = sh.S[batch];
  const int lo = max(1, (W + num_parts - 1) / num_parts);

  // ---- the snap table (short cost lines): positions within split_cost of a sequence start ----
  const bool table = W <= kSnapTable;
  if (table) {
    for (int x = tid; x < W; x += kSchedThreads) sh.snap[x] = 255;
    __syncthreads();
    if (tid < batch) {
      const int s0 = sh.S[tid], s1 = min(s0 + split_cost, sh.S[tid + 1] - 1);
      for (int x = s0; x <= s1; ++x) sh.snap[x] = static_cast<uint8_t>(x - s0);
    }
    __syncthreads();
  }
  // ---- one candidate budget per wavefront: its range starts, and whether they place all ----
  if (table) {
    if (wave == 0) walk_candidates_table(sh, W, lo, split_cost, num_parts);
  } else if (wave <= split_cost) {
    if (batch < 4 * 64)
      walk_candidate<4>(sh, batch, W, lo + wave, split_cost, num_parts);
    else
      walk_candidate<kSchedChunks>(sh, batch, W, lo + wave, split_cost, num_parts);
  }
  __syncthreads();
  int c = 0;
  while (c < split_cost && sh.ok[c] == 0) ++c;      // c = split_cost is always feasible
  const int32_t* V = sh.V[c];
  const int n = sh.nranges[c];

  auto count_le = [&](int x) {                      // #{q in [0, n) : V[q] <= x}
    int a = 0, z = n;
    while (a < z) {
      const int m = (a + z) >> 1;
      if (V[m] <= x) a = m + 1; else z = m;
    }
    return a;
  };
  auto count_lt = [&](int x) {                      // #{q in [0, n) : V[q] < x}
    int a = 0, z = n;
    while (a < z) {
      const int m = (a + z) >> 1;
      if (V[m] < x) a = m + 1; else z = m;
    }
    return a;
  };
  auto seq_at = [&](int x) {                        // max { b < batch : S[b] <= x }
    int a = 0, z = batch - 1;
    while (a < z) {
      const int m = (a + z + 1) >> 1;
      if (sh.S[m] <= x) a = m; else z = m - 1;
    }
    return a;
  };

  // ---- rows: range p covers [V[p], V[p + 1]) of the cost line --------------------------------
  for (int p = tid; p < num_parts; p += kSchedThreads) {
    int32_t row[kMetaInts];
    row[6] = batch;
    row[7] = 0;
    if (p >= n) {
      row[0] = -1; row[1] = 0; row[2] = -2; row[3] = 0; row[4] = 0; row[5] = 0;
    } else {
      const int v0 = V[p], v1 = V[p + 1];
      const int bb = seq_at(v0);
      int eb, ep;
      if (v1 >= W) {
        eb = batch - 1;
        ep = sh.npages[batch - 1];
      } else {
        const int a = seq_at(v1);
        if (v1 == sh.S[a]) {                        // the next range starts sequence a afresh
          eb = a - 1;
          ep = sh.npages[a - 1];
        } else {                                    // sequence a is cut after page v1 - S[a]
          eb = a;
          ep = v1 - sh.S[a];
        }
      }
      row[0] = bb;
      row[1] = v0 - sh.S[bb];
      row[2] = eb;
      row[3] = ep;
      row[4] = p - (count_le(sh.S[bb]) - 1);        // pieces of bb in the ranges before p
      uint32_t chk = kChkSeed;
      for (int b = bb; b <= eb; ++b) chk = chk_step(chk, seq_npages(seqlens[b]));
      row[5] = static_cast<int32_t>(chk);
    }
#pragma unroll
    for (int k = 0; k < kMetaInts; ++k) meta[static_cast<int64_t>(p) * kMetaInts + k] = row[k];
  }

  // ---- pieces per sequence (the ranges meeting [S[b], S[b + 1])) and their prefix sums -------
  const int pieces = tid < batch ? count_lt(sh.S[tid + 1]) - (count_le(sh.S[tid]) - 1) : 0;
  const int run = block_scan(sh.scan, pieces);
  if (tid == 0) num_splits[0] = 0;
  if (tid < batch) num_splits[tid + 1] = run;
}

}  // namespace

bool schedule_device_supported(int batch, int num_parts, int split_cost, int min_pages) {
  return batch >= 1 && batch <= kSchedMaxBatch && num_parts >= 1 && num_parts <= kSchedMaxParts &&
         split_cost >= 1 && split_cost < kSchedWaves && min_pages == 1;
}

hipError_t launch_schedule_device(const int32_t* seqlens, int batch, int num_parts, int split_cost, int32_t* meta,
                                  int32_t* num_splits, hipStream_t stream) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, seqlens, batch, num_parts, split_cost,
                     meta, num_splits);
  return hipGetLastError();
}

}  // namespace mla
