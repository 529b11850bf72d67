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
// W = S_batch. Between snaps the walk is arithmetic: from a sequence start S_e
// the range starts are S_e + k (Bd - split_cost) until a range end falls
// within split_cost of a later sequence start S_a, where the walk snaps to
// S_a. So, per candidate budget, every sequence start gets its run (the number
// of range starts before the next snap, and the sequence it snaps to) in
// parallel; the number of ranges is the sum of the runs along the chain of
// snaps from sequence 0, found by pointer jumping; and once the budget is
// chosen, every range start follows at once by binary lifting over that chain.
// The rows, their first piece indices, the piece counts and the checksums then
// follow from the range starts in parallel. (The tile scheduler of the wmrh.cn
// FlashMLA深度解析 page, "计算流水线设计", spreads requests and blocks over
// the SMs; this cost model and layout are this library's own.)
#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.h"

namespace mla {
namespace {

constexpr int kSchedThreads = 1024;                 // 16 wavefronts
constexpr int kSchedWaves = kSchedThreads / 64;
constexpr int kSchedMaxBatch = 1023;                // one sequence per thread; node indices fit 11 bits
constexpr int kSchedMaxParts = 1024;
constexpr int kSchedMaxPages = 1 << 20;             // per sequence

constexpr int kSchedNodes = kSchedMaxBatch + 1;    // sequence starts 0..batch-1 and the end (batch)
constexpr int kSchedLevels = 11;                    // lifting levels: 2^10 >= kSchedNodes - 1 snaps
// A jump word: (ranges up to the target, saturated at kJumpSat) << 11 | target node. Saturation
// only marks a budget as infeasible: every count that matters is at most num_parts <= 1024.
constexpr uint32_t kJumpSat = (1u << 21) - 1;
__device__ __forceinline__ uint32_t jump_word(uint32_t ranges, uint32_t target) {
  return (ranges < kJumpSat ? ranges : kJumpSat) << 11 | target;
}

struct SchedShared {
  int32_t npages[kSchedMaxBatch];
  int32_t S[kSchedMaxBatch + 1];                    // cost-line start of each sequence; S[batch] = W
  int32_t scan[kSchedThreads];
  int32_t nranges[kSchedWaves];                     // ranges each candidate budget needs
  int32_t V[kSchedMaxParts + 1];                    // range starts of the chosen budget, then W
  uint32_t run0[kSchedWaves][kSchedNodes];          // per candidate: each sequence start's run (jump word)
  union {
    uint32_t jump[kSchedWaves][kSchedNodes];        // per candidate: pointer jumping over the runs
    struct {
      int16_t up[kSchedLevels][kSchedNodes];        // the node 2^k snaps ahead (batch: the end)
      int32_t cnt[kSchedLevels][kSchedNodes];       // ranges from a node up to that one
    } lift;
  };
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

// max { b < batch : S[b] <= x } for x in [S[lo], W), searching b in [lo, batch - 1]
__device__ __forceinline__ int seq_holding(const int32_t* S, int batch, int lo, int x) {
  int a = lo, z = batch - 1;
  while (a < z) {
    const int m = (a + z + 1) >> 1;
    if (S[m] <= x) a = m; else z = m - 1;
  }
  return a;
}

// floor(x / d) for 0 <= x < 2^31, 1 <= d < 2^30, from a float reciprocal estimate
// made exact by correction steps (unsigned products stay below 2^32)
__device__ __forceinline__ uint32_t div_floor(uint32_t x, uint32_t d, float inv_d) {
  uint32_t q = static_cast<uint32_t>(static_cast<float>(x) * inv_d);
  while (q > 0 && q * d > x) --q;
  while ((q + 1) * d <= x) ++q;
  return q;
}

// The run of budget bd from the start of sequence e: K range starts S_e + k step
// (step = bd - split_cost, k < K), then the snap to the start of sequence nx, or
// the end of the work (nx = batch). e = batch (the end): no range.
__device__ __forceinline__ void run_of(const int32_t* S, int batch, int W, int bd, int split_cost, int e, int& K,
                                       int& nx) {
  K = 0;
  nx = batch;
  if (e >= batch) return;
  const int step = bd - split_cost;
  const float inv_step = 1.f / static_cast<float>(step);
  const int E0 = S[e] + bd;                         // end of the run's first range
  if (E0 >= W) {
    K = 1;
    return;
  }
  int a = seq_holding(S, batch, e, E0);
  // region [sa, sa1) of sequence a holds E; sa2 is the boundary after it, read one step early
  // (S[batch] = W closes the last region)
  int sa = S[a], sa1 = S[a + 1], sa2 = S[min(a + 2, batch)];
  int k = 0, E = E0;
  for (;;) {
    if (E - sa <= split_cost) {                     // the range ends too close to S_a: snap there
      K = k + 1;
      nx = a;
      return;
    }
    // the first range whose end reaches sa1 (the next sequence start, or the end)
    k += 1 + static_cast<int>(div_floor(static_cast<uint32_t>(sa1 - E - 1), static_cast<uint32_t>(step), inv_step));
    E = E0 + k * step;
    if (E >= W) {
      K = k + 1;
      return;
    }
    // the sequence holding E: step ahead a few regions, then search
    int guard = 0;
    do {
      ++a;
      sa = sa1;
      sa1 = sa2;
      sa2 = S[min(a + 2, batch)];
    } while (sa1 <= E && ++guard < 4);
    if (sa1 <= E) {
      a = seq_holding(S, batch, a, E);
      sa = S[a];
      sa1 = S[a + 1];
      sa2 = S[min(a + 2, batch)];
    }
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

  const int lane = tid & 63;
  const int nodes = batch + 1;                      // the sequence starts and the end (node batch)

  // ---- per candidate budget: the runs of every sequence start (all (candidate, sequence)
  // pairs spread over the workgroup), then the ranges it needs -------------------------------
  const int ncand = split_cost + 1;
  for (int pr = tid; pr < ncand * nodes; pr += kSchedThreads) {
    const int cc = pr / nodes, e = pr - cc * nodes;
    const int bd = lo + cc;
    int K = 0, nx = batch;
    if (bd > split_cost) run_of(sh.S, batch, W, bd, split_cost, e, K, nx);
    const uint32_t w = jump_word(static_cast<uint32_t>(K), static_cast<uint32_t>(nx));
    sh.run0[cc][e] = w;
    sh.jump[cc][e] = w;
  }
  __syncthreads();
  // Pointer jumping in place, one wavefront per candidate: a node's jump word is read and written
  // whole, so every word is a valid jump at any time and the wavefront needs no barrier; a round
  // at least doubles every jump, and no chain has more than batch snaps.
  if (wave <= split_cost) {
    const int bd = lo + wave;
    uint32_t* const jw = sh.jump[wave];
    int need = 0x7FFFFFFF;
    if (bd > split_cost) {
      for (int r = 0; (1 << r) <= batch; ++r)
        for (int e = lane; e < nodes; e += 64) {
          const uint32_t w = jw[e];
          const uint32_t t = w & 2047u;
          if (t != static_cast<uint32_t>(batch)) {
            const uint32_t w2 = jw[t];
            jw[e] = jump_word((w >> 11) + (w2 >> 11), w2 & 2047u);
          }
        }
      const uint32_t w0 = jw[0];
      if ((w0 & 2047u) == static_cast<uint32_t>(batch) && (w0 >> 11) < kJumpSat) need = static_cast<int>(w0 >> 11);
    }
    if (lane == 0) sh.nranges[wave] = need;
  }
  __syncthreads();
  int c = 0;
  while (c < split_cost && sh.nranges[c] > num_parts) ++c;   // c = split_cost is always feasible
  const int step = lo + c - split_cost;
  const int n = min(sh.nranges[c], num_parts);

  // ---- the chosen budget: lifting tables over its chain of snaps, then every range start ----
  // (a node's ranges to the end never exceed those from sequence 0: the walk is monotone)
  int levels = 1;
  while ((1 << levels) - 1 < batch) ++levels;       // 2^levels - 1 >= the snaps on the chain
  for (int e = tid; e < nodes; e += kSchedThreads) {   // (every wavefront is past its jumping)
    const uint32_t w = sh.run0[c][e];
    sh.lift.up[0][e] = static_cast<int16_t>(w & 2047u);
    sh.lift.cnt[0][e] = static_cast<int32_t>(w >> 11);
  }
  __syncthreads();
  for (int k = 0; k + 1 < levels; ++k) {
    for (int e = tid; e < nodes; e += kSchedThreads) {
      const int u = sh.lift.up[k][e];
      sh.lift.up[k + 1][e] = sh.lift.up[k][u];
      sh.lift.cnt[k + 1][e] = sh.lift.cnt[k][e] + sh.lift.cnt[k][u];
    }
    __syncthreads();
  }
  for (int q = tid; q < n; q += kSchedThreads) {    // range q: in the run of the last chain node
    int cur = 0, acc = 0;                           // whose first range is at or before q
    for (int k = levels - 1; k >= 0; --k) {
      const int u = sh.lift.up[k][cur];
      const int cn = sh.lift.cnt[k][cur];
      if (u != batch && acc + cn <= q) {
        acc += cn;
        cur = u;
      }
    }
    sh.V[q] = sh.S[cur] + (q - acc) * step;
  }
  if (tid == 0) sh.V[n] = W;
  __syncthreads();
  const int32_t* V = sh.V;

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
