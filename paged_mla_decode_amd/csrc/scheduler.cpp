// scheduler.cpp -- host tile scheduler for split-KV MLA decode.
//
// FlashMLA computes tile-scheduler metadata once per decode step and reuses it
// for every layer (usage example in "功能 1" of the kdjingpai.com post; the
// metadata shapes [num_sm_parts, TileSchedulerMetaDataSize] and [batch + 1] in
// "代码解读：flash_api.cpp 核心逻辑" of the mmssai.com article). The pages give
// only those shapes; the field layout and the cut rule below are this
// library's own.
//
// Cost line: sequence b occupies split_cost + n_b units, n_b = ceil(L_b / 64)
// pages, sequences laid end to end in batch order. Range p is the interval
// [floor(p * T / P), floor((p + 1) * T / P)) of the line (T = total cost,
// P = ranges). A cut that falls inside a sequence's fixed cost moves to the
// start of that sequence; one that falls inside its pages cuts between pages,
// snapped to the sequence's start or end when it would leave a piece smaller
// than min_pages. Cuts are monotone, so the ranges partition every
// (sequence, page) exactly once, in order, and every sequence -- also one of
// length 0 -- lies in exactly one range or spans several consecutive ones.
#include <algorithm>
#include <cstring>
#include <vector>

#include "plan.h"

namespace mla {
namespace {

struct Cut {
  int b;      // sequence
  int64_t i;  // page within b; normalised so that i < n_b unless n_b == 0 (then i == 0)
};

}  // namespace

int schedule(const int32_t* seqlens, int batch, int num_parts, int split_cost, int min_pages,
             int32_t* meta, int32_t* num_splits) {
  std::vector<int64_t> npages(batch), start(batch + 1);
  int64_t total = 0;
  for (int b = 0; b < batch; ++b) {
    npages[b] = (static_cast<int64_t>(seqlens[b]) + kPage - 1) / kPage;
    start[b] = total;
    total += split_cost + npages[b];
  }
  start[batch] = total;

  // Cut position x on the cost line -> (sequence, page), normalised.
  auto cut_at = [&](int64_t x) -> Cut {
    if (x >= total) return Cut{batch, 0};
    int b = static_cast<int>(std::upper_bound(start.begin(), start.begin() + batch + 1, x) - start.begin()) - 1;
    int64_t i = x - start[b] - split_cost;
    if (i <= 0 || i < min_pages) return Cut{b, 0};
    if (npages[b] - i < min_pages) return Cut{b + 1, 0};
    return Cut{b, i};
  };

  std::vector<Cut> cuts(num_parts + 1);
  for (int p = 0; p <= num_parts; ++p) {
    int64_t x = (p == num_parts) ? total : static_cast<int64_t>((static_cast<__int128>(p) * total) / num_parts);
    cuts[p] = cut_at(x);
  }
  cuts[0] = Cut{0, 0};
  cuts[num_parts] = Cut{batch, 0};

  std::vector<int32_t> pieces(batch, 0);
  std::memset(meta, 0, sizeof(int32_t) * static_cast<size_t>(num_parts) * kMetaInts);
  for (int p = 0; p < num_parts; ++p) {
    int32_t* m = meta + static_cast<size_t>(p) * kMetaInts;
    const Cut a = cuts[p], e = cuts[p + 1];
    const bool empty = (a.b == e.b && a.i == e.i) || a.b >= batch;
    if (empty) {
      m[0] = -1; m[1] = 0; m[2] = -2; m[3] = 0; m[4] = 0;
      continue;
    }
    int end_b;
    int64_t end_page;
    if (e.i == 0) {             // ends at the end of the previous sequence
      end_b = e.b - 1;
      end_page = npages[end_b];
    } else {
      end_b = e.b;
      end_page = e.i;
    }
    m[0] = a.b;
    m[1] = static_cast<int32_t>(a.i);
    m[2] = end_b;
    m[3] = static_cast<int32_t>(end_page);
    m[4] = pieces[a.b];
    for (int b = a.b; b <= end_b; ++b) pieces[b] += 1;
  }
  num_splits[0] = 0;
  for (int b = 0; b < batch; ++b) num_splits[b + 1] = num_splits[b] + pieces[b];
  return num_splits[batch];
}

}  // namespace mla
