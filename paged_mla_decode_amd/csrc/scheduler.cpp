// scheduler.cpp -- host tile scheduler for split-KV MLA decode.
//
// FlashMLA computes tile-scheduler metadata once per decode step and reuses it
// for every layer (usage example in "功能 1" of the kdjingpai.com post; the
// metadata shapes [num_sm_parts, TileSchedulerMetaDataSize] and [batch + 1] in
// "代码解读：flash_api.cpp 核心逻辑" of the mmssai.com article). The pages give
// only those shapes; the field layout and the cut rule below are this
// library's own.
//
// Greedy fill: every piece of a sequence costs split_cost (its fixed work:
// loading Q, writing a partial result, merging it) plus its pages. Every
// range gets the same budget and takes sequences in batch order while they
// fit; the sequence that does not fit is cut between pages so that the range
// uses its budget, unless that would leave a piece smaller than min_pages
// (then the range stops before it, or takes its few remaining pages). The
// budget is the smallest one with which this pass places all the work in
// the ranges (binary search; a guessed budget such as ceil(T / P) +
// split_cost lets ranges that take only whole sequences run ahead and leaves
// the last ranges empty). Ranges are consecutive, so every
// (sequence, page) lies in exactly one range, in order, and every sequence --
// also one of length 0 -- lies in exactly one range or spans several
// consecutive ones.
#include <cstring>
#include <vector>

#include "plan.h"

namespace mla {

namespace {

// One greedy pass with a fixed budget per range. Returns true when every
// (sequence, page) fits into the num_parts ranges; when `meta` is non-null it
// also writes the ranges (the last range then takes whatever is left) and
// counts the pieces of each sequence.
bool fill(const std::vector<int64_t>& npages, int num_parts, int split_cost, int min_pages, int64_t budget,
          int32_t* meta, std::vector<int32_t>* pieces) {
  const int batch = static_cast<int>(npages.size());
  int b = 0;        // position: sequence b, page i
  int64_t i = 0;
  for (int p = 0; p < num_parts; ++p) {
    const int b0 = b;
    const int64_t i0 = i;
    int64_t room = budget;
    const bool take_rest = meta != nullptr && p == num_parts - 1;
    while (b < batch) {
      const int64_t left = npages[b] - i;
      if (take_rest || split_cost + left <= room) {        // the rest of sequence b fits
        room -= split_cost + left;
        ++b;
        i = 0;
        continue;
      }
      const int64_t take = room - split_cost;
      if (take < min_pages || take <= 0) break;            // nothing worth a new piece fits
      if (left - take < min_pages) {                       // do not leave a sliver behind
        ++b;
        i = 0;
      } else {
        i += take;
      }
      break;
    }
    if (meta == nullptr) continue;
    int32_t* m = meta + static_cast<size_t>(p) * kMetaInts;
    m[6] = batch;
    if (b0 == b && i0 == i) {                              // empty range
      m[0] = -1; m[1] = 0; m[2] = -2; m[3] = 0; m[4] = 0;
      continue;
    }
    int end_b;
    int64_t end_page;
    if (i == 0) {               // ends at the end of the previous sequence
      end_b = b - 1;
      end_page = npages[end_b];
    } else {
      end_b = b;
      end_page = i;
    }
    m[0] = b0;
    m[1] = static_cast<int32_t>(i0);
    m[2] = end_b;
    m[3] = static_cast<int32_t>(end_page);
    m[4] = (*pieces)[b0];
    uint32_t chk = kChkSeed;
    for (int s = b0; s <= end_b; ++s) {
      (*pieces)[s] += 1;
      chk = chk_step(chk, static_cast<int32_t>(npages[s]));
    }
    m[5] = static_cast<int32_t>(chk);
  }
  return b >= batch;
}

}  // namespace

int schedule(const int32_t* seqlens, int batch, int num_parts, int split_cost, int min_pages,
             int32_t* meta, int32_t* num_splits) {
  std::vector<int64_t> npages(batch);
  int64_t total = 0;
  for (int b = 0; b < batch; ++b) {
    npages[b] = (static_cast<int64_t>(seqlens[b]) + kPage - 1) / kPage;
    total += split_cost + npages[b];
  }
  // smallest budget with which the greedy pass places everything (binary
  // search: a larger budget never needs more ranges)
  int64_t lo = (total + num_parts - 1) / num_parts, hi = total + split_cost;
  if (lo < 1) lo = 1;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (fill(npages, num_parts, split_cost, min_pages, mid, nullptr, nullptr))
      hi = mid;
    else
      lo = mid + 1;
  }
  std::vector<int32_t> pieces(batch, 0);
  std::memset(meta, 0, sizeof(int32_t) * static_cast<size_t>(num_parts) * kMetaInts);
  fill(npages, num_parts, split_cost, min_pages, lo, meta, &pieces);
  num_splits[0] = 0;
  for (int s = 0; s < batch; ++s) num_splits[s + 1] = num_splits[s] + pieces[s];
  return num_splits[batch];
}

}  // namespace mla
