// Cross-batch scheduling: choosing the next batch from a sequence pool.
//
// Source: Batch Speculative Decoding Done Right (gist.science ko summary,
// section 2 Methodology, EXSPEC): instead of a fixed batch, a pool of
// sequences is kept and sequences of equal length are grouped dynamically;
// such a batch needs no realignment, and the alignment of EQSPEC is the
// fallback when lengths differ.  The pages fix neither the group choice nor
// the fallback's members; the reading here: the largest group of equal end
// columns (smallest end on ties) is taken whole or cut to the batch size,
// and when it is smaller than the caller's minimum group it is filled with
// the sequences whose end is nearest to it.
#include <algorithm>
#include <cstdlib>
#include <vector>

#include "svt_internal.h"

namespace svt {

int pool_pick(const int32_t* end, const int32_t* active, int n_slots, int max_batch, int min_group,
              int32_t* slots, int32_t* n_out) {
  struct E {
    int32_t end, slot;
  };
  std::vector<E> act;
  act.reserve((size_t)n_slots);
  for (int s = 0; s < n_slots; ++s)
    if (active[s]) act.push_back({end[s], s});
  *n_out = 0;
  if (act.empty()) return 1;
  std::sort(act.begin(), act.end(), [](const E& x, const E& y) { return x.end != y.end ? x.end < y.end : x.slot < y.slot; });
  // largest run of equal ends; the first (smallest end) wins ties
  size_t best = 0, best_n = 0;
  for (size_t i = 0; i < act.size();) {
    size_t j = i;
    while (j < act.size() && act[j].end == act[i].end) ++j;
    if (j - i > best_n) {
      best = i;
      best_n = j - i;
    }
    i = j;
  }
  const int e0 = act[best].end;
  const size_t thr = (size_t)std::min(max_batch, min_group);
  std::vector<int32_t> pick;
  if (best_n >= thr) {
    for (size_t k = 0; k < best_n && pick.size() < (size_t)max_batch; ++k) pick.push_back(act[best + k].slot);
  } else {
    for (size_t k = 0; k < best_n; ++k) pick.push_back(act[best + k].slot);
    std::vector<E> rest;
    for (size_t i = 0; i < act.size(); ++i)
      if (act[i].end != e0) rest.push_back(act[i]);
    std::sort(rest.begin(), rest.end(), [e0](const E& x, const E& y) {
      const long dx = std::labs((long)x.end - e0), dy = std::labs((long)y.end - e0);
      if (dx != dy) return dx < dy;
      return x.end != y.end ? x.end < y.end : x.slot < y.slot;
    });
    for (size_t k = 0; k < rest.size() && pick.size() < (size_t)max_batch; ++k) pick.push_back(rest[k].slot);
  }
  std::sort(pick.begin(), pick.end());
  bool same = true;
  for (int32_t s : pick) same = same && end[s] == e0;
  for (size_t k = 0; k < pick.size(); ++k) slots[k] = pick[k];
  *n_out = (int32_t)pick.size();
  return same ? 1 : 0;
}

}  // namespace svt
