// Key-range split plan of an attention launch (host side): which q-tiles take the
// whole key range in one workgroup and into how many parts the others are split, from a
// model of how the grid is dispatched over the chip.
#include <algorithm>
#include <array>
#include <map>
#include <mutex>

#include "kernels.h"

namespace dit {

// Key-range split plan of a launch.  Workgroups are modelled as dispatched in grid
// order, round-robin over the 8 XCDs, each XCD list-scheduling its share on slots/8
// concurrent slots; a workgroup of k key tiles takes k + ATTN_WG_FIXED tile-times.  For
// every split count (1..4) and first split q-tile qt0 the plan takes the modelled
// makespan plus the merge pass (ATTN_MERGE_COST tile-times per split part of a
// (head, q-tile), spread over the chip) and keeps the cheapest; at equal cost, fewer
// parts and fewer split q-tiles.  Splitting needs at least 2 tiles per part and partial
// storage for nsplit * nq rows.  Plans are memoised per shape.
constexpr int ATTN_WG_FIXED = 2;
constexpr double ATTN_MERGE_COST = 0.02;

// Makespan of list scheduling on S equal slots: k1 items of cost c1, then k2 of cost c2,
// each to the earliest free slot.  Slots with equal load form one group, so equal-cost
// items are placed a group at a time (a few dozen steps instead of one per item).
static long long list_makespan(long long k1, long long k2, long long S, long long c1, long long c2) {
  std::map<long long, long long> g;  // load -> slots
  g[k1 / S * c1] += S - k1 % S;
  if (k1 % S) g[(k1 / S + 1) * c1] += k1 % S;
  while (k2 > 0) {
    auto it = g.begin();
    const long long load = it->first, t = std::min(it->second, k2);
    k2 -= t;
    if ((it->second -= t) == 0) g.erase(it);
    g[load + c2] += t;
  }
  return g.rbegin()->first;
}

// Modelled time of a plan in tile-times x ns: grid order round robin over the 8 XCDs,
// whole-range items (cost key_tiles + ATTN_WG_FIXED) first, then the split parts.
static double attention_makespan(int nqt, int H, int key_tiles, int ns, int qt0, int slots) {
  constexpr int NXCD = 8;
  const long long per = slots / NXCD > 0 ? slots / NXCD : 1;
  const long long n1 = (long long)qt0 * H;
  const long long n = n1 + (long long)(nqt - qt0) * H * ns;
  const long long c1 = ((long long)key_tiles + ATTN_WG_FIXED) * ns, c2 = key_tiles + ATTN_WG_FIXED * ns;
  long long worst = 0;
  for (int x = 0; x < NXCD && x < n; ++x) {
    const long long cnt = n / NXCD + (x < n % NXCD), k1 = n1 / NXCD + (x < n1 % NXCD);
    worst = std::max(worst, list_makespan(k1, cnt - k1, per, c1, c2));
  }
  return (double)worst / ns;
}

AttnSplit attention_plan(int nq, int H, int key_tiles, int partial_rows, int slots) {
  AttnSplit best{1, 0, nullptr, nullptr};
  if (nq <= 0 || H <= 0 || key_tiles <= 0) return best;
  static std::mutex mu;
  static std::map<std::array<int, 5>, std::pair<int, int>> memo;
  const std::array<int, 5> key{nq, H, key_tiles, partial_rows, slots};
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = memo.find(key);
    if (it != memo.end()) {
      best.nsplit = it->second.first;
      best.qt0 = it->second.second;
      return best;
    }
  }
  const int nqt = (nq + ATTN_QTILE - 1) / ATTN_QTILE;
  double best_cost = attention_makespan(nqt, H, key_tiles, 1, 0, slots);
  for (int ns = 2; ns <= 4; ++ns) {
    if (key_tiles < 2 * ns || (long long)ns * nq > partial_rows) break;
    for (int qt0 = nqt - 1; qt0 >= 0; --qt0) {
      const double cost = attention_makespan(nqt, H, key_tiles, ns, qt0, slots) +
                          ATTN_MERGE_COST * ns * (double)(nqt - qt0) * H;
      if (cost < best_cost - 1e-9) {
        best_cost = cost;
        best.nsplit = ns;
        best.qt0 = qt0;
      }
    }
  }
  std::lock_guard<std::mutex> g(mu);
  memo.emplace(key, std::make_pair(best.nsplit, best.qt0));
  return best;
}

}  // namespace dit
