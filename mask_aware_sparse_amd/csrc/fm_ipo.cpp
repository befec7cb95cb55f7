// Stage-1 chunk balancing of HCC-IPO (FlashMask-3 page, §3.3 "Balance the work, not the
// length", and its IPO ablation table): n = P * kappa chunk loads go to P ranks, exactly
// kappa each, minimising the makespan (the largest rank load).  LB = max(ceil(sum / P),
// max w) certifies optimality when reached.  Host code only.
//
// The page names the phases (LPT, exact pairwise repartition P2, three-rank
// repartition P3) without pseudo-code; the reading implemented here:
//   LPT  chunks by (weight desc, index asc); each to the least loaded rank with fewer
//        than kappa chunks (ties: lowest rank).
//   P2   ranks a by (load desc, index asc); partners b by (load asc, index asc) with
//        load(b) <= load(a) - 2; the 2 kappa chunks of {a, b} are re-split exactly and
//        the first split whose larger half is below load(a) is applied; repeated until
//        no pair improves or the makespan is LB.
//   P3   the same over triples {a, b, c}, b < c both dominated by a (lower load, or
//        equal load and higher index), by (load(b) + load(c) asc, (b, c) asc), skipped
//        when 2 load(a) - load(b) - load(c) < 2; after each applied move P2 runs again.
// The exact re-split is a depth-first search over the pool in (weight desc, index asc)
// order; a chunk goes to group 0, 1, ... (kappa per group, only the first empty group
// is tried), a branch is cut when a group would reach the best maximum so far (initially
// the current maximum: only strictly better splits count), and the search stops when
// the pool's own bound max(ceil(S / k), max w) is reached.  Group g goes to the g-th
// smallest rank index of the move.
#include "fm.h"

#include <algorithm>
#include <cstdint>
#include <numeric>
#include <vector>

namespace {

using i64 = int64_t;

struct Split {
  int k, kappa;
  std::vector<int> order;   // pool, sorted by (w desc, index asc)
  const i64* w;
  i64 target;               // pool bound: nothing can be better
  i64 best;                 // best maximum so far (exclusive bound at the start)
  std::vector<int> place, best_place;
  i64 sums[3];
  int cnts[3];
  bool found = false;

  void dfs(size_t pos) {
    if (best <= target) return;
    if (pos == order.size()) {
      i64 m = sums[0];
      for (int g = 1; g < k; ++g) m = std::max(m, sums[g]);
      if (m < best) {
        best = m;
        best_place = place;
        found = true;
      }
      return;
    }
    const i64 wi = w[order[pos]];
    bool seen_empty = false;
    for (int g = 0; g < k; ++g) {
      if (cnts[g] == kappa) continue;
      if (cnts[g] == 0) {
        if (seen_empty) continue;
        seen_empty = true;
      }
      if (sums[g] + wi >= best) continue;
      sums[g] += wi;
      cnts[g] += 1;
      place[pos] = g;
      dfs(pos + 1);
      sums[g] -= wi;
      cnts[g] -= 1;
      if (best <= target) return;
    }
  }
};

// Re-split the chunks of `ranks` (sorted ascending); true if a split with maximum below
// `bound` was applied to owner.
bool resplit(const i64* w, std::vector<int>& owner, const std::vector<std::vector<int>>& members,
             const int* ranks, int k, int kappa, i64 bound) {
  Split s;
  s.k = k;
  s.kappa = kappa;
  s.w = w;
  for (int t = 0; t < k; ++t)
    s.order.insert(s.order.end(), members[ranks[t]].begin(), members[ranks[t]].end());
  std::sort(s.order.begin(), s.order.end(), [w](int a, int b) {
    return w[a] != w[b] ? w[a] > w[b] : a < b;
  });
  i64 total = 0, mx = 0;
  for (int i : s.order) {
    total += w[i];
    mx = std::max(mx, w[i]);
  }
  s.target = std::max((total + k - 1) / k, mx);
  s.best = bound;
  s.place.assign(s.order.size(), 0);
  for (int g = 0; g < 3; ++g) { s.sums[g] = 0; s.cnts[g] = 0; }
  s.dfs(0);
  if (!s.found) return false;
  int sorted_ranks[3];
  std::copy(ranks, ranks + k, sorted_ranks);
  std::sort(sorted_ranks, sorted_ranks + k);
  for (size_t p = 0; p < s.order.size(); ++p) owner[s.order[p]] = sorted_ranks[s.best_place[p]];
  return true;
}

struct State {
  const i64* w;
  int n, P, kappa;
  std::vector<int> owner;
  std::vector<i64> load;
  std::vector<std::vector<int>> members;
  i64 lb;
  int moves = 0;

  void refresh() {
    load.assign(P, 0);
    members.assign(P, {});
    for (int i = 0; i < n; ++i) {
      load[owner[i]] += w[i];
      members[owner[i]].push_back(i);
    }
  }
  i64 makespan() const { return *std::max_element(load.begin(), load.end()); }
  std::vector<int> by_load(bool desc) const {
    std::vector<int> r(P);
    std::iota(r.begin(), r.end(), 0);
    std::sort(r.begin(), r.end(), [&](int a, int b) {
      if (load[a] != load[b]) return desc ? load[a] > load[b] : load[a] < load[b];
      return a < b;
    });
    return r;
  }

  void lpt() {
    std::vector<int> order(n);
    std::iota(order.begin(), order.end(), 0);
    std::sort(order.begin(), order.end(), [this](int a, int b) {
      return w[a] != w[b] ? w[a] > w[b] : a < b;
    });
    std::vector<i64> l(P, 0);
    std::vector<int> cnt(P, 0);
    owner.assign(n, -1);
    for (int i : order) {
      int best = -1;
      for (int r = 0; r < P; ++r)
        if (cnt[r] < kappa && (best < 0 || l[r] < l[best])) best = r;
      owner[i] = best;
      l[best] += w[i];
      cnt[best] += 1;
    }
    refresh();
  }

  void p2() {
    for (;;) {
      if (makespan() <= lb) return;
      bool moved = false;
      const std::vector<int> desc = by_load(true), asc = by_load(false);
      for (int a : desc) {
        for (int b : asc) {
          if (b == a || load[b] > load[a] - 2) continue;
          const int rk[2] = {a, b};
          if (resplit(w, owner, members, rk, 2, kappa, load[a])) {
            ++moves;
            moved = true;
            break;
          }
        }
        if (moved) break;
      }
      if (!moved) return;
      refresh();
    }
  }

  // one P3 move; false if no triple improves
  bool p3_move() {
    if (makespan() <= lb) return false;
    for (int a : by_load(true)) {
      std::vector<int> others;
      for (int r = 0; r < P; ++r)
        if (r != a && (load[r] < load[a] || (load[r] == load[a] && r > a))) others.push_back(r);
      std::vector<std::pair<int, int>> pairs;
      for (size_t x = 0; x < others.size(); ++x)
        for (size_t y = x + 1; y < others.size(); ++y) pairs.emplace_back(others[x], others[y]);
      std::sort(pairs.begin(), pairs.end(), [this](const std::pair<int, int>& p,
                                                   const std::pair<int, int>& q) {
        const i64 sp = load[p.first] + load[p.second], sq = load[q.first] + load[q.second];
        return sp != sq ? sp < sq : p < q;
      });
      for (const auto& bc : pairs) {
        if (2 * load[a] - load[bc.first] - load[bc.second] < 2) continue;
        const int rk[3] = {a, bc.first, bc.second};
        if (resplit(w, owner, members, rk, 3, kappa, load[a])) {
          ++moves;
          refresh();
          return true;
        }
      }
    }
    return false;
  }
};

}  // namespace

extern "C" fm_status fm_ipo_balance(const int64_t* weights, int32_t n_chunks, int32_t ranks,
                                    int32_t stages, int32_t* owner, fm_ipo_report* report) {
  if (!weights || !owner || !report || ranks <= 0 || n_chunks <= 0 || n_chunks % ranks != 0 ||
      stages < 1 || stages > 3)
    return FM_ERR_INVALID_ARG;
  const int kappa = n_chunks / ranks;
  if (kappa > FM_IPO_MAX_KAPPA) return FM_ERR_UNSUPPORTED;
  i64 total = 0, mx = 0;
  for (int i = 0; i < n_chunks; ++i) {
    if (weights[i] < 0) return FM_ERR_INVALID_ARG;
    total += weights[i];
    mx = std::max(mx, (i64)weights[i]);
  }
  State st;
  st.w = weights;
  st.n = n_chunks;
  st.P = ranks;
  st.kappa = kappa;
  st.lb = std::max((total + ranks - 1) / ranks, mx);
  st.lpt();
  report->lb = st.lb;
  report->makespan_lpt = st.makespan();
  if (stages >= 2) st.p2();
  report->makespan_p2 = st.makespan();
  if (stages >= 3)
    while (st.p3_move()) st.p2();
  report->makespan = st.makespan();
  report->certified = report->makespan == st.lb ? 1 : 0;
  report->moves = st.moves;
  std::copy(st.owner.begin(), st.owner.end(), owner);
  return FM_OK;
}
