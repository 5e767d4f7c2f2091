// Owner assignment by makespan minimization (see assign.hpp).
#include "assign.hpp"

#include <algorithm>
#include <numeric>

namespace muon {
namespace {

// Relative margin below which two makespans count as equal (summation order
// alone can move a total by a few ulps).
constexpr double kTol = 1e-12;

struct Search {
  const std::vector<double>& c;      // costs in search order (decreasing)
  int k;
  int64_t limit;
  std::vector<double> suffix;        // suffix[j] = sum of c[j..]
  std::vector<double> load;
  std::vector<int32_t> cur, best_owner;
  double best;
  int64_t nodes = 0;
  bool aborted = false;

  Search(const std::vector<double>& costs, int owners, int64_t node_limit, double start,
         const std::vector<int32_t>& start_owner)
      : c(costs), k(owners), limit(node_limit), suffix(costs.size() + 1, 0.0), load(owners, 0.0),
        cur(costs.size(), 0), best_owner(start_owner), best(start) {
    for (size_t j = costs.size(); j-- > 0;) suffix[j] = suffix[j + 1] + costs[j];
  }

  void dfs(size_t j, double cur_max) {
    if (aborted) return;
    if (++nodes > limit) {
      aborted = true;
      return;
    }
    if (j == c.size()) {
      if (cur_max < best * (1 - kTol)) {
        best = cur_max;
        best_owner = cur;
      }
      return;
    }
    // every remaining item lands somewhere: the final makespan is at least the
    // current one, the average total, and the least-loaded owner plus item j
    const double total = suffix[0];
    double min_load = load[0];
    for (int o = 1; o < k; ++o) min_load = std::min(min_load, load[o]);
    const double bound = std::max({cur_max, total / k, min_load + c[j]});
    if (bound >= best * (1 - kTol)) return;
    // owners by increasing load; owners of equal load are interchangeable
    int ord[64];
    std::vector<int> ordv;
    int* o_list = ord;
    if (k > 64) {
      ordv.resize(k);
      o_list = ordv.data();
    }
    for (int o = 0; o < k; ++o) o_list[o] = o;
    std::stable_sort(o_list, o_list + k, [&](int a, int b) { return load[a] < load[b]; });
    double prev = -1.0;
    for (int t = 0; t < k; ++t) {
      const int o = o_list[t];
      if (t > 0 && load[o] == prev) continue;
      prev = load[o];
      const double nl = load[o] + c[j];
      if (nl >= best * (1 - kTol)) break;   // owners are in increasing load order
      load[o] = nl;
      cur[j] = o;
      dfs(j + 1, std::max(cur_max, nl));
      load[o] = prev;
      if (aborted) return;
    }
  }
};

double max_load(const std::vector<double>& costs, const std::vector<int32_t>& owner, int k,
                std::vector<double>* loads_out = nullptr) {
  std::vector<double> load(k, 0.0);
  for (size_t i = 0; i < costs.size(); ++i) load[owner[i]] += costs[i];
  if (loads_out) *loads_out = load;
  return costs.empty() ? 0.0 : *std::max_element(load.begin(), load.end());
}

// Moves and swaps that lower the most loaded owner's total, until none does.
void improve(const std::vector<double>& costs, std::vector<int32_t>& owner, int k) {
  const size_t n = costs.size();
  std::vector<double> load;
  max_load(costs, owner, k, &load);
  for (size_t iter = 0; iter < 4 * n * (size_t)k + 64; ++iter) {
    const int M = (int)(std::max_element(load.begin(), load.end()) - load.begin());
    const double top = load[M] * (1 - kTol);
    bool done = false;
    for (size_t i = 0; i < n && !done; ++i) {
      if (owner[i] != M || costs[i] <= 0) continue;
      for (int o = 0; o < k && !done; ++o)
        if (o != M && load[o] + costs[i] < top) {
          load[M] -= costs[i];
          load[o] += costs[i];
          owner[i] = o;
          done = true;
        }
    }
    for (size_t i = 0; i < n && !done; ++i) {
      if (owner[i] != M) continue;
      for (size_t j = 0; j < n && !done; ++j) {
        const int o = owner[j];
        if (o == M || costs[j] >= costs[i]) continue;
        if (load[o] - costs[j] + costs[i] < top) {
          load[M] += costs[j] - costs[i];
          load[o] += costs[i] - costs[j];
          owner[i] = o;
          owner[j] = M;
          done = true;
        }
      }
    }
    if (!done) break;
  }
}

}  // namespace

AssignResult assign_owners(const std::vector<double>& costs, int n_owners, int64_t node_limit) {
  AssignResult r;
  const size_t n = costs.size();
  const int k = n_owners;
  r.owner.assign(n, 0);
  if (n == 0) {
    r.optimal = true;
    return r;
  }
  // search order: decreasing cost, then index
  std::vector<size_t> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) { return costs[a] > costs[b]; });
  std::vector<double> sorted(n);
  for (size_t j = 0; j < n; ++j) sorted[j] = costs[order[j]];
  // LPT: each item, largest first, to the least-loaded owner (lowest index on ties)
  std::vector<double> load(k, 0.0);
  std::vector<int32_t> lpt(n);
  for (size_t j = 0; j < n; ++j) {
    const int o = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    lpt[j] = o;
    load[o] += sorted[j];
  }
  const double lpt_span = *std::max_element(load.begin(), load.end());
  const double total = std::accumulate(sorted.begin(), sorted.end(), 0.0);
  const double lower = std::max(sorted[0], total / k);
  std::vector<int32_t> best = lpt;
  bool optimal = lpt_span <= lower * (1 + kTol);
  if (!optimal) {
    Search s(sorted, k, node_limit, lpt_span, lpt);
    s.dfs(0, 0.0);
    best = s.best_owner;
    r.nodes = s.nodes;
    optimal = !s.aborted;
  }
  for (size_t j = 0; j < n; ++j) r.owner[order[j]] = best[j];
  if (!optimal) improve(costs, r.owner, k);
  r.makespan = max_load(costs, r.owner, k);
  r.optimal = optimal;
  return r;
}

}  // namespace muon
