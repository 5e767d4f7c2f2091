// Owner assignment: host-only, no device calls.
//
// DMuon announcement (wjxwpt.net), improvement 3 "computation-aware load
// balancing"; DMuon announcement (zaocj.com), third of the three moves: each
// matrix's update is computed by exactly one owner, the per-shape step time is
// measured once, and the assignment minimizes the finishing time of the
// slowest owner (the page solves it as a mixed integer linear program).
//
// Here: the makespan max_o sum_{i: owner[i] = o} cost[i] is minimized exactly
// by depth-first branch and bound (items in decreasing cost; owners of equal
// load tried once; bound max(current max load, total / owners)), seeded with
// the LPT schedule.  When the node budget runs out the best schedule found so
// far is returned, improved by moves and swaps off the most loaded owner, and
// flagged as not proven optimal.
#pragma once
#include <stdint.h>

#include <vector>

namespace muon {

struct AssignResult {
  std::vector<int32_t> owner;   // owner of each item, in [0, n_owners)
  double makespan = 0;
  bool optimal = false;         // proven minimal (search finished or LPT met the lower bound)
  int64_t nodes = 0;            // branch-and-bound nodes visited
};

// costs: n >= 0 finite, non-negative values; n_owners >= 1; node_limit > 0.
AssignResult assign_owners(const std::vector<double>& costs, int n_owners, int64_t node_limit);

}  // namespace muon
