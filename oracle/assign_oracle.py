"""Brute-force owner assignment: the plain definition of what the library's
owner-assignment solver computes.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests use it.  It shares no code with the
library's solver.

DMuon announcement (wjxwpt.net), improvement 3 "computation-aware load
balancing", and DMuon announcement (zaocj.com), third of the three moves:
every matrix's update is computed by exactly one owner; the per-shape step
time is measured once, and matrices are assigned to owners so that the
slowest owner finishes as early as possible (the page names a mixed integer
linear program for it).  The objective is therefore the makespan

    C(owner) = max over owners o of  sum of costs[i] for i with owner[i] == o

and the solver's result is an assignment that minimizes it.  Here that
minimum is found by trying every one of n_owners ** n assignments, so only
tiny instances are possible.
"""
import itertools


def makespan(costs, owner, n_owners):
    """Largest per-owner total of an assignment (owner[i] in [0, n_owners))."""
    loads = [0.0] * n_owners
    for c, o in zip(costs, owner):
        loads[o] += c
    return max(loads) if loads else 0.0


def best_makespan(costs, n_owners):
    """Minimum makespan over all assignments, and one assignment reaching it."""
    n = len(costs)
    if n == 0:
        return 0.0, []
    best, arg = None, None
    for owner in itertools.product(range(n_owners), repeat=n):
        m = makespan(costs, owner, n_owners)
        if best is None or m < best:
            best, arg = m, list(owner)
    return best, arg


def best_makespan_by_counts(costs, n_owners, max_states=200000):
    """Minimum makespan by dynamic programming over how many items of each
    distinct cost every owner takes: with d distinct costs c_j held n_j times,
    f(owners, r) = min over a take t <= r of max(sum_j t_j c_j, f(owners - 1, r - t))
    and f(1, r) = sum_j r_j c_j.  Exact; practical when the items come in few
    distinct costs (the workloads' matrix sets).  Returns None when the count
    vectors exceed max_states."""
    from functools import lru_cache

    groups = {}
    for c in costs:
        groups[c] = groups.get(c, 0) + 1
    vals = sorted(groups)
    counts = tuple(groups[v] for v in vals)
    states = 1
    for n in counts:
        states *= n + 1
    if states > max_states:
        return None
    if not costs:
        return 0.0
    takes = list(itertools.product(*(range(n + 1) for n in counts)))

    def load(t):
        return sum(k * v for k, v in zip(t, vals))

    @lru_cache(maxsize=None)
    def f(owners, rem):
        if owners == 1:
            return load(rem)
        best = load(rem)          # this owner takes everything left
        for t in takes:
            if any(a > b for a, b in zip(t, rem)):
                continue
            lt = load(t)
            if lt >= best:
                continue
            rest = f(owners - 1, tuple(b - a for a, b in zip(t, rem)))
            best = min(best, max(lt, rest))
        return best

    return f(n_owners, counts)
