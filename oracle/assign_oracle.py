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
