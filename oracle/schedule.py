"""List scheduling of weighted items over P identical slots (oracle; tests only).

FlashMask-3 page, §3.3 ("Balance the work, not the length"): a rank's load is the
sum of its chunks' weights; the makespan is the largest load; a lower bound is
LB = max(ceil(sum w / P), max w).  The IPO ablation table compares
longest-processing-time-first (LPT) list scheduling with an exact optimum.  On one
GPU the slots are the compute units and the items are attention work items; the
order in which a kernel's workgroups are dispatched is this list.
"""
import heapq
import itertools
import math


def list_schedule(weights_in_order, P):
    """Greedy list scheduling: each item, in the given order, goes to the slot
    that becomes free first (ties to the lowest slot).  Returns (makespan, loads)."""
    heap = [(0, s) for s in range(P)]
    loads = [0] * P
    for w in weights_in_order:
        t, s = heapq.heappop(heap)
        loads[s] = t + w
        heapq.heappush(heap, (t + w, s))
    return max(loads) if loads else 0, loads


def lower_bound(weights, P):
    w = list(weights)
    if not w:
        return 0
    return max(math.ceil(sum(w) / P), max(w))


def brute_force_optimum(weights, P):
    """Exact minimum makespan by trying every assignment (tiny instances only)."""
    w = list(weights)
    best = sum(w)
    for assign in itertools.product(range(P), repeat=len(w)):
        loads = [0] * P
        for wi, s in zip(w, assign):
            loads[s] += wi
        best = min(best, max(loads))
    return best
