"""Stage-1 chunk balancing of HCC-IPO (oracle; test infrastructure only).

FlashMask-3 page, §3.3 ("Balance the work, not the length"): context parallelism cuts
the query axis into n = P * kappa chunks, each rank receives exactly kappa of them,
and the makespan Phi = max over ranks of the summed chunk loads is minimised under
that cardinality constraint.  The lower bound is LB = max(ceil(sum w / P), max w); a
result whose makespan reaches LB is certified optimal.  The page's ablation table
names three phases: longest-processing-time-first (LPT), exact pairwise repartition
(P2) and three-rank repartition (P3).  The page gives no pseudo-code; the reading
written out here (and restated in the library) is:

  LPT  chunks in (weight descending, index ascending) order; each goes to the least
       loaded rank that still has fewer than kappa chunks (ties: lowest rank).
  P2   repeat: for ranks a in (load descending, index ascending) order and partners
       b in (load ascending, index ascending) order with load(b) <= load(a) - 2,
       re-split the 2 kappa chunks of {a, b} exactly (minimum larger half, kappa
       chunks each) and apply the first split whose maximum is below load(a); stop
       when no pair improves or Phi = LB.  Every move lowers the larger load of its
       pair, so the sum of squared loads falls and the loop ends.
  P3   the same over triples: a in (load descending, index ascending) order, {b, c}
       other ranks that a dominates (load below load(a), or equal with a higher index),
       in (load(b) + load(c) ascending, then (b, c) lexicographic) order, skipped when
       3 load(a) - load(a) - load(b) - load(c) < 2; the first exact three-way re-split
       whose maximum is below load(a) is applied and P2 runs again; stop when no triple
       improves or Phi = LB.

The exact re-split is a depth-first search: chunks in (weight descending, index
ascending) order, each placed in group 0, 1, ... (at most kappa per group; an empty
group is tried only if no earlier group is empty); a branch is cut when a group sum
would reach the best maximum found so far; the search starts from the current
maximum (only strictly better splits count) and stops once the pool's own bound
max(ceil(S / k), max w) is reached.  Groups go to the ranks in ascending rank order.
"""
import math


def lower_bound(w, P):
    w = list(w)
    if not w:
        return 0
    return max(math.ceil(sum(w) / P), max(w))


def loads_of(w, owner, P):
    L = [0] * P
    for wi, r in zip(w, owner):
        L[r] += wi
    return L


def lpt(w, P, kappa):
    """LPT under the cardinality constraint; returns owner[i] (rank of chunk i)."""
    n = len(w)
    assert n == P * kappa
    order = sorted(range(n), key=lambda i: (-w[i], i))
    load = [0] * P
    cnt = [0] * P
    owner = [-1] * n
    for i in order:
        best = None
        for r in range(P):
            if cnt[r] < kappa and (best is None or load[r] < load[best]):
                best = r
        owner[i] = best
        load[best] += w[i]
        cnt[best] += 1
    return owner


def exact_split(items, weights, k, kappa, bound):
    """Best split of `items` (chunk ids) into k groups of `kappa` with maximum group
    sum strictly below `bound`; returns (max, groups) or None if none is below it."""
    order = sorted(items, key=lambda i: (-weights[i], i))
    total = sum(weights[i] for i in order)
    target = max(math.ceil(total / k), max(weights[i] for i in order))
    best = [bound, None]
    sums = [0] * k
    cnts = [0] * k
    place = [0] * len(order)

    def dfs(pos):
        if best[0] <= target:
            return
        if pos == len(order):
            m = max(sums)
            if m < best[0]:
                best[0] = m
                best[1] = list(place)
            return
        wi = weights[order[pos]]
        seen_empty = False
        for g in range(k):
            if cnts[g] == kappa:
                continue
            if cnts[g] == 0:
                if seen_empty:
                    continue
                seen_empty = True
            if sums[g] + wi >= best[0]:
                continue
            sums[g] += wi
            cnts[g] += 1
            place[pos] = g
            dfs(pos + 1)
            sums[g] -= wi
            cnts[g] -= 1
            if best[0] <= target:
                return

    dfs(0)
    if best[1] is None:
        return None
    groups = [[] for _ in range(k)]
    for pos, g in enumerate(best[1]):
        groups[g].append(order[pos])
    return best[0], groups


def _apply(owner, ranks, groups):
    for r, grp in zip(sorted(ranks), groups):
        for i in grp:
            owner[i] = r


def ipo(w, P, kappa, stages=3):
    """LPT, then P2 (stages >= 2) and P3 (stages >= 3).  Returns (owner, report) with
    report = {lb, lpt, p2, final, certified, moves}: makespans after LPT, after the first
    P2 convergence, and at the end."""
    w = [int(x) for x in w]
    owner = lpt(w, P, kappa)
    lb = lower_bound(w, P)
    rep = {"lb": lb, "lpt": max(loads_of(w, owner, P)), "moves": 0}
    members = lambda r: [i for i in range(len(w)) if owner[i] == r]
    by_load_desc = lambda load: sorted(range(P), key=lambda r: (-load[r], r))

    def p2():
        while True:
            load = loads_of(w, owner, P)
            if max(load) <= lb:
                return
            moved = False
            for a in by_load_desc(load):
                for b in sorted(range(P), key=lambda r: (load[r], r)):
                    if b == a or load[b] > load[a] - 2:
                        continue
                    res = exact_split(members(a) + members(b), w, 2, kappa, load[a])
                    if res is not None:
                        _apply(owner, (a, b), res[1])
                        rep["moves"] += 1
                        moved = True
                        break
                if moved:
                    break
            if not moved:
                return

    def dominated(a, r, load):
        return r != a and (load[r] < load[a] or (load[r] == load[a] and r > a))

    if stages >= 2:
        p2()
    rep["p2"] = max(loads_of(w, owner, P))
    while stages >= 3:
        load = loads_of(w, owner, P)
        if max(load) <= lb:
            break
        moved = False
        for a in by_load_desc(load):
            others = [r for r in range(P) if dominated(a, r, load)]
            pairs = sorted(((b, c) for x, b in enumerate(others) for c in others[x + 1:]),
                           key=lambda bc: (load[bc[0]] + load[bc[1]], bc))
            for b, c in pairs:
                if 3 * load[a] - load[a] - load[b] - load[c] < 2:
                    continue
                res = exact_split(members(a) + members(b) + members(c), w, 3, kappa, load[a])
                if res is not None:
                    _apply(owner, (a, b, c), res[1])
                    rep["moves"] += 1
                    moved = True
                    break
            if moved:
                break
        if not moved:
            break
        p2()
    rep["final"] = max(loads_of(w, owner, P))
    rep["certified"] = rep["final"] == lb
    return owner, rep


def brute_force_optimum(w, P, kappa):
    """Exact minimum makespan under the cardinality constraint, by enumerating every
    assignment (tiny instances only)."""
    n = len(w)
    best = [sum(w)]
    load = [0] * P
    cnt = [0] * P

    def rec(i):
        if i == n:
            best[0] = min(best[0], max(load))
            return
        for r in range(P):
            if cnt[r] < kappa:
                load[r] += w[i]
                cnt[r] += 1
                rec(i + 1)
                load[r] -= w[i]
                cnt[r] -= 1

    rec(0)
    return best[0]
