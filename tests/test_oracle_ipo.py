"""Pins of the HCC-IPO stage-1 balancer oracle (FlashMask-3 page, §3.3 and the IPO
ablation table) against brute force, the lower bound and hand-worked cases."""
import itertools
import random

import pytest

from oracle import ipo


def _valid(owner, P, kappa):
    return all(owner.count(r) == kappa for r in range(P))


def test_lpt_hand_example():
    # weights 9 8 7 6 5 4 over P=2, kappa=3: LPT order 9,8,7,6,5,4
    # 9->r0, 8->r1, 7->r1 (8<9), 6->r0 (9<15), 5->r1 (15 = 15 -> lowest index r0? no:
    # r0 has 15, r1 has 15 -> r0), then r0 is full (3 chunks) so 4 -> r1
    owner = ipo.lpt([9, 8, 7, 6, 5, 4], 2, 3)
    assert owner == [0, 1, 1, 0, 0, 1]
    assert ipo.loads_of([9, 8, 7, 6, 5, 4], owner, 2) == [20, 19]


def _brute_split(items, w, k, kappa):
    best = None
    for lab in itertools.product(range(k), repeat=len(items)):
        if any(lab.count(g) != kappa for g in range(k)):
            continue
        m = max(sum(w[i] for i, l in zip(items, lab) if l == g) for g in range(k))
        best = m if best is None else min(best, m)
    return best


@pytest.mark.parametrize("seed", range(40))
def test_exact_split_matches_brute_force(seed):
    rng = random.Random(seed)
    k = rng.choice([2, 3])
    kappa = rng.choice([1, 2, 3])
    n = k * kappa
    w = [rng.randint(0, 30) for _ in range(n + 3)]
    items = rng.sample(range(len(w)), n)
    opt = _brute_split(items, w, k, kappa)
    res = ipo.exact_split(items, w, k, kappa, 10**9)
    assert res is not None and res[0] == opt
    groups = res[1]
    assert sorted(i for g in groups for i in g) == sorted(items)
    assert all(len(g) == kappa for g in groups)
    assert max(sum(w[i] for i in g) for g in groups) == opt
    # with the optimum itself as the bound nothing strictly better exists
    assert ipo.exact_split(items, w, k, kappa, opt) is None


@pytest.mark.parametrize("P,kappa", [(2, 2), (2, 4), (3, 2), (3, 3)])
@pytest.mark.parametrize("seed", range(8))
def test_ipo_exact_when_its_moves_cover_all_ranks(P, kappa, seed):
    """With P = 2 the pairwise step, and with P = 3 the three-rank step, re-split every
    chunk at once, so the result must be the brute-force optimum."""
    rng = random.Random(100 * P + 10 * kappa + seed)
    w = [rng.randint(1, 50) for _ in range(P * kappa)]
    owner, rep = ipo.ipo(w, P, kappa, stages=P)
    assert _valid(owner, P, kappa)
    assert rep["final"] == max(ipo.loads_of(w, owner, P))
    assert rep["final"] == ipo.brute_force_optimum(w, P, kappa)


@pytest.mark.parametrize("seed", range(25))
def test_ipo_bounds_on_tiny_instances(seed):
    rng = random.Random(seed)
    P, kappa = rng.choice([(4, 2), (3, 3), (5, 2)])
    w = [rng.randint(0, rng.choice([10, 100, 1000])) for _ in range(P * kappa)]
    opt = ipo.brute_force_optimum(w, P, kappa)
    o1, r1 = ipo.ipo(w, P, kappa, stages=1)
    o2, r2 = ipo.ipo(w, P, kappa, stages=2)
    o3, r3 = ipo.ipo(w, P, kappa, stages=3)
    for o in (o1, o2, o3):
        assert _valid(o, P, kappa)
    lb = ipo.lower_bound(w, P)
    assert lb <= opt <= r3["final"] <= r2["final"] <= r1["final"] == r1["lpt"]
    assert r3["lpt"] == r1["lpt"] and r2["p2"] == r2["final"]
    if r3["certified"]:
        assert r3["final"] == opt == lb


def test_repartition_closes_most_of_the_lpt_gap():
    """The ablation table's qualitative ordering on its uniform family (n = 64, P = 16,
    kappa = 4, weights uniform in [1, 1000]): LPT misses the lower bound on most
    instances, and the pairwise and three-rank repartitions close most of that gap.
    (The page reports LB-certified optima for every instance; under the move order
    adopted here the final makespan is within a few units of LB instead.)"""
    rng = random.Random(11)
    lpt_gap = p2_gap = final_gap = lpt_miss = 0
    trials = 12
    for _ in range(trials):
        w = [rng.randint(1, 1000) for _ in range(64)]
        _, rep = ipo.ipo(w, 16, 4, stages=3)
        assert rep["final"] <= rep["p2"] <= rep["lpt"]
        lpt_miss += rep["lpt"] > rep["lb"]
        lpt_gap += rep["lpt"] - rep["lb"]
        p2_gap += rep["p2"] - rep["lb"]
        final_gap += rep["final"] - rep["lb"]
    assert lpt_miss >= 0.8 * trials
    assert p2_gap <= 0.25 * lpt_gap
    assert final_gap <= 0.1 * lpt_gap
