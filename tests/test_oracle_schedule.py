"""Pins for the list-scheduling helpers used to reason about LPT dispatch."""
import math

import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("seed", range(30))
def test_lpt_bounds_on_tiny_instances(seed):
    rng = np.random.default_rng(seed)
    P = int(rng.integers(2, 4))
    w = rng.integers(1, 20, int(rng.integers(3, 8))).tolist()
    opt = oracle.brute_force_optimum(w, P)
    lb = oracle.lower_bound(w, P)
    order = oracle.lpt_order(w)
    lpt, loads = oracle.list_schedule([w[i] for i in order], P)
    assert sum(loads) == sum(w)
    assert lb <= opt <= lpt
    # Graham's bound for LPT: makespan <= (4/3 - 1/(3P)) * OPT
    assert lpt <= (4 / 3 - 1 / (3 * P)) * opt + 1e-9


def test_lower_bound_closed_form():
    assert oracle.lower_bound([5, 5, 5, 1], 2) == 8
    assert oracle.lower_bound([9, 1, 1], 3) == 9
    assert oracle.lower_bound([], 4) == 0


def test_known_lpt_gap():
    # the classic instance where LPT is not optimal: {3,3,2,2,2} on 2 slots
    w = [3, 3, 2, 2, 2]
    lpt, _ = oracle.list_schedule([w[i] for i in oracle.lpt_order(w)], 2)
    assert lpt == 7 and oracle.brute_force_optimum(w, 2) == 6
