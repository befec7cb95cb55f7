"""fm_ipo_balance (host C++ in libfm) against the oracle: identical assignments and
reports on random instances, brute-force optimality where the moves cover all ranks,
argument checks.  Host code: runs without a GPU."""
import random

import numpy as np
import pytest

import mask_aware_sparse_amd as fm
from oracle import ipo


def _case(seed):
    rng = random.Random(seed)
    P = rng.choice([2, 3, 4, 6, 8, 16])
    kappa = rng.choice([1, 2, 3, 4])
    wmax = rng.choice([1, 5, 200, 1000, 10**4, 10**9])
    w = [rng.randint(0, wmax) for _ in range(P * kappa)]
    if rng.random() < 0.2:                     # causal-like chunk loads
        w = [i + 1 for i in range(P * kappa)]
    return w, P, kappa


@pytest.mark.parametrize("seed", range(60))
@pytest.mark.parametrize("stages", [1, 2, 3])
def test_matches_oracle(seed, stages):
    w, P, kappa = _case(seed)
    owner, rep = fm.ipo_balance(w, P, stages)
    o_ref, r_ref = ipo.ipo(w, P, kappa, stages)
    assert owner.tolist() == o_ref
    for key in ("lb", "lpt", "p2", "final", "certified", "moves"):
        assert rep[key] == r_ref[key], key
    assert all((owner == r).sum() == kappa for r in range(P))


@pytest.mark.parametrize("seed", range(6))
def test_table_sizes_match_oracle(seed):
    """The ablation table's instance sizes (n = 64, P = 16, kappa = 4)."""
    rng = random.Random(1000 + seed)
    w = [rng.randint(1, 1000) for _ in range(64)]
    owner, rep = fm.ipo_balance(w, 16, 3)
    o_ref, r_ref = ipo.ipo(w, 16, 4, 3)
    assert owner.tolist() == o_ref and rep["final"] == r_ref["final"]


@pytest.mark.parametrize("P,kappa", [(2, 3), (3, 2), (3, 3)])
@pytest.mark.parametrize("seed", range(5))
def test_exact_when_moves_cover_all_ranks(P, kappa, seed):
    rng = random.Random(7 * seed + P)
    w = [rng.randint(1, 99) for _ in range(P * kappa)]
    _, rep = fm.ipo_balance(w, P, P)
    assert rep["final"] == ipo.brute_force_optimum(w, P, kappa)


def test_argument_checks():
    lib = fm.library()
    w = np.arange(8, dtype=np.int64)
    with pytest.raises(fm.FMError):
        fm.ipo_balance(w, 3)             # 8 chunks over 3 ranks
    with pytest.raises(fm.FMError):
        fm.ipo_balance(w, 0)
    with pytest.raises(fm.FMError):
        fm.ipo_balance(w, 2, stages=4)
    with pytest.raises(fm.FMError):
        fm.ipo_balance(np.array([1, -1], dtype=np.int64), 1)
    with pytest.raises(fm.FMError):      # kappa = 17 > FM_IPO_MAX_KAPPA
        fm.ipo_balance(np.ones(17, dtype=np.int64), 1)
    assert fm.ipo_balance(np.ones(16, dtype=np.int64), 1)[1]["certified"]
