"""Host logic of bench.py (CPU only): the attended-pair counts behind the effective
TFLOP/s metric, by interval arithmetic, against dense counts from the oracle's mask."""
import numpy as np
import pytest

import bench
import oracle
import workloads


@pytest.mark.parametrize("seed", [0, 1])
def test_attended_pairs_four_vector_form(seed):
    w = workloads.random_intervals(seed, 120, batch=2, heads_q=3)
    dense = sum(int((~oracle.dense_mask(*(x[b] for x in w.vectors()))).sum()) for b in range(2))
    assert bench.attended_pairs(w) == 3 * dense


def test_attended_pairs_per_head_sets():
    w = workloads.random_intervals(4, 96, batch=2, heads_q=4, mask_heads=2)
    dense = sum(int((~oracle.dense_mask(*(x[b, m] for x in w.vectors()))).sum())
                for b in range(2) for m in range(2))
    assert bench.attended_pairs(w) == 2 * dense     # two query heads per set


@pytest.mark.parametrize("M,hm", [(1, 0), (3, 0), (4, 2)])
def test_attended_pairs_multi_interval(M, hm):
    w = workloads.random_multi_intervals(M, 110, batch=2, heads_q=4, n_intervals=M,
                                         mask_heads=hm)
    sets = [(w.starts[b], w.ends[b]) for b in range(2)] if hm == 0 else \
        [(w.starts[b, m], w.ends[b, m]) for b in range(2) for m in range(hm)]
    dense = sum(int((~oracle.dense_mask_multi(s, e)).sum()) for s, e in sets)
    assert bench.attended_pairs_multi(w) == dense * (4 // max(hm, 1))


@pytest.mark.parametrize("hm", [0, 2])
def test_attended_pairs_block_sparse(hm):
    n = 300                                        # ragged last block row and column
    w = workloads.random_blocks(hm + 1, n, batch=2, heads_q=4, density=0.4, mask_heads=hm)
    grids = [w.blocks[b] for b in range(2)] if hm == 0 else \
        [w.blocks[b, m] for b in range(2) for m in range(hm)]
    dense = sum(int((~oracle.dense_mask_blocks(g, n, n)).sum()) for g in grids)
    assert bench.attended_pairs_blocks(w) == dense * (4 // max(hm, 1))


def test_benchmark_workloads_pair_counts_are_positive():
    for name in workloads.CONFIG_NAMES[:2] + workloads.VARIANT_NAMES:
        w = workloads.make_workload(name)
        if isinstance(w, workloads.BlockWorkload):
            a = bench.attended_pairs_blocks(w)
        elif isinstance(w, workloads.MultiWorkload):
            a = bench.attended_pairs_multi(w)
        else:
            a = bench.attended_pairs(w)
        assert 0 < a <= w.batch * w.heads_q * w.seqlen ** 2


def test_clock_mean_needs_enough_samples():
    """A mean clock is reported only from MIN_SAMPLES readings on: short runs catch the clock
    ramping or idle between launches."""
    c = bench.ClockSampler.__new__(bench.ClockSampler)
    c.samples = [1900.0] * (bench.ClockSampler.MIN_SAMPLES - 1)
    assert c.mean() is None
    c.samples.append(1800.0)
    assert abs(c.mean() - (1900.0 * (len(c.samples) - 1) + 1800.0) / len(c.samples)) < 1e-9
