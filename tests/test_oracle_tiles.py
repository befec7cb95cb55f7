"""Pins for the oracle's tile classification, queues, costs and LPT order."""
import numpy as np
import pytest

import oracle
import workloads
from oracle.tiles import PARTIAL, SKIP, UNMASKED


def nb(n, b):
    return (n + b - 1) // b


def rule_lts_ute(lts, ute, n, bq, bk):
    """The rule exactly as the FlashMask-3 page states it (§3.1), valid when LTE = N
    and UTS = 0: skip if q0 >= max LTS or q1 <= min UTE; unmasked if q1 <= min LTS
    and q0 >= max UTE; otherwise partial."""
    out = np.zeros((nb(n, bq), nb(n, bk)), dtype=np.uint8)
    for qb in range(nb(n, bq)):
        q0, q1 = qb * bq, min(qb * bq + bq, n)
        for kb in range(nb(n, bk)):
            c = slice(kb * bk, min(kb * bk + bk, n))
            if q0 >= lts[c].max() or q1 <= ute[c].min():
                out[qb, kb] = SKIP
            elif q1 <= lts[c].min() and q0 >= ute[c].max():
                out[qb, kb] = UNMASKED
            else:
                out[qb, kb] = PARTIAL
    return out


def rule_fms_fme(fms, fme, n, bq, bk):
    """The FlashMask Guide's statement ("On-Chip Block-Skipping Logic") with an
    inclusive row range [R_start, R_end] and an inclusive visible interval
    FMS <= i <= FME: skip if R_end < min FMS or R_start > max FME; fully visible
    if R_start >= max FMS and R_end <= min FME."""
    out = np.zeros((nb(n, bq), nb(n, bk)), dtype=np.uint8)
    for qb in range(nb(n, bq)):
        r0, r1 = qb * bq, min(qb * bq + bq, n) - 1
        for kb in range(nb(n, bk)):
            c = slice(kb * bk, min(kb * bk + bk, n))
            if r1 < fms[c].min() or r0 > fme[c].max():
                out[qb, kb] = SKIP
            elif r0 >= fms[c].max() and r1 <= fme[c].min():
                out[qb, kb] = UNMASKED
            else:
                out[qb, kb] = PARTIAL
    return out


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("shape", [(64, 8, 8), (100, 16, 8), (77, 8, 16), (256, 32, 64)])
def test_rule_equals_both_printed_statements(seed, shape):
    n, bq, bk = shape
    rng = np.random.default_rng(seed)
    # LTS/UTE masks (LTE = N, UTS = 0) from random visible intervals FMS <= FME
    a = rng.integers(0, n, (2, n))
    fms, fme = np.minimum(a[0], a[1]), np.maximum(a[0], a[1])
    lts, lte, uts, ute = oracle.visible_interval_to_vectors(fms, fme, n)
    cls = oracle.classify(lts[None], lte[None], uts[None], ute[None], bq, bk)[0]
    assert (cls == rule_lts_ute(lts, ute, n, bq, bk)).all()
    assert (cls == rule_fms_fme(fms, fme, n, bq, bk)).all()


@pytest.mark.parametrize("seed", range(25))
def test_rule_sound_on_adversarial_vectors(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 90))
    bq, bk = (int(x) for x in rng.choice([1, 2, 4, 8, 16], 2))
    w = workloads.random_intervals(seed, n, batch=2, p_empty=0.3)
    cls = oracle.classify(*w.vectors(), bq, bk)
    truth = oracle.tile_truth(*w.vectors(), bq, bk)
    assert ((cls != SKIP) | (truth == SKIP)).all()           # skip => all hidden
    assert ((cls != UNMASKED) | (truth == UNMASKED)).all()   # unmasked => none hidden
    assert ((truth != SKIP) | (cls != UNMASKED)).all()


@pytest.mark.parametrize("make,bq,bk", [
    (lambda: workloads.causal_doc(0), 128, 128),
    (lambda: workloads.causal_doc(1), 64, 32),
    (lambda: workloads.prefix_lm_doc(0, n=2048, lo=128, hi=512), 128, 64),
    (lambda: workloads.sliding_window_sinks(n=4096, window=512, sinks=64), 128, 128),
    (lambda: workloads.sliding_window_sinks(n=2000, window=300, sinks=10), 64, 128),
    (lambda: workloads.random_eviction(0, n=1024), 128, 64),
    (lambda: workloads.random_eviction(2, n=1000), 8, 8),
])
def test_rule_exact_on_workload_families(make, bq, bk):
    w = make()
    cls = oracle.classify(*w.vectors(), bq, bk)
    assert (cls == oracle.tile_truth(*w.vectors(), bq, bk)).all()


def test_rule_conservative_example():
    # N=16, Bq=4, Bk=16: LTS_j = 4 for j < 8 and N otherwise, UTE_j = j.  Rows 4..7
    # are hidden in every column (lower interval for j < 8, upper for j >= 8), yet
    # the block min/max cannot tell: the rule calls the tile partial.
    n = 16
    lts = np.where(np.arange(n) < 8, 4, n)[None]
    lte = np.full((1, n), n); uts = np.zeros((1, n)); ute = np.arange(n)[None]
    cls = oracle.classify(lts, lte, uts, ute, 4, 16)
    truth = oracle.tile_truth(lts, lte, uts, ute, 4, 16)
    assert truth[0, 1, 0] == SKIP and cls[0, 1, 0] == PARTIAL


def test_ragged_tail_clamped():
    # N=10 with 4x4 tiles: the last Q block holds rows 8..9 only, the last KV block
    # columns 8..9 only.  Causal: tile (2, 2) is partial, (2, 1) unmasked.
    n = 10
    w = workloads.causal(n)
    cls = oracle.classify(*w.vectors(), 4, 4)[0]
    assert cls.shape == (3, 3)
    assert cls[2, 2] == PARTIAL and cls[2, 1] == UNMASKED and cls[1, 2] == SKIP


def test_queues_counts_costs_order():
    w = workloads.causal_doc(0)
    cls = oracle.classify(*w.vectors(), 128, 64)
    qq, qc, kq, kc = oracle.queues(cls)
    B, nqb, nkb = cls.shape
    for qb in range(nqb):
        live = [kb for kb in range(nkb) if cls[0, qb, kb] != SKIP][::-1]
        n = len(live)
        got = qq[0, qb, :n].view(np.uint32)
        assert list(got & 0x7FFFFFFF) == live                     # right to left
        assert list(got >> 31) == [int(cls[0, qb, kb] == PARTIAL) for kb in live]
        assert (qq[0, qb, n:] == -1).all()
        assert qc[0, qb, 0] == (cls[0, qb] == PARTIAL).sum()
        assert qc[0, qb, 1] == (cls[0, qb] == UNMASKED).sum()
    for kb in range(nkb):
        live = [qb for qb in range(nqb) if cls[0, qb, kb] != SKIP]
        got = kq[0, kb, :len(live)].view(np.uint32)
        assert list(got & 0x7FFFFFFF) == live
        assert kc[0, kb].sum() == len(live)
    cost = oracle.tile_costs(qc)
    assert (cost == 11 * qc[..., 0] + 10 * qc[..., 1]).all()
    order = oracle.lpt_order(cost)
    flat = cost.reshape(-1)
    assert sorted(order.tolist()) == list(range(flat.size))
    for a, b in zip(order[:-1], order[1:]):
        assert flat[a] > flat[b] or (flat[a] == flat[b] and a < b)


def test_lpt_order_examples():
    assert oracle.lpt_order([3, 7, 7, 0, 5]).tolist() == [1, 2, 4, 0, 3]
    assert oracle.lpt_order(np.array([[1, 2], [2, 1]])).tolist() == [1, 2, 0, 3]
