"""Pins of the key-reordering oracle (oracle/keyorder.py): hand-worked examples of the
rule, the minimality of the sorted candidate against brute force, the natural order kept
on masks whose lower starts never decrease, and the invariance of attention (forward and
backward) under the joint permutation of K, V and the vectors."""
import itertools

import numpy as np
import pytest

import oracle
import workloads


def test_hand_example_sorted_and_natural_superblocks():
    # 16 keys, super-blocks of 8, groups of 4, N_q = 16; UTE_j = j (causal), LTE = 16.
    # Super-block 0: LTS = 9 3 12 5 | 9 2 15 7.  Natural groups {0..3}, {4..7}:
    #   LTS ranges 12-3 = 9 and 15-2 = 13, UTE ranges 3 and 3 -> spread 28.
    # Stable sort by LTS: 2(5) 3(1) 5(3) 7(7) | 9(0) 9(4) 12(2) 15(6):
    #   LTS ranges 5 and 6, UTE ranges {1,3,5,7} -> 6 and {0,2,4,6} -> 6 -> spread 23 < 28.
    # Super-block 1: LTS = 8..15 ascending -> the sorted order is the natural one (a tie:
    #   natural kept).
    lts = np.array([9, 3, 12, 5, 9, 2, 15, 7] + list(range(8, 16)))
    lte = np.full(16, 16)
    uts = np.zeros(16, dtype=np.int64)
    ute = np.arange(16)
    perm = oracle.key_order(lts, lte, uts, ute, 16, span=8, group=4)
    assert perm.tolist() == [5, 1, 3, 7, 0, 4, 2, 6] + list(range(8, 16))
    assert oracle.spread([x[:8] for x in (lts, lte, uts, ute)], 16, 4) == 28
    assert oracle.spread([x[perm[:8]] for x in (lts, lte, uts, ute)], 16, 4) == 23


def test_hand_example_sort_would_widen():
    # 4 keys, one super-block, groups of 2, N_q = 100.  LTS = 10 0 10 0, UTE = 0 0 90 90.
    # Natural: groups {0,1}: LTS range 10, UTE 0; {2,3}: LTS 10, UTE 0 -> spread 20.
    # Sorted by LTS: 1 3 0 2: {1,3}: LTS 0, UTE 90; {0,2}: LTS 0, UTE 90 -> 180 > 20.
    lts = np.array([10, 0, 10, 0])
    lte = np.full(4, 100)
    uts = np.zeros(4, dtype=np.int64)
    ute = np.array([0, 0, 90, 90])
    assert oracle.key_order(lts, lte, uts, ute, 100, span=4, group=2).tolist() == [0, 1, 2, 3]


def test_clipping_to_query_rows():
    # Bounds beyond N_q count as N_q: LTS = 50 and 90 with N_q = 40 are the same row.
    # Natural groups of 2: {50, 10}, {90, 5} -> ranges 30 and 35 (clipped 40-10, 40-5).
    # Sorted: 5(3) 10(1) | 50(0) 90(2) -> ranges 5 and 0: sorted wins.
    lts = np.array([50, 10, 90, 5])
    z = np.zeros(4, dtype=np.int64)
    assert oracle.spread([lts, z, z, z], 40, 2) == 65
    assert oracle.key_order(lts, z, z, z, 40, span=4, group=2).tolist() == [3, 1, 0, 2]


def test_ragged_last_superblock_and_group():
    # 11 keys, super-blocks of 8 (the last holds 3), groups of 4 (ragged inside too).
    rng = np.random.default_rng(3)
    lts = rng.integers(0, 50, 11)
    z = np.zeros(11, dtype=np.int64)
    perm = oracle.key_order(lts, z, z, z, 50, span=8, group=4)
    # keys stay in their super-block, and with only LTS varying the sorted order is taken
    # whenever it is not the natural order
    assert sorted(perm[:8].tolist()) == list(range(8))
    assert sorted(perm[8:].tolist()) == [8, 9, 10]
    for s0, s1 in ((0, 8), (8, 11)):
        seg = np.arange(s0, s1)
        srt = seg[np.argsort(lts[seg], kind="stable")]
        nat = oracle.spread([lts[seg], z[seg], z[seg], z[seg]], 50, 4)
        sv = oracle.spread([lts[srt], z[seg], z[seg], z[seg]], 50, 4)
        assert perm[s0:s1].tolist() == (srt.tolist() if sv < nat else seg.tolist())


@pytest.mark.parametrize("seed", range(12))
def test_sorted_candidate_minimizes_lts_spread_brute_force(seed):
    # Over all orders of a tiny super-block, no order has a smaller LTS spread than the
    # sorted one; with only LTS varying, the rule's result attains that minimum.
    rng = np.random.default_rng(seed)
    n, g = 6, int(rng.integers(2, 4))
    lts = rng.integers(0, 30, n)
    z = np.zeros(n, dtype=np.int64)
    best = min(oracle.spread([lts[list(o)], z, z, z], 30, g)
               for o in itertools.permutations(range(n)))
    perm = oracle.key_order(lts, z, z, z, 30, span=n, group=g)
    assert oracle.spread([lts[perm], z, z, z], 30, g) == best
    assert sorted(perm.tolist()) == list(range(n))


@pytest.mark.parametrize("name", ["c1_causal_doc_1k", "c2_prefix_lm_doc_8k",
                                  "c3_share_question_32k", "c4_sliding_window_128k"])
def test_structured_masks_keep_natural_order(name):
    w = workloads.make_workload(name)
    vecs = [np.asarray(x).reshape(-1, w.seqlen) for x in w.vectors()]
    perm = oracle.key_order_rows(*vecs, w.seqlen)
    assert np.array_equal(perm, np.broadcast_to(np.arange(w.seqlen), perm.shape))


def test_random_eviction_sorts_and_narrows():
    w = workloads.random_eviction(0, n=16384, heads_q=1)
    v = [np.asarray(x).reshape(-1, w.seqlen)[0] for x in w.vectors()]
    perm = oracle.key_order(*v, w.seqlen)
    sorted_blocks = 0
    for s0 in range(0, w.seqlen, 2048):
        nat = np.arange(s0, s0 + 2048)
        chosen = perm[s0:s0 + 2048]
        a = oracle.spread([x[chosen] for x in v], w.seqlen, 64)
        b = oracle.spread([x[nat] for x in v], w.seqlen, 64)
        assert a <= b
        sorted_blocks += int(not np.array_equal(chosen, nat))
    assert sorted_blocks >= 6
    # and the forward tile cost drops by over a third (by half at 128K keys)
    pv = [x[perm] for x in v]
    def cost(vv):
        cls = oracle.classify(*(x[None, :] for x in vv), 128, 64)
        return 11 * int((cls == 1).sum()) + 10 * int((cls == 2).sum())
    assert cost(pv) < 0.65 * cost(v)


@pytest.mark.parametrize("seed", range(3))
def test_attention_invariant_under_joint_permutation(seed):
    # O, LSE, dQ from the permuted keys, and dK, dV permuted back, equal the natural ones.
    w = workloads.random_eviction(seed, n=300, heads_q=2, heads_kv=1)
    q, k, v, do = (t.double().numpy() for t in workloads.make_tensors(w))
    vecs = w.vectors()
    perm = oracle.key_order(*(np.asarray(x).reshape(-1, 300)[0] for x in vecs), 300,
                            span=128, group=16)
    assert not np.array_equal(perm, np.arange(300))
    ref = oracle.attention_fwd_bwd(q, k, v, do, *vecs)
    pvecs = [np.asarray(x)[..., perm] for x in vecs]
    got = oracle.attention_fwd_bwd(q, k[..., perm, :], v[..., perm, :], do, *pvecs)
    inv = np.argsort(perm)
    for a, b in zip(got[:3], ref[:3]):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got[3][..., inv, :], ref[3], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got[4][..., inv, :], ref[4], rtol=1e-12, atol=1e-12)
