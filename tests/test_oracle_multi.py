"""Pins for the oracle's multi-interval mask form (FlashMask Guide, "Multi-Interval Sparse
Masks": up to 4 active row intervals per key column), CPU only.

The dense expansion is checked against a loop over the definition and against the
four-vector form on the masks both can write; attention against autograd through a
separately written dense-mask attention in torch; the tile rule against brute force
(sound everywhere, exact on block-aligned masks) and against the four-vector rule where
the forms coincide; localization through Theorem 1 of the FlashMask-3 page (§3.2)."""
import numpy as np
import pytest
import torch

import oracle
import workloads


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_dense_expansion_matches_the_definition():
    w = workloads.random_multi_intervals(1, 37, batch=2, n_intervals=4)
    for b in range(2):
        s, e = w.starts[b], w.ends[b]
        got = oracle.dense_mask_multi(s, e)
        want = np.ones((37, 37), dtype=bool)
        for i in range(37):
            for j in range(37):
                for m in range(4):
                    if s[m, j] <= i < e[m, j]:
                        want[i, j] = False
        assert np.array_equal(got, want)


def _one_interval_as_four_vectors(s, e, n):
    """Visible [s, e) == hidden [e, n) and [0, s): LTS = e, LTE = n, UTS = 0, UTE = s."""
    return e, np.full_like(e, n), np.zeros_like(s), s


def test_one_interval_equals_the_four_vector_form():
    n = 50
    w = workloads.random_multi_intervals(2, n, batch=3, n_intervals=1)
    for b in range(3):
        s, e = w.starts[b, 0].astype(np.int64), w.ends[b, 0].astype(np.int64)
        four = _one_interval_as_four_vectors(s, e, n)
        assert np.array_equal(oracle.dense_mask_multi(w.starts[b], w.ends[b]),
                              oracle.dense_mask(*four))
    # the tile rules agree on these masks too
    four = [np.stack(x) for x in zip(*[_one_interval_as_four_vectors(
        w.starts[b, 0].astype(np.int64), w.ends[b, 0].astype(np.int64), n) for b in range(3)])]
    for bq, bk in ((8, 8), (16, 4), (64, 32)):
        assert np.array_equal(oracle.classify_multi(w.starts, w.ends, bq, bk),
                              oracle.classify(*four, bq, bk))


def test_two_intervals_around_a_gap_equal_one_hidden_interval():
    n = 40
    rng = np.random.default_rng(3)
    a = np.sort(rng.integers(0, n + 1, (2, n)), axis=0)
    starts = np.stack([np.zeros(n, dtype=np.int64), a[1]])[None]
    ends = np.stack([a[0], np.full(n, n)])[None]
    four = (a[0], a[1], np.zeros(n, dtype=np.int64), np.zeros(n, dtype=np.int64))
    q, k, v, do = (rand((1, 2, n, 8), s) for s in range(4))
    got = oracle.attention_fwd_bwd_multi(q, k[:, :1], v[:, :1], do, starts, ends)
    want = oracle.attention_fwd_bwd(q, k[:, :1], v[:, :1], do, *(x[None] for x in four))
    for x, y in zip(got, want):
        assert np.array_equal(x, y)


def torch_dense(q, k, v, hidden, scale):
    g = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(g, dim=1)
    v = v.repeat_interleave(g, dim=1)
    s = scale * q @ k.transpose(-1, -2)
    s = s.masked_fill(hidden, float("-inf"))
    return torch.softmax(s, dim=-1) @ v, torch.logsumexp(s, dim=-1)


@pytest.mark.parametrize("M,hq,hkv,hm", [(1, 2, 1, 0), (2, 4, 2, 0), (3, 4, 2, 2), (4, 3, 1, 3)])
def test_multi_attention_vs_autograd(M, hq, hkv, hm):
    n, d, B = 36, 16, 2
    w = workloads.random_multi_intervals(M + 10, n, batch=B, heads_q=hq, heads_kv=hkv,
                                         n_intervals=M, mask_heads=hm, p_empty=0.3)
    per = hq // max(hm, 1)
    set_of = (lambda b, h: (w.starts[b], w.ends[b])) if hm == 0 else \
        (lambda b, h: (w.starts[b, h // per], w.ends[b, h // per]))
    hid = torch.from_numpy(np.stack([np.stack([oracle.dense_mask_multi(*set_of(b, h))
                                               for h in range(hq)]) for b in range(B)]))
    dead = hid.all(dim=-1)
    q, k, v, do = (rand(s, 70 + t) for t, s in
                   enumerate([(B, hq, n, d), (B, hkv, n, d), (B, hkv, n, d), (B, hq, n, d)]))
    O, LSE, dQ, dK, dV = oracle.attention_fwd_bwd_multi(q, k, v, do, w.starts, w.ends)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    hid_t = hid.clone()
    hid_t[dead] = False
    To, Tl = torch_dense(tq, tk, tv, hid_t, 1 / np.sqrt(d))
    live = ~dead
    (To * torch.from_numpy(do) * live[..., None].to(torch.float64)).sum().backward()
    L = live.numpy()
    assert np.abs(O[L] - To.detach().numpy()[L]).max() < 1e-12
    assert np.abs(LSE[L] - Tl.detach().numpy()[L]).max() < 1e-12
    assert np.abs(dQ[L] - tq.grad.numpy()[L]).max() < 1e-11
    assert np.abs(dK - tk.grad.numpy()).max() < 1e-11
    assert np.abs(dV - tv.grad.numpy()).max() < 1e-11
    assert (O[~L] == 0).all() and np.isneginf(LSE[~L]).all() and (dQ[~L] == 0).all()


def test_multi_rows_and_cols_consistent():
    n, d = 90, 8
    w = workloads.random_multi_intervals(4, n, batch=1, heads_q=2, n_intervals=4)
    q, do = rand((1, 2, n, d), 1), rand((1, 2, n, d), 2)
    k, v = rand((1, 1, n, d), 3), rand((1, 1, n, d), 4)
    O, LSE, dQ, dK, dV = oracle.attention_fwd_bwd_multi(q, k, v, do, w.starts, w.ends)
    rows = [0, 44, 89]
    Or, Lr, dQr = oracle.attention_rows_multi(q, k, v, do, w.starts, w.ends, 0, 1, rows)
    assert np.abs(Or - O[0, 1, rows]).max() < 1e-13 and np.abs(dQr - dQ[0, 1, rows]).max() < 1e-13
    cols = [0, 45, 89]
    dKc, dVc = oracle.attention_cols_multi(q, k, v, do, w.starts, w.ends, 0, 0, cols,
                                           row_block=16)
    assert np.abs(dKc - dK[0, 0, cols]).max() < 1e-12 and np.abs(dVc - dV[0, 0, cols]).max() < 1e-12


def test_block_minmax_multi():
    w = workloads.random_multi_intervals(5, 100, batch=2, n_intervals=3)
    mm = oracle.block_minmax_multi(w.starts, w.ends, 16)
    assert mm.shape == (2, 7, 12)
    for b in range(2):
        for kb in range(7):
            c = slice(kb * 16, min(kb * 16 + 16, 100))
            for m in range(3):
                s, e = w.starts[b, m, c], w.ends[b, m, c]
                assert list(mm[b, kb, 4 * m:4 * m + 4]) == [s.min(), s.max(), e.min(), e.max()]


@pytest.mark.parametrize("M", [1, 2, 4])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_multi_rule_is_sound(M, seed):
    n = 150
    w = workloads.random_multi_intervals(seed, n, batch=2, n_intervals=M, p_empty=0.3)
    for bq, bk, nq in ((16, 16, None), (32, 8, None), (8, 32, 100)):
        cls = oracle.classify_multi(w.starts, w.ends, bq, bk, nq=nq)
        truth = oracle.tile_truth_multi(w.starts, w.ends, bq, bk, nq=nq)
        for c in (0, 2):                  # skipped, unmasked
            sel = cls == c
            assert (truth[sel] == c).all()


def test_multi_rule_is_exact_on_block_aligned_masks():
    """Block-sparse masks whose intervals are whole query blocks, equal across each key
    block: every tile is entirely visible or entirely hidden, and the rule finds it."""
    n, blk = 2048, 128
    rng = np.random.default_rng(0)
    starts = np.zeros((2, 3, n), dtype=np.int64)      # unused intervals stay [0, 0)
    ends = np.zeros((2, 3, n), dtype=np.int64)
    for b in range(2):
        for kb in range(n // blk):
            qbs = np.sort(rng.choice(n // blk, size=int(rng.integers(0, 4)), replace=False))
            for t, qb in enumerate(qbs):
                starts[b, t, kb * blk:(kb + 1) * blk] = qb * blk
                ends[b, t, kb * blk:(kb + 1) * blk] = (qb + 1) * blk
    for bq, bk in ((128, 128), (64, 128), (128, 64), (32, 32)):
        cls = oracle.classify_multi(starts, ends, bq, bk)
        assert np.array_equal(cls, oracle.tile_truth_multi(starts, ends, bq, bk))
        assert (cls == 1).sum() == 0 and (cls == 2).sum() > 0


def test_theorem1_for_multi_intervals():
    """Localized multi-interval columns select exactly the rank's rows of the global
    intervals (the localization is the same renumbering of every row bound)."""
    n, C = 256, 32
    w = workloads.random_multi_intervals(8, n, batch=1, n_intervals=4)
    offs = [32, 96, 160, 224]
    rows = oracle.rank_rows(offs, C)
    ls = oracle.localize(w.starts, offs, C)
    le = oracle.localize(w.ends, offs, C)
    glob = oracle.dense_mask_multi(w.starts[0], w.ends[0])[rows]
    loc = oracle.dense_mask_multi(ls[0], le[0], nq=len(rows))
    assert np.array_equal(glob, loc)
