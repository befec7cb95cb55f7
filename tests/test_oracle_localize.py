"""Pins of the mask localization oracle (FlashMask-3 page, §3.2 and Theorem 1):
the sum form against the page's printed max form and a brute-force count, and the
localized mask and attention against the global ones restricted to the rank's rows."""
import numpy as np
import pytest

import oracle
import workloads


def _chunks(rng, n_total, chunk_len, k):
    nchunks = n_total // chunk_len
    return sorted(int(c) * chunk_len for c in rng.choice(nchunks, size=k, replace=False))


@pytest.mark.parametrize("seed", range(20))
def test_sum_form_equals_max_form_and_count(seed):
    rng = np.random.default_rng(seed)
    C = int(rng.integers(1, 9))
    n = C * int(rng.integers(2, 12))
    offs = _chunks(rng, n, C, int(rng.integers(1, n // C + 1)))
    x = np.arange(0, n + 1)
    rows = oracle.rank_rows(offs, C)
    brute = np.array([(rows < xi).sum() for xi in x])
    assert np.array_equal(oracle.localize(x, offs, C), brute)
    assert np.array_equal(oracle.localize_max_form(x, offs, C), brute)


@pytest.mark.parametrize("name", ["c1", "random"])
@pytest.mark.parametrize("seed", range(4))
def test_localized_mask_is_the_global_mask_on_the_rank_rows(name, seed):
    rng = np.random.default_rng(seed)
    w = (workloads.causal_doc(seed) if name == "c1" else
         workloads.random_intervals(seed, 512, batch=1))
    n = w.seqlen
    C = 64
    offs = _chunks(rng, n, C, int(rng.integers(1, n // C)))
    rows = oracle.rank_rows(offs, C)
    glob = oracle.masked_rows(*(x[0] for x in w.vectors()), 0, n)
    loc_vec = oracle.localize_vectors([x[:1] for x in w.vectors()], offs, C)
    loc = oracle.masked_rows(*(x[0] for x in loc_vec), 0, len(rows))
    assert np.array_equal(loc, glob[rows])


def test_rank_attention_equals_global_rows():
    """Attention of a rank's rows against all keys with localized vectors equals the
    global attention at those rows (float64, up to summation order)."""
    rng = np.random.default_rng(3)
    w = workloads.prefix_lm_doc(1, n=512, batch=1, heads_q=2, heads_kv=1, lo=64, hi=200)
    q, k, v, do = (t.double().numpy() for t in workloads.make_tensors(w))
    C = 32
    offs = _chunks(rng, 512, C, 5)
    rows = oracle.rank_rows(offs, C)
    O, L, dQ, dK, dV = oracle.attention_fwd_bwd(q, k, v, do, *w.vectors())
    lv = oracle.localize_vectors(w.vectors(), offs, C)
    Ol, Ll, dQl, dKl, dVl = oracle.attention_fwd_bwd(q[:, :, rows], k, v, do[:, :, rows], *lv)
    assert np.allclose(Ol, O[:, :, rows], atol=1e-12)
    fin = np.isfinite(L[:, :, rows])
    assert np.array_equal(fin, np.isfinite(Ll))
    assert np.allclose(Ll[fin], L[:, :, rows][fin], atol=1e-12)
    assert np.allclose(dQl, dQ[:, :, rows], atol=1e-12)
    # the rank's dK/dV are its rows' share; the other ranks add the rest
    rest = np.setdiff1d(np.arange(512), rows)
    offs_rest = sorted(set(range(0, 512, C)) - set(offs))
    lr = oracle.localize_vectors(w.vectors(), offs_rest, C)
    _, _, _, dKr, dVr = oracle.attention_fwd_bwd(q[:, :, rest], k, v, do[:, :, rest], *lr)
    assert np.allclose(dKl + dKr, dK, atol=1e-10)
    assert np.allclose(dVl + dVr, dV, atol=1e-10)


@pytest.mark.parametrize("seed", range(6))
def test_rule_sound_on_localized_vectors(seed):
    """The tile rule on N_q local rows x N_k keys: a skipped tile is fully hidden and an
    unmasked tile has nothing hidden (brute force over the dense local mask)."""
    from oracle import tiles
    rng = np.random.default_rng(seed)
    w = workloads.random_intervals(seed, 640, batch=2)
    C = 32
    offs = _chunks(rng, 640, C, 7)
    lv = oracle.localize_vectors(w.vectors(), offs, C)
    nq = 7 * C
    for bq, bk in ((32, 64), (64, 32), (16, 128)):
        cls = tiles.classify(*lv, bq, bk, nq=nq)
        truth = tiles.tile_truth(*lv, bq, bk, nq=nq)
        assert cls.shape == (2, -(-nq // bq), -(-640 // bk))
        assert ((cls == tiles.SKIP) <= (truth == tiles.SKIP)).all()
        assert ((cls == tiles.UNMASKED) <= (truth == tiles.UNMASKED)).all()
