"""Pins for the oracle's dense-mask expansion and encoders (CPU only)."""
import os

import numpy as np
import pytest

import oracle
import workloads
from conftest import read_golden_pictures

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mask_pictures.txt")


def visible_from_fms_fme(fms, fme, n):
    vec = oracle.visible_interval_to_vectors(fms, fme, n)
    return ~oracle.dense_mask(*vec)


def test_printed_mask_pictures():
    pics = read_golden_pictures(GOLDEN)
    n = 8
    # causal panel: rows 0-5
    vis = visible_from_fms_fme(*oracle.encode_causal(n), n)
    assert (vis[0:6].astype(int) == np.array(pics["causal"]["rows"])).all()
    # document panel: both completions of the third document give the printed rows
    for docs in ([2, 2, 4], [2, 2, 2, 2]):
        vis = visible_from_fms_fme(*oracle.encode_packed(docs, causal=True), n)
        assert (vis[0:6].astype(int) == np.array(pics["document"]["rows"])).all()
    # DPO panel: rows 1-6 of prompt=2, chosen=3, rejected=3
    vis = visible_from_fms_fme(*oracle.encode_dpo(2, 3, 3), n)
    assert (vis[1:7].astype(int) == np.array(pics["dpo"]["rows"])).all()


def test_printed_pictures_reject_plausible_mistakes():
    pics = read_golden_pictures(GOLDEN)
    n = 8
    # an inclusive end on the upper interval (i <= UTE) would hide the diagonal
    fms, fme = oracle.encode_causal(n)
    lts, lte, uts, ute = oracle.visible_interval_to_vectors(fms, fme, n)
    i = np.arange(n)[:, None]
    wrong = ~(((lts <= i) & (i < lte)) | ((uts <= i) & (i <= ute)))
    assert not (wrong[0:6].astype(int) == np.array(pics["causal"]["rows"])).all()


@pytest.mark.parametrize("n", [1, 7, 33, 64])
def test_causal_closed_form(n):
    vis = visible_from_fms_fme(*oracle.encode_causal(n), n)
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    assert (vis == (j <= i)).all()


@pytest.mark.parametrize("docs", [[3, 5, 1, 7], [16], [1, 1, 1], [10, 22]])
def test_packed_closed_form(docs):
    n = sum(docs)
    seg = np.repeat(np.arange(len(docs)), docs)
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    vis = visible_from_fms_fme(*oracle.encode_packed(docs, causal=True), n)
    assert (vis == ((seg[i] == seg[j]) & (j <= i))).all()
    vis = visible_from_fms_fme(*oracle.encode_packed(docs, causal=False), n)
    # bidirectional form: FMS_j = doc start, FME_j = doc end
    assert (vis == (seg[i] == seg[j])).all()


@pytest.mark.parametrize("pcr", [(2, 3, 3), (5, 1, 4), (1, 6, 2)])
def test_dpo_closed_form(pcr):
    P, C, R = pcr
    n = P + C + R
    part = np.r_[np.zeros(P), np.ones(C), 2 * np.ones(R)].astype(int)
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    direct = (j <= i) & ((part[j] == 0) | (part[i] == part[j]))
    vis = visible_from_fms_fme(*oracle.encode_dpo(P, C, R), n)
    assert (vis == direct).all()


def interval_visible_count(lts, lte, uts, ute, n):
    """Visible rows per column by interval arithmetic (independent of the oracle)."""
    lts, lte, uts, ute = (np.asarray(x, dtype=np.int64) for x in (lts, lte, uts, ute))
    a1 = np.clip(lts, 0, n); b1 = np.clip(lte, 0, n)
    a2 = np.clip(uts, 0, n); b2 = np.clip(ute, 0, n)
    l1 = np.maximum(b1 - a1, 0); l2 = np.maximum(b2 - a2, 0)
    inter = np.maximum(np.minimum(b1, b2) - np.maximum(a1, a2), 0)
    inter = np.where((l1 > 0) & (l2 > 0), inter, 0)
    return n - (l1 + l2 - inter)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("n", [5, 64, 97])
def test_dense_count_matches_interval_arithmetic(seed, n):
    w = workloads.random_intervals(seed, n, batch=2)
    for b in range(2):
        vec = [x[b] for x in w.vectors()]
        vis = ~oracle.dense_mask(*vec)
        assert (vis.sum(axis=0) == interval_visible_count(*vec, n)).all()


def test_workload_families_direct_definitions():
    i_of = lambda n: np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    # c1 causal document at full size: visible iff same doc and j <= i
    w = workloads.causal_doc(0)
    n = w.seqlen
    seg = np.repeat(np.arange(4), w.info["doc_lengths"][0])
    i, j = i_of(n)
    vis = ~oracle.dense_mask(*(x[0] for x in w.vectors()))
    assert (vis == ((seg[i] == seg[j]) & (j <= i))).all()
    L = np.array(w.info["doc_lengths"][0])
    assert vis.sum() == (L * (L + 1) // 2).sum() == 181243
    # prefix-LM docs (smaller N): same doc and (j <= i or j in the doc's prefix)
    w = workloads.prefix_lm_doc(1, n=2048, lo=100, hi=600)
    for b in range(w.batch):
        lens = w.info["doc_lengths"][b]
        seg = np.repeat(np.arange(len(lens)), lens)
        starts = np.r_[0, np.cumsum(lens)[:-1]]
        pre = np.concatenate([np.arange(L) < L // 4 for L in lens])
        i, j = i_of(w.seqlen)
        direct = (seg[i] == seg[j]) & ((j <= i) | pre[j])
        vis = ~oracle.dense_mask(*(x[b] for x in w.vectors()))
        assert (vis == direct).all()
    # share-question (smaller N): prompt keys seen by their sample's rows at or
    # after them; answer keys seen causally inside their answer; padding hidden
    w = workloads.share_question(2, n=4096, prompt_range=(200, 400), answer_range=(100, 200))
    lay = w.info["layout"][0]
    n = w.seqlen
    sample = np.full(n, -1); part = np.full(n, -1)
    s = 0
    for k in range(4):
        sample[s:s + lay["prompts"][k]] = k; part[s:s + lay["prompts"][k]] = 0
        s += lay["prompts"][k]
        for a in range(3):
            sample[s:s + lay["answers"][k][a]] = k; part[s:s + lay["answers"][k][a]] = a + 1
            s += lay["answers"][k][a]
    assert s == lay["pad_start"]
    i, j = i_of(n)
    direct = (sample[j] >= 0) & (sample[i] == sample[j]) & (j <= i) & (
        (part[j] == 0) | (part[i] == part[j]))
    vis = ~oracle.dense_mask(*(x[0] for x in w.vectors()))
    assert (vis == direct).all()
    assert (~vis[lay["pad_start"]:]).all()       # padding rows see nothing
    # sliding window + sinks (smaller N, same closed form as at 128K)
    n, W, S = 8192, 1024, 64
    w = workloads.sliding_window_sinks(n=n, window=W, sinks=S)
    i, j = i_of(n)
    direct = (j <= i) & ((j < S) | (i - j < W))
    vis = ~oracle.dense_mask(*(x[0] for x in w.vectors()))
    assert (vis == direct).all()
    jj = np.arange(n)
    closed = (n - jj[:S]).sum() + np.minimum(W, n - jj[S:]).sum()
    assert vis.sum() == closed


def test_sliding_window_full_size_closed_form():
    # attended pairs per head at N=131072, W=4096, 64 sinks (interval arithmetic
    # against the closed form sum_{j<64}(N-j) + sum_{j>=64} min(4096, N-j))
    w = workloads.sliding_window_sinks()
    n = w.seqlen
    cnt = interval_visible_count(*(x[0] for x in w.vectors()), n).sum()
    assert cnt == 536608800


def test_random_eviction_count_near_expectation():
    # E[A] = sum_j E[LTS_j - j] = sum_j (N-j+1)/2 = N(N+3)/4; the spread is
    # sqrt(sum_j ((N-j)^2-1)/12) ~ N^1.5/6
    w = workloads.random_eviction()
    n = w.seqlen
    A = interval_visible_count(*(x[0] for x in w.vectors()), n).sum()
    assert A == 4291726033
    sigma = np.sqrt((((n - np.arange(n)) ** 2 - 1) / 12.0).sum())
    assert abs(A - n * (n + 3) / 4) < 3 * sigma
