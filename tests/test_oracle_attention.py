"""Pins for the oracle's masked attention forward/backward (CPU only).

The oracle is numpy float64; the pins use torch (CPU, float64) as an independent
library: scaled_dot_product_attention for the special cases, and autograd through a
separately written dense-mask attention for the general case."""
import numpy as np
import pytest
import torch

import oracle
import workloads


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def torch_dense(q, k, v, hidden, scale):
    """Independent dense-mask attention in torch float64 (autograd-capable); `hidden` is
    [B][N_q][N_k] (every head) or [B][H_q][N_q][N_k] (per head)."""
    g = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(g, dim=1)
    v = v.repeat_interleave(g, dim=1)
    s = scale * q @ k.transpose(-1, -2)
    s = s.masked_fill(hidden if hidden.dim() == 4 else hidden[:, None], float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    p = torch.softmax(s, dim=-1)
    return p @ v, lse


def hidden_of(w):
    return torch.from_numpy(np.stack([oracle.dense_mask(*(x[b] for x in w.vectors()))
                                      for b in range(w.batch)]))


@pytest.mark.parametrize("n,d", [(16, 8), (40, 16), (130, 32)])
def test_no_mask_and_causal_vs_sdpa(n, d):
    q, k, v = (rand((2, 3, n, d), s) for s in (1, 2, 3))
    B = 2
    none = [np.full((B, n), n), np.full((B, n), n), np.zeros((B, n)), np.zeros((B, n))]
    O, _ = oracle.attention_fwd(q, k, v, *none)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)))
    assert np.abs(O - ref.numpy()).max() < 1e-12
    causal = [np.full((B, n), n), np.full((B, n), n), np.zeros((B, n)),
              np.tile(np.arange(n), (B, 1))]
    O, _ = oracle.attention_fwd(q, k, v, *causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)), is_causal=True)
    assert np.abs(O - ref.numpy()).max() < 1e-12


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (3, 1)])
def test_fwd_bwd_vs_autograd(seed, hq, hkv):
    n, d = 48, 16
    w = workloads.random_intervals(seed, n, batch=2, p_empty=0.3)
    hid = hidden_of(w)
    rows_dead = hid.all(dim=-1)
    live = ~rows_dead
    q, k, v, do = (rand(s, seed * 10 + t) for t, s in
                   enumerate([(2, hq, n, d), (2, hkv, n, d), (2, hkv, n, d), (2, hq, n, d)]))
    scale = 1 / np.sqrt(d)
    O, LSE, dQ, dK, dV = oracle.attention_fwd_bwd(q, k, v, do, *w.vectors())
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    # all-hidden rows: exclude them from torch (softmax of all -inf is nan there)
    hid_t = hid.clone()
    hid_t[rows_dead] = False
    To, Tl = torch_dense(tq, tk, tv, hid_t, scale)
    sel = live[:, None, :, None].expand_as(To).to(torch.float64)
    (To * torch.from_numpy(do) * sel).sum().backward()
    L = live[:, None, :].expand(2, hq, n).numpy()
    assert np.abs(O[L] - To.detach().numpy()[L]).max() < 1e-12
    assert np.abs(LSE[L] - Tl.detach().numpy()[L]).max() < 1e-12
    assert np.abs(dQ[L] - tq.grad.numpy()[L]).max() < 1e-11
    assert np.abs(dK - tk.grad.numpy()).max() < 1e-11
    assert np.abs(dV - tv.grad.numpy()).max() < 1e-11
    # all-hidden rows: O = 0, LSE = -inf, dQ = 0 (the stated convention)
    D = ~L
    assert (O[D] == 0).all() and np.isneginf(LSE[D]).all() and (dQ[D] == 0).all()


def test_bwd_finite_differences():
    # d/dX of L = sum(O * dO) by central differences, independent of any formula
    n, d = 12, 4
    w = workloads.random_intervals(7, n, p_empty=0.1)
    q, k, v, do = (rand(s, t) for t, s in enumerate([(1, 2, n, d), (1, 1, n, d),
                                                     (1, 1, n, d), (1, 2, n, d)]))
    _, _, dQ, dK, dV = oracle.attention_fwd_bwd(q, k, v, do, *w.vectors())
    eps = 1e-6

    def loss(q_, k_, v_):
        O, _ = oracle.attention_fwd(q_, k_, v_, *w.vectors())
        return (O * do).sum()

    rng = np.random.default_rng(0)
    for X, G, which in ((q, dQ, 0), (k, dK, 1), (v, dV, 2)):
        for _ in range(12):
            idx = tuple(rng.integers(0, s) for s in X.shape)
            Xp = X.copy(); Xp[idx] += eps
            Xm = X.copy(); Xm[idx] -= eps
            args_p = [q, k, v]; args_p[which] = Xp
            args_m = [q, k, v]; args_m[which] = Xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - G[idx]) < 1e-6 * max(1.0, abs(fd))


def test_single_visible_key_rows_exact():
    # a row that sees exactly one key j: O_i = V_j and LSE_i = scale * q_i . k_j
    w = workloads.causal_doc(0)
    n, d = w.seqlen, 128
    q, k, v = (rand(s, t) for t, s in enumerate([(1, 1, n, d)] * 3))
    starts = np.r_[0, np.cumsum(w.info["doc_lengths"][0])[:-1]]
    O, LSE, _ = oracle.attention_rows(q, k, v, None, *w.vectors(), 0, 0, starts)
    for t, s in enumerate(starts):
        assert (O[t] == v[0, 0, s]).all()
        assert abs(LSE[t] - (q[0, 0, s] @ k[0, 0, s]) / np.sqrt(d)) < 1e-12


def test_gqa_equals_repeated_heads():
    n, d = 64, 16
    w = workloads.random_intervals(3, n, batch=1)
    q, do = rand((1, 6, n, d), 1), rand((1, 6, n, d), 2)
    k, v = rand((1, 2, n, d), 3), rand((1, 2, n, d), 4)
    O, LSE, dQ, dK, dV = oracle.attention_fwd_bwd(q, k, v, do, *w.vectors())
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    O2, LSE2, dQ2, dK2, dV2 = oracle.attention_fwd_bwd(q, kr, vr, do, *w.vectors())
    assert np.abs(O - O2).max() < 1e-13 and np.abs(dQ - dQ2).max() < 1e-13
    assert np.array_equal(np.isneginf(LSE), np.isneginf(LSE2))
    assert np.abs(dK - dK2.reshape(1, 2, 3, n, d).sum(2)).max() < 1e-12
    assert np.abs(dV - dV2.reshape(1, 2, 3, n, d).sum(2)).max() < 1e-12


def test_key_permutation_invariance():
    n, d = 50, 8
    w = workloads.random_intervals(4, n, batch=1)
    q, k, v = rand((1, 1, n, d), 1), rand((1, 1, n, d), 2), rand((1, 1, n, d), 3)
    perm = np.random.default_rng(9).permutation(n)
    O, LSE = oracle.attention_fwd(q, k, v, *w.vectors())
    Op, LSEp = oracle.attention_fwd(q, k[:, :, perm], v[:, :, perm],
                                    *(x[:, perm] for x in w.vectors()))
    fin = np.isfinite(LSE)
    assert np.abs(O - Op).max() < 1e-13
    assert np.abs(LSE[fin] - LSEp[fin]).max() < 1e-13
    assert np.array_equal(fin, np.isfinite(LSEp))


def test_gradient_sum_invariants():
    # sum_j dS_ij = 0 gives sum_j dK_j = 0; sum_j P_ij = 1 gives
    # sum_j dV_j = sum over live rows of dO
    n, d = 96, 16
    w = workloads.share_question(0, n=96, prompt_range=(8, 12), answer_range=(4, 8), heads_q=4)
    q, do = rand((1, 4, n, d), 1), rand((1, 4, n, d), 2)
    k, v = rand((1, 1, n, d), 3), rand((1, 1, n, d), 4)
    _, LSE, dQ, dK, dV = oracle.attention_fwd_bwd(q, k, v, do, *w.vectors())
    assert np.abs(dK.sum(axis=2)).max() < 1e-12
    live = np.isfinite(LSE)[..., None]
    assert np.abs(dV.sum(axis=2)[0, 0] - (do * live).sum(axis=(1, 2))[0]).max() < 1e-12
    assert (dQ[~np.isfinite(LSE)] == 0).all()


def test_dead_rows_add_nothing():
    n, d = 80, 8
    w = workloads.share_question(1, n=n, prompt_range=(3, 5), answer_range=(2, 4))
    q, k, v, do = (rand(s, t) for t, s in enumerate([(1, 1, n, d)] * 4))
    _, LSE, _, dK, dV = oracle.attention_fwd_bwd(q, k, v, do, *w.vectors())
    dead = ~np.isfinite(LSE[0, 0])
    assert dead.any()
    do2 = do.copy(); do2[0, 0, dead] = 1e3
    q2 = q.copy(); q2[0, 0, dead] = -7.0
    _, _, _, dK2, dV2 = oracle.attention_fwd_bwd(q2, k, v, do2, *w.vectors())
    assert np.array_equal(dK, dK2) and np.array_equal(dV, dV2)


def test_rows_cols_and_block_size_consistent():
    n, d = 200, 16
    w = workloads.random_intervals(11, n, batch=2, heads_q=2, heads_kv=1)
    q, do = rand((2, 2, n, d), 1), rand((2, 2, n, d), 2)
    k, v = rand((2, 1, n, d), 3), rand((2, 1, n, d), 4)
    O, LSE, dQ, dK, dV = oracle.attention_fwd_bwd(q, k, v, do, *w.vectors())
    O7, LSE7, dQ7, dK7, dV7 = oracle.attention_fwd_bwd(q, k, v, do, *w.vectors(), row_block=7)
    assert np.abs(O - O7).max() < 1e-13 and np.abs(dK - dK7).max() < 1e-12
    rows = [0, 5, 77, 199]
    Or, Lr, dQr = oracle.attention_rows(q, k, v, do, *w.vectors(), 1, 1, rows)
    assert np.abs(Or - O[1, 1, rows]).max() < 1e-13
    assert np.abs(dQr - dQ[1, 1, rows]).max() < 1e-13
    cols = [3, 100, 150, 199]
    dKc, dVc = oracle.attention_cols(q, k, v, do, *w.vectors(), 1, 0, cols, row_block=32)
    assert np.abs(dKc - dK[1, 0, cols]).max() < 1e-12
    assert np.abs(dVc - dV[1, 0, cols]).max() < 1e-12


# ---- per-head mask sets: vectors [B][H_m][N]; query head h uses set h // (H_q / H_m) ----

@pytest.mark.parametrize("hq,hkv,hm", [(4, 2, 4), (4, 2, 2), (4, 1, 2), (6, 3, 3), (2, 2, 1)])
def test_per_head_sets_vs_autograd(hq, hkv, hm):
    """Against autograd through dense attention whose [B][H][N][N] mask is expanded per
    head from the set the head's group uses (the mapping written out here, per head)."""
    n, d, B = 40, 16, 2
    w = workloads.random_intervals(7, n, batch=B, heads_q=hq, heads_kv=hkv, p_empty=0.3,
                                   mask_heads=hm)
    vecs = w.vectors()
    assert vecs[0].shape == (B, hm, n)
    per = hq // hm
    hid = torch.from_numpy(np.stack([np.stack([oracle.dense_mask(*(x[b, h // per] for x in vecs))
                                               for h in range(hq)]) for b in range(B)]))
    dead = hid.all(dim=-1)                                   # [B][H][N]
    q, k, v, do = (rand(s, 40 + t) for t, s in
                   enumerate([(B, hq, n, d), (B, hkv, n, d), (B, hkv, n, d), (B, hq, n, d)]))
    O, LSE, dQ, dK, dV = oracle.attention_fwd_bwd(q, k, v, do, *vecs)
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
    assert (O[~L] == 0).all() and np.isneginf(LSE[~L]).all()


def test_per_head_sets_that_agree_equal_the_shared_set():
    n, d = 64, 16
    w = workloads.random_intervals(3, n, batch=2, heads_q=4, heads_kv=2)
    q, do = rand((2, 4, n, d), 1), rand((2, 4, n, d), 2)
    k, v = rand((2, 2, n, d), 3), rand((2, 2, n, d), 4)
    shared = oracle.attention_fwd_bwd(q, k, v, do, *w.vectors())
    stacked = [np.repeat(x[:, None, :], 4, axis=1) for x in w.vectors()]
    per_head = oracle.attention_fwd_bwd(q, k, v, do, *stacked)
    for a, b in zip(shared, per_head):
        assert np.array_equal(a, b)


def test_per_head_rows_and_cols_consistent():
    n, d = 120, 16
    w = workloads.random_intervals(5, n, batch=1, heads_q=4, heads_kv=1, mask_heads=2)
    q, do = rand((1, 4, n, d), 1), rand((1, 4, n, d), 2)
    k, v = rand((1, 1, n, d), 3), rand((1, 1, n, d), 4)
    O, LSE, dQ, dK, dV = oracle.attention_fwd_bwd(q, k, v, do, *w.vectors())
    rows = [0, 31, 119]
    for h in range(4):
        Or, Lr, dQr = oracle.attention_rows(q, k, v, do, *w.vectors(), 0, h, rows)
        assert np.abs(Or - O[0, h, rows]).max() < 1e-13
        assert np.abs(dQr - dQ[0, h, rows]).max() < 1e-13
    cols = [0, 60, 119]
    dKc, dVc = oracle.attention_cols(q, k, v, do, *w.vectors(), 0, 0, cols, row_block=16)
    assert np.abs(dKc - dK[0, 0, cols]).max() < 1e-12
    assert np.abs(dVc - dV[0, 0, cols]).max() < 1e-12
