"""Pins for the oracle's block-sparse form (128 x 128 blocks, each visible or hidden), CPU
only: the dense expansion against a loop over the definition and against the four-vector
form on masks both can write; attention against autograd through a separately written
dense-mask attention in torch; the tile rule against brute force (exact)."""
import numpy as np
import pytest
import torch

import oracle
import workloads

B128 = 128


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_dense_expansion_matches_the_definition():
    w = workloads.random_blocks(1, 300, batch=1, density=0.4)
    blk = w.blocks[0]
    got = oracle.dense_mask_blocks(blk, 300, 300)
    for i in range(0, 300, 7):
        for j in range(0, 300, 5):
            assert got[i, j] == (blk[i // B128, j // B128] == 0)


def test_block_diagonal_equals_document_vectors():
    """Block-diagonal grids are document masks with 128-aligned documents: hidden rows of
    key j are [0, doc start) and [doc end, N), the four-vector form (UTS=0, UTE=start,
    LTS=end, LTE=N)."""
    n = 640
    ends = [256, 384, 640]
    blk = np.zeros((5, 5), dtype=np.uint8)
    starts = [0] + ends[:-1]
    for s0, e0 in zip(starts, ends):
        blk[s0 // B128:e0 // B128, s0 // B128:e0 // B128] = 1
    j = np.arange(n)
    ds = np.array([s0 for s0, e0 in zip(starts, ends) for _ in range(e0 - s0)])
    de = np.array([e0 for s0, e0 in zip(starts, ends) for _ in range(e0 - s0)])
    four = (de, np.full(n, n), np.zeros(n, dtype=np.int64), ds)
    assert np.array_equal(oracle.dense_mask_blocks(blk, n, n), oracle.dense_mask(*four))
    q, k, v, do = (rand((1, 2, n, 8), s) for s in range(4))
    got = oracle.attention_fwd_bwd_blocks(q, k[:, :1], v[:, :1], do, blk[None])
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


@pytest.mark.parametrize("hq,hkv,hm", [(2, 1, 0), (4, 2, 2), (4, 2, 4)])
def test_block_attention_vs_autograd(hq, hkv, hm):
    n, d, B = 300, 8, 2
    w = workloads.random_blocks(hm + 3, n, batch=B, heads_q=hq, heads_kv=hkv, density=0.5,
                                mask_heads=hm)
    per = hq // max(hm, 1)
    grid = (lambda b, h: w.blocks[b]) if hm == 0 else (lambda b, h: w.blocks[b, h // per])
    hid = torch.from_numpy(np.stack([np.stack([oracle.dense_mask_blocks(grid(b, h), n, n)
                                               for h in range(hq)]) for b in range(B)]))
    dead = hid.all(dim=-1)
    q, k, v, do = (rand(s, 90 + t) for t, s in
                   enumerate([(B, hq, n, d), (B, hkv, n, d), (B, hkv, n, d), (B, hq, n, d)]))
    O, LSE, dQ, dK, dV = oracle.attention_fwd_bwd_blocks(q, k, v, do, w.blocks)
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


@pytest.mark.parametrize("bq,bk", [(128, 64), (32, 128), (64, 64), (256, 256), (16, 32)])
def test_block_rule_is_exact(bq, bk):
    n = 700                                    # ragged last block row and column
    w = workloads.random_blocks(4, n, batch=2, density=0.4)
    cls = oracle.classify_blocks(w.blocks, bq, bk, n, n)
    assert np.array_equal(cls, oracle.tile_truth_blocks(w.blocks, bq, bk, n, n))
    if bq <= 128 and bk <= 128:                # tiles inside one block: never partial
        assert (cls == 1).sum() == 0


def test_rows_and_cols_consistent():
    n, d = 400, 8
    w = workloads.random_blocks(6, n, batch=1, heads_q=2, density=0.5)
    q, do = rand((1, 2, n, d), 1), rand((1, 2, n, d), 2)
    k, v = rand((1, 1, n, d), 3), rand((1, 1, n, d), 4)
    O, LSE, dQ, dK, dV = oracle.attention_fwd_bwd_blocks(q, k, v, do, w.blocks)
    rows = [0, 200, 399]
    Or, Lr, dQr = oracle.attention_rows_blocks(q, k, v, do, w.blocks, 0, 1, rows)
    assert np.abs(Or - O[0, 1, rows]).max() < 1e-13 and np.abs(dQr - dQ[0, 1, rows]).max() < 1e-13
    cols = [0, 250, 399]
    dKc, dVc = oracle.attention_cols_blocks(q, k, v, do, w.blocks, 0, 0, cols, row_block=32)
    assert np.abs(dKc - dK[0, 0, cols]).max() < 1e-12 and np.abs(dVc - dV[0, 0, cols]).max() < 1e-12
