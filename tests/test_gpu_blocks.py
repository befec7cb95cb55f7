"""Block-sparse masks (128 x 128 blocks, each visible or hidden) on the GPU: the kernels
against the fp64 oracle across head layouts and ragged lengths, the classification against
the oracle's (bit-exact, including tiles that straddle blocks), the dense expansion, bit
identity with the four-vector form on block-diagonal documents, and sampled rows and key
columns of the BigBird-style benchmark workload."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import (GRAD_TOL, LSE_TOL, O_TOL, check_fwd, check_grads, log, rel_l2, to_np)

pytestmark = pytest.mark.gpu

# name: (N, H_q, H_kv, H_m (0 = one grid per batch row), density)
CASES = {
    "ragged_gqa": (700, 4, 2, 0, 0.4),
    "mqa6_sparse": (512, 6, 1, 0, 0.15),
    "per_head_grids": (384, 4, 2, 4, 0.5),
    "dense_blocks": (256, 2, 1, 0, 1.0),
}


def _inputs(w):
    q, k, v, do = workloads.make_tensors(w, device="cuda")
    (blk,) = workloads.mask_tensors(w, device="cuda")
    return q, k, v, do, blk


@pytest.mark.parametrize("name", list(CASES))
def test_blocks_match_oracle(name):
    import mask_aware_sparse_amd as fm
    n, hq, hkv, hm, dens = CASES[name]
    w = workloads.random_blocks(list(CASES).index(name), n, batch=2, heads_q=hq, heads_kv=hkv,
                                density=dens, mask_heads=hm)
    log(f"blocks {name}: N={n} Hq={hq} Hkv={hkv} Hm={hm} density={dens}")
    q, k, v, do, blk = _inputs(w)
    O, L = fm.attn_fwd_blocks(q, k, v, blk)
    dq, dk, dv = fm.attn_bwd_blocks(q, k, v, O, L, do, blk)
    torch.cuda.synchronize()
    ref = oracle.attention_fwd_bwd_blocks(*(to_np(x) for x in (q, k, v, do)), w.blocks)
    check_fwd(O, L, ref[0], ref[1], ctx=name)
    check_grads(dq, dk, dv, ref[2:], ref[1], ctx=name)


@pytest.mark.parametrize("bq,bk", [(128, 64), (32, 128), (256, 256), (64, 32)])
def test_blocks_classification(bq, bk):
    import mask_aware_sparse_amd as fm
    n = 900
    w = workloads.random_blocks(8, n, batch=2, density=0.4, mask_heads=2)
    (blk,) = workloads.mask_tensors(w, device="cuda")
    out = fm.classify_tiles_blocks(blk, bq, bk, n, n)
    torch.cuda.synchronize()
    flat = w.blocks.reshape(-1, *w.blocks.shape[-2:])
    cls = oracle.classify_blocks(flat, bq, bk, n, n)
    qq, qc, kq, kc = oracle.queues(cls)
    assert np.array_equal(out["tile_class"].cpu().numpy(), cls)
    assert np.array_equal(out["q_queue"].cpu().numpy(), qq)
    assert np.array_equal(out["q_count"].cpu().numpy(), qc)
    assert np.array_equal(out["k_queue"].cpu().numpy(), kq)
    assert np.array_equal(out["k_count"].cpu().numpy(), kc)
    assert np.array_equal(out["q_order"].cpu().numpy(), oracle.lpt_order(oracle.tile_costs(qc)))
    assert np.array_equal(out["k_order"].cpu().numpy(), oracle.lpt_order(oracle.tile_costs(kc)))


def test_blocks_classification_many_tiles():
    """Many tiles (2 x 256 x 256, every classification workgroup walking 256 blocks in
    chunks): bit-exact."""
    import mask_aware_sparse_amd as fm
    n = 8192
    w = workloads.random_blocks(13, n, batch=2, density=0.3)
    (blk,) = workloads.mask_tensors(w, device="cuda")
    out = fm.classify_tiles_blocks(blk, 32, 32, n, n)
    torch.cuda.synchronize()
    cls = oracle.classify_blocks(w.blocks, 32, 32, n, n)
    qq, qc, kq, kc = oracle.queues(cls)
    assert np.array_equal(out["tile_class"].cpu().numpy(), cls)
    assert np.array_equal(out["q_queue"].cpu().numpy(), qq)
    assert np.array_equal(out["k_queue"].cpu().numpy(), kq)
    assert np.array_equal(out["q_order"].cpu().numpy(), oracle.lpt_order(oracle.tile_costs(qc)))
    assert np.array_equal(out["k_order"].cpu().numpy(), oracle.lpt_order(oracle.tile_costs(kc)))


@pytest.mark.parametrize("batch,n,bq,bk", [(3, 1499 * 16 - 5, 16, 128), (5, 1999 * 16 - 3, 16, 256)])
def test_blocks_classification_long_lists(batch, n, bq, bk):
    """More than 4096 / 8192 queue rows (2 / 4 Q-blocks per classification workgroup, a
    Q-block count neither divides): bit-exact."""
    import mask_aware_sparse_amd as fm
    w = workloads.random_blocks(32, n, batch=batch, density=0.3)
    (blk,) = workloads.mask_tensors(w, device="cuda")
    out = fm.classify_tiles_blocks(blk, bq, bk, n, n)
    torch.cuda.synchronize()
    cls = oracle.classify_blocks(w.blocks, bq, bk, n, n)
    qq, qc, kq, kc = oracle.queues(cls)
    assert np.array_equal(out["tile_class"].cpu().numpy(), cls)
    assert np.array_equal(out["q_queue"].cpu().numpy(), qq)
    assert np.array_equal(out["q_count"].cpu().numpy(), qc)
    assert np.array_equal(out["k_queue"].cpu().numpy(), kq)
    assert np.array_equal(out["q_order"].cpu().numpy(), oracle.lpt_order(oracle.tile_costs(qc)))
    assert np.array_equal(out["k_order"].cpu().numpy(), oracle.lpt_order(oracle.tile_costs(kc)))


def test_blocks_dense_expansion():
    import mask_aware_sparse_amd as fm
    n = 450
    w = workloads.random_blocks(9, n, batch=2, density=0.5)
    (blk,) = workloads.mask_tensors(w, device="cuda")
    for b in range(2):
        got = fm.debug_expand_mask_blocks(blk, b, 0, n, n, n).cpu().numpy().astype(bool)
        assert np.array_equal(got, oracle.dense_mask_blocks(w.blocks[b], n, n))
    got = fm.debug_expand_mask_blocks(blk, 1, 100, 333, n, n).cpu().numpy().astype(bool)
    assert np.array_equal(got, oracle.dense_mask_blocks(w.blocks[1], n, n)[100:333])


def test_block_diagonal_equals_documents_bit_for_bit():
    """Documents of 128-aligned lengths: the block grid and the four vectors give the same
    tiles in the same order, so every output is bit-identical."""
    import mask_aware_sparse_amd as fm
    n, ends = 1024, [256, 384, 768, 1024]
    starts = [0] + ends[:-1]
    blk = np.zeros((1, 8, 8), dtype=np.uint8)
    for s0, e0 in zip(starts, ends):
        blk[0, s0 // 128:e0 // 128, s0 // 128:e0 // 128] = 1
    ds = np.array([s0 for s0, e0 in zip(starts, ends) for _ in range(e0 - s0)])
    de = np.array([e0 for s0, e0 in zip(starts, ends) for _ in range(e0 - s0)])
    four = [torch.from_numpy(x[None].astype(np.int32)).cuda()
            for x in (de, np.full(n, n), np.zeros(n), ds)]
    w = workloads.causal(n, heads_q=4, heads_kv=2)
    q, k, v, do = workloads.make_tensors(w, device="cuda")
    g = torch.from_numpy(blk).cuda()
    a = fm.attn_fwd_blocks(q, k, v, g)
    b = fm.attn_fwd(q, k, v, *four)
    ga = fm.attn_bwd_blocks(q, k, v, *a, do, g)
    gb = fm.attn_bwd(q, k, v, *b, do, *four)
    torch.cuda.synchronize()
    for x, y in zip(a + ga, b + gb):
        assert torch.equal(x, y)


def test_full_size_bigbird_sampled():
    """The block-sparse benchmark workload (N = 32K, 32 query heads, 8 kv heads) in the launch
    configuration the benchmark times: sampled rows (including a global row that sees every
    block) and key columns of the first and a middle block."""
    import mask_aware_sparse_amd as fm
    w = workloads.make_workload("v4_bigbird_blocks_32k")
    log(f"full-size block-sparse: Hq={w.heads_q} Hkv={w.heads_kv} N={w.seqlen}")
    q, k, v, do, blk = _inputs(w)
    O, L = fm.attn_fwd_blocks(q, k, v, blk)
    dq, dk, dv = fm.attn_bwd_blocks(q, k, v, O, L, do, blk)
    torch.cuda.synchronize()
    g = w.heads_q // w.heads_kv
    n = w.seqlen
    rng = np.random.default_rng(5)
    rows = sorted({0, 127, 128, n - 1} | set(rng.integers(0, n, 6).tolist()))
    sub = lambda t, hh: to_np(t[:1, hh:hh + 1])
    for h in (0, w.heads_q - 1):
        kvh = h // g
        Or, Lr, dQr = oracle.attention_rows_blocks(sub(q, h), sub(k, kvh), sub(v, kvh),
                                                   sub(do, h), w.blocks, 0, 0, rows)
        assert np.abs(to_np(O[0, h, rows]) - Or).max() <= O_TOL, h
        assert np.abs(to_np(L[0, h, rows]) - Lr).max() <= LSE_TOL, h
        assert rel_l2(to_np(dq[0, h, rows]), dQr) <= GRAD_TOL, h
    # a middle key block: seen by its window rows, the global row block and a few random rows
    cols = [16000, 16100]
    kvh = w.heads_kv - 1
    grp = slice(kvh * g, (kvh + 1) * g)
    dKr, dVr = oracle.attention_cols_blocks(to_np(q[:1, grp]), to_np(k[:1, kvh:kvh + 1]),
                                            to_np(v[:1, kvh:kvh + 1]), to_np(do[:1, grp]),
                                            w.blocks, 0, 0, cols)
    assert rel_l2(to_np(dk[0, kvh, cols]), dKr) <= GRAD_TOL
    assert rel_l2(to_np(dv[0, kvh, cols]), dVr) <= GRAD_TOL
