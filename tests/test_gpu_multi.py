"""Multi-interval column masks (up to 4 active row intervals per key column) on the GPU.

The kernels against the fp64 oracle for 1 to 4 intervals under several head layouts
(GQA, a group of 6 summed over two work items, per-head sets) with ragged lengths; the
classification, block min/max and dense expansion bit-exact against the oracle; masks
both forms can write give bit-identical results through either entry point; mask
localization and one rank's share (Theorem 1); and the variant's full-size workload on
sampled rows and columns."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import (GRAD_TOL, LSE_TOL, O_TOL, check_fwd, check_grads, log, rel_l2, to_np)

pytestmark = pytest.mark.gpu

# name: (M, H_q, H_kv, H_m (0 = shared), N)
CASES = {
    "one_interval_gqa": (1, 4, 2, 0, 320),
    "two_intervals_mqa6": (2, 6, 1, 0, 256),
    "three_intervals_ragged": (3, 2, 1, 0, 200),
    "four_intervals_gqa": (4, 8, 2, 0, 448),
    "four_intervals_per_head": (4, 4, 2, 4, 384),
}


def _inputs(w, device="cuda"):
    q, k, v, do = workloads.make_tensors(w, device=device)
    s, e = workloads.mask_tensors(w, device=device)
    return q, k, v, do, s, e


@pytest.mark.parametrize("name", list(CASES))
def test_multi_matches_oracle(name):
    import mask_aware_sparse_amd as fm
    M, hq, hkv, hm, n = CASES[name]
    w = workloads.random_multi_intervals(list(CASES).index(name), n, batch=2, heads_q=hq,
                                         heads_kv=hkv, n_intervals=M, mask_heads=hm,
                                         p_empty=0.25)
    log(f"multi {name}: M={M} Hq={hq} Hkv={hkv} Hm={hm} N={n}")
    q, k, v, do, s, e = _inputs(w)
    O, L = fm.attn_fwd_multi(q, k, v, s, e)
    dq, dk, dv = fm.attn_bwd_multi(q, k, v, O, L, do, s, e)
    torch.cuda.synchronize()
    ref = oracle.attention_fwd_bwd_multi(*(to_np(x) for x in (q, k, v, do)), w.starts, w.ends)
    check_fwd(O, L, ref[0], ref[1], ctx=name)
    check_grads(dq, dk, dv, ref[2:], ref[1], ctx=name)


@pytest.mark.parametrize("bq,bk", [(128, 64), (32, 128), (64, 64), (16, 256)])
@pytest.mark.parametrize("M", [1, 3, 4])
def test_multi_classification_matches_oracle(bq, bk, M):
    import mask_aware_sparse_amd as fm
    w = workloads.random_multi_intervals(M, 1000, batch=2, n_intervals=M, mask_heads=2)
    s, e = workloads.mask_tensors(w, device="cuda")
    out = fm.classify_tiles_multi(s, e, bq, bk)
    torch.cuda.synchronize()
    flat_s = w.starts.reshape(-1, M, w.seqlen)
    flat_e = w.ends.reshape(-1, M, w.seqlen)
    assert np.array_equal(out["block_minmax"].cpu().numpy(),
                          oracle.block_minmax_multi(flat_s, flat_e, bk))
    cls = oracle.classify_multi(flat_s, flat_e, bq, bk)
    qq, qc, kq, kc = oracle.queues(cls)
    assert np.array_equal(out["tile_class"].cpu().numpy(), cls)
    assert np.array_equal(out["q_queue"].cpu().numpy(), qq)
    assert np.array_equal(out["q_count"].cpu().numpy(), qc)
    assert np.array_equal(out["k_queue"].cpu().numpy(), kq)
    assert np.array_equal(out["k_count"].cpu().numpy(), kc)
    assert np.array_equal(out["q_order"].cpu().numpy(), oracle.lpt_order(oracle.tile_costs(qc)))
    assert np.array_equal(out["k_order"].cpu().numpy(), oracle.lpt_order(oracle.tile_costs(kc)))


def test_multi_classification_many_tiles():
    """Many tiles (2 x 256 x 256, every classification workgroup walking 256 blocks in
    chunks): bit-exact as well."""
    import mask_aware_sparse_amd as fm
    w = workloads.random_multi_intervals(12, 8192, batch=2, n_intervals=3)
    s, e = workloads.mask_tensors(w, device="cuda")
    out = fm.classify_tiles_multi(s, e, 32, 32)
    torch.cuda.synchronize()
    cls = oracle.classify_multi(w.starts, w.ends, 32, 32)
    qq, qc, kq, kc = oracle.queues(cls)
    assert np.array_equal(out["block_minmax"].cpu().numpy(),
                          oracle.block_minmax_multi(w.starts, w.ends, 32))
    assert np.array_equal(out["tile_class"].cpu().numpy(), cls)
    assert np.array_equal(out["q_queue"].cpu().numpy(), qq)
    assert np.array_equal(out["k_queue"].cpu().numpy(), kq)
    assert np.array_equal(out["q_order"].cpu().numpy(), oracle.lpt_order(oracle.tile_costs(qc)))
    assert np.array_equal(out["k_order"].cpu().numpy(), oracle.lpt_order(oracle.tile_costs(kc)))


@pytest.mark.parametrize("n,bq,bk", [(1499 * 16 - 5, 16, 128), (5555 * 16 - 7, 16, 256)])
def test_multi_classification_long_lists(n, bq, bk):
    """More than 4096 / 16384 queue rows (2 / 8 Q-blocks per classification workgroup, a
    Q-block count neither divides): bit-exact."""
    import mask_aware_sparse_amd as fm
    w = workloads.random_multi_intervals(31, n, batch=3, n_intervals=3)
    s, e = workloads.mask_tensors(w, device="cuda")
    out = fm.classify_tiles_multi(s, e, bq, bk)
    torch.cuda.synchronize()
    cls = oracle.classify_multi(w.starts, w.ends, bq, bk)
    qq, qc, kq, kc = oracle.queues(cls)
    assert np.array_equal(out["block_minmax"].cpu().numpy(),
                          oracle.block_minmax_multi(w.starts, w.ends, bk))
    assert np.array_equal(out["tile_class"].cpu().numpy(), cls)
    assert np.array_equal(out["q_queue"].cpu().numpy(), qq)
    assert np.array_equal(out["q_count"].cpu().numpy(), qc)
    assert np.array_equal(out["k_queue"].cpu().numpy(), kq)
    assert np.array_equal(out["q_order"].cpu().numpy(), oracle.lpt_order(oracle.tile_costs(qc)))
    assert np.array_equal(out["k_order"].cpu().numpy(), oracle.lpt_order(oracle.tile_costs(kc)))


def test_multi_dense_expansion():
    import mask_aware_sparse_amd as fm
    w = workloads.random_multi_intervals(11, 300, batch=2, n_intervals=4)
    s, e = workloads.mask_tensors(w, device="cuda")
    for b in range(2):
        got = fm.debug_expand_mask_multi(s, e, b, 0, 300).cpu().numpy().astype(bool)
        assert np.array_equal(got, oracle.dense_mask_multi(w.starts[b], w.ends[b]))
    got = fm.debug_expand_mask_multi(s, e, 1, 37, 101).cpu().numpy().astype(bool)
    assert np.array_equal(got, oracle.dense_mask_multi(w.starts[1], w.ends[1])[37:101])


def _four_vector_twin(n, B, seed):
    """Masks both forms can write: one visible interval [s, e) (= hidden [e, N) and
    [0, s)), and two visible intervals around a gap [a, b) (= hidden [a, b))."""
    rng = np.random.default_rng(seed)
    s = rng.integers(0, n + 1, (B, n)); e = rng.integers(0, n + 1, (B, n))
    s, e = np.minimum(s, e), np.maximum(s, e)
    one = ((s[:, None], e[:, None]), (e, np.full_like(e, n), np.zeros_like(s), s))
    a = np.sort(rng.integers(0, n + 1, (2, B, n)), axis=0)
    two = ((np.stack([np.zeros_like(a[0]), a[1]], 1), np.stack([a[0], np.full_like(a[0], n)], 1)),
           (a[0], a[1], np.zeros_like(a[0]), np.zeros_like(a[0])))
    return [one, two]


@pytest.mark.parametrize("hq,hkv", [(2, 1), (6, 1)])
def test_forms_agree_bit_for_bit(hq, hkv):
    """Same mask through both entry points: bit-identical, except dK/dV of a group above 4
    heads, which fp32 atomics sum in arrival order (then within the gradient tolerance)."""
    import mask_aware_sparse_amd as fm
    n, B = 384, 2
    w = workloads.causal(n, batch=B, heads_q=hq, heads_kv=hkv)
    q, k, v, do = workloads.make_tensors(w, device="cuda")
    cu = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
    for (se, four) in _four_vector_twin(n, B, 5):
        s, e = cu(se[0]), cu(se[1])
        vec = [cu(x) for x in four]
        a = fm.attn_fwd_multi(q, k, v, s, e)
        b = fm.attn_fwd(q, k, v, *vec)
        ga = fm.attn_bwd_multi(q, k, v, *a, do, s, e)
        gb = fm.attn_bwd(q, k, v, *b, do, *vec)
        torch.cuda.synchronize()
        for x, y in zip(a + ga[:1], b + gb[:1]):
            assert torch.equal(x, y)
        for x, y in zip(ga[1:], gb[1:]):
            if hq // hkv <= 4:
                assert torch.equal(x, y)
            else:
                assert rel_l2(to_np(x), to_np(y)) <= 1e-3


def test_multi_localize_and_rank_share():
    """Localized intervals (bit-exact against the oracle) and Theorem 1: a rank's O, LSE
    and dQ equal the global run's rows bit for bit."""
    import mask_aware_sparse_amd as fm
    n, C = 1024, 64
    w = workloads.random_multi_intervals(21, n, batch=1, heads_q=2, n_intervals=3)
    q, k, v, do, s, e = _inputs(w)
    offs = [64, 320, 512, 960]
    ls, le = fm.localize_mask_multi(s, e, torch.tensor(offs, dtype=torch.int32, device="cuda"), C)
    torch.cuda.synchronize()
    assert np.array_equal(ls.cpu().numpy(), oracle.localize(w.starts, offs, C))
    assert np.array_equal(le.cpu().numpy(), oracle.localize(w.ends, offs, C))
    O, L = fm.attn_fwd_multi(q, k, v, s, e)
    dq, _, _ = fm.attn_bwd_multi(q, k, v, O, L, do, s, e)
    rows = torch.from_numpy(oracle.rank_rows(offs, C)).cuda()
    qr, dor = q[:, :, rows].contiguous(), do[:, :, rows].contiguous()
    Or, Lr = fm.attn_fwd_multi(qr, k, v, ls, le)
    dqr, _, _ = fm.attn_bwd_multi(qr, k, v, Or, Lr, dor, ls, le)
    torch.cuda.synchronize()
    assert torch.equal(Or, O[:, :, rows]) and torch.equal(Lr, L[:, :, rows])
    assert torch.equal(dqr, dq[:, :, rows])


def test_full_size_variant_sampled():
    """The variant's benchmark workload (window + three random distant query blocks per
    key block, N = 32K, 32 query heads, 8 kv heads) in the launch configuration the
    benchmark times: sampled rows against the oracle, and dK/dV of sampled key columns."""
    import mask_aware_sparse_amd as fm
    w = workloads.make_workload("v2_block_sparse_window_32k")
    log(f"full-size multi-interval: Hq={w.heads_q} Hkv={w.heads_kv} M={w.n_intervals} "
        f"N={w.seqlen}")
    q, k, v, do, s, e = _inputs(w)
    O, L = fm.attn_fwd_multi(q, k, v, s, e)
    dq, dk, dv = fm.attn_bwd_multi(q, k, v, O, L, do, s, e)
    torch.cuda.synchronize()
    g = w.heads_q // w.heads_kv
    n = w.seqlen
    rng = np.random.default_rng(4)
    rows = sorted({0, 1, 2047, 2048, n - 1} | set(rng.integers(0, n, 6).tolist()))
    sub = lambda t, hh: to_np(t[:1, hh:hh + 1])
    for h in (0, 13, w.heads_q - 1):
        kvh = h // g
        Or, Lr, dQr = oracle.attention_rows_multi(sub(q, h), sub(k, kvh), sub(v, kvh),
                                                  sub(do, h), w.starts, w.ends, 0, 0, rows)
        assert np.abs(to_np(O[0, h, rows]) - Or).max() <= O_TOL, h
        assert np.abs(to_np(L[0, h, rows]) - Lr).max() <= LSE_TOL, h
        assert rel_l2(to_np(dq[0, h, rows]), dQr) <= GRAD_TOL, h
    # columns of the last key blocks: seen by their window's rows only (no distant block
    # lies past them), so few rows need recomputing
    cols = [n - 200, n - 129, n - 1]
    kvh = w.heads_kv - 1
    grp = slice(kvh * g, (kvh + 1) * g)
    dKr, dVr = oracle.attention_cols_multi(to_np(q[:1, grp]), to_np(k[:1, kvh:kvh + 1]),
                                           to_np(v[:1, kvh:kvh + 1]), to_np(do[:1, grp]),
                                           w.starts, w.ends, 0, 0, cols)
    assert rel_l2(to_np(dk[0, kvh, cols]), dKr) <= GRAD_TOL
    assert rel_l2(to_np(dv[0, kvh, cols]), dVr) <= GRAD_TOL
