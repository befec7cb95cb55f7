"""Head dimension 256 on the GPU: the kernels built for d = 256 (one workgroup per CU) against
the fp64 oracle (masked attention is defined for any d; the softmax scale defaults to
1/sqrt(256)), across mask forms, head layouts, ragged lengths and a query share, plus
sampled rows and key columns of the d = 256 benchmark workload."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import (GRAD_TOL, LSE_TOL, O_TOL, check_fwd, check_grads, gpu_inputs, log, rel_l2,
                    to_np)

pytestmark = pytest.mark.gpu

D = 256
CASES = {
    "causal_doc_1k": lambda: workloads.causal_doc(0),
    "random_intervals_gqa_ragged": lambda: workloads.random_intervals(3, 700, batch=2, heads_q=4,
                                                                      heads_kv=2, p_empty=0.3),
    "sliding_window_sinks_mqa6": lambda: workloads.sliding_window_sinks(n=2048, heads_q=6,
                                                                        heads_kv=1, window=200,
                                                                        sinks=16),
    "per_head_sets_g2": lambda: workloads.random_intervals(4, 384, batch=2, heads_q=4, heads_kv=2,
                                                           mask_heads=4),
    "prefix_lm_doc_2k_g8": lambda: workloads.prefix_lm_doc(1, n=2048, batch=1, heads_q=8,
                                                           heads_kv=1, lo=256, hi=1024),
}


@pytest.mark.parametrize("name", list(CASES))
def test_d256_matches_oracle(name):
    import mask_aware_sparse_amd as fm
    w = workloads.with_head_dim(CASES[name](), D)
    log(f"d256 {name}: B={w.batch} Hq={w.heads_q} Hkv={w.heads_kv} N={w.seqlen}")
    q, k, v, do, vec = gpu_inputs(w)
    assert q.shape[-1] == D
    O, L = fm.attn_fwd(q, k, v, *vec)
    dq, dk, dv = fm.attn_bwd(q, k, v, O, L, do, *vec)
    torch.cuda.synchronize()
    ref = oracle.attention_fwd_bwd(*(to_np(x) for x in (q, k, v, do)), *w.vectors())
    check_fwd(O, L, ref[0], ref[1], ctx=name)
    check_grads(dq, dk, dv, ref[2:], ref[1], ctx=name)


def test_d256_multi_interval():
    import mask_aware_sparse_amd as fm
    w = workloads.with_head_dim(
        workloads.random_multi_intervals(0, 500, batch=2, heads_q=4, heads_kv=1, n_intervals=4),
        D)
    log("d256 multi-interval N=500 M=4")
    q, k, v, do = workloads.make_tensors(w, device="cuda")
    s, e = workloads.mask_tensors(w, device="cuda")
    O, L = fm.attn_fwd_multi(q, k, v, s, e)
    dq, dk, dv = fm.attn_bwd_multi(q, k, v, O, L, do, s, e)
    torch.cuda.synchronize()
    ref = oracle.attention_fwd_bwd_multi(*(to_np(x) for x in (q, k, v, do)), w.starts, w.ends)
    check_fwd(O, L, ref[0], ref[1], ctx="multi")
    check_grads(dq, dk, dv, ref[2:], ref[1], ctx="multi")


def test_d256_block_sparse():
    import mask_aware_sparse_amd as fm
    w = workloads.with_head_dim(
        workloads.random_blocks(2, 700, batch=2, heads_q=4, heads_kv=2, density=0.4), D)
    log("d256 block-sparse N=700")
    q, k, v, do = workloads.make_tensors(w, device="cuda")
    (blk,) = workloads.mask_tensors(w, device="cuda")
    O, L = fm.attn_fwd_blocks(q, k, v, blk)
    dq, dk, dv = fm.attn_bwd_blocks(q, k, v, O, L, do, blk)
    torch.cuda.synchronize()
    ref = oracle.attention_fwd_bwd_blocks(*(to_np(x) for x in (q, k, v, do)), w.blocks)
    check_fwd(O, L, ref[0], ref[1], ctx="blocks")
    check_grads(dq, dk, dv, ref[2:], ref[1], ctx="blocks")


def test_d256_rank_share_reproduces_global_rows():
    """One context-parallel rank's share (its query chunks against every key, the vectors
    localized) gives the global run's O, LSE and dQ rows bit for bit."""
    import mask_aware_sparse_amd as fm
    n, C = 1024, 64
    w = workloads.with_head_dim(workloads.random_intervals(7, n, batch=1, heads_q=2), D)
    q, k, v, do, vec = gpu_inputs(w)
    offs = [64, 320, 512, 960]
    loc = fm.localize_mask(*vec, torch.tensor(offs, dtype=torch.int32, device="cuda"), C)
    O, L = fm.attn_fwd(q, k, v, *vec)
    dq, _, _ = fm.attn_bwd(q, k, v, O, L, do, *vec)
    rows = torch.from_numpy(oracle.rank_rows(offs, C)).cuda()
    qr, dor = q[:, :, rows].contiguous(), do[:, :, rows].contiguous()
    Or, Lr = fm.attn_fwd(qr, k, v, *loc)
    dqr, _, _ = fm.attn_bwd(qr, k, v, Or, Lr, dor, *loc)
    torch.cuda.synchronize()
    assert torch.equal(Or, O[:, :, rows]) and torch.equal(Lr, L[:, :, rows])
    assert torch.equal(dqr, dq[:, :, rows])


def test_full_size_d256_sampled():
    """The d = 256 benchmark workload (prefix-LM documents, B = 4, 32 query heads, 8 kv heads,
    N = 8192) in the launch configuration the benchmark times: sampled rows of two heads and
    sampled key columns of one kv head against the oracle."""
    import mask_aware_sparse_amd as fm
    w = workloads.make_workload("v5_prefix_lm_doc_8k_d256")
    log(f"full-size d256: B={w.batch} Hq={w.heads_q} Hkv={w.heads_kv} N={w.seqlen}")
    q, k, v, do, vec = gpu_inputs(w)
    O, L = fm.attn_fwd(q, k, v, *vec)
    dq, dk, dv = fm.attn_bwd(q, k, v, O, L, do, *vec)
    torch.cuda.synchronize()
    g = w.heads_q // w.heads_kv
    n = w.seqlen
    rng = np.random.default_rng(9)
    rows = sorted({0, 1, 127, 128, n - 1} | set(rng.integers(0, n, 5).tolist()))
    sub = lambda t, b, hh: to_np(t[b:b + 1, hh:hh + 1])
    vb = lambda b: [x[b:b + 1] for x in w.vectors()]
    for b, h in ((0, 0), (3, w.heads_q - 1)):
        kvh = h // g
        Or, Lr, dQr = oracle.attention_rows(sub(q, b, h), sub(k, b, kvh), sub(v, b, kvh),
                                            sub(do, b, h), *vb(b), 0, 0, rows)
        assert np.abs(to_np(O[b, h, rows]) - Or).max() <= O_TOL, (b, h)
        assert np.abs(to_np(L[b, h, rows]) - Lr).max() <= LSE_TOL, (b, h)
        assert rel_l2(to_np(dq[b, h, rows]), dQr) <= GRAD_TOL, (b, h)
    cols = [n - 300, n - 129, n - 1]
    kvh = 3
    grp = slice(kvh * g, (kvh + 1) * g)
    dKr, dVr = oracle.attention_cols(to_np(q[:1, grp]), to_np(k[:1, kvh:kvh + 1]),
                                     to_np(v[:1, kvh:kvh + 1]), to_np(do[:1, grp]),
                                     *vb(0), 0, 0, cols)
    assert rel_l2(to_np(dk[0, kvh, cols]), dKr) <= GRAD_TOL
    assert rel_l2(to_np(dv[0, kvh, cols]), dVr) <= GRAD_TOL
