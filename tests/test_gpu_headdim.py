"""Head dimension 64 on the GPU: the same kernels built for d = 64 against the fp64
oracle (masked attention is defined for any d; the softmax scale defaults to 1/sqrt(64)),
across mask forms, head layouts, ragged lengths and query shares, plus sampled rows of
the d = 64 benchmark workload."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import (GRAD_TOL, LSE_TOL, O_TOL, check_fwd, check_grads, gpu_inputs, log, rel_l2,
                    to_np)

pytestmark = pytest.mark.gpu

D = 64
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
def test_d64_matches_oracle(name):
    import mask_aware_sparse_amd as fm
    w = workloads.with_head_dim(CASES[name](), D)
    log(f"d64 {name}: B={w.batch} Hq={w.heads_q} Hkv={w.heads_kv} N={w.seqlen}")
    q, k, v, do, vec = gpu_inputs(w)
    assert q.shape[-1] == D
    O, L = fm.attn_fwd(q, k, v, *vec)
    dq, dk, dv = fm.attn_bwd(q, k, v, O, L, do, *vec)
    torch.cuda.synchronize()
    ref = oracle.attention_fwd_bwd(*(to_np(x) for x in (q, k, v, do)), *w.vectors())
    check_fwd(O, L, ref[0], ref[1], ctx=name)
    check_grads(dq, dk, dv, ref[2:], ref[1], ctx=name)


def test_d64_multi_interval():
    """Seed 0.  Over seeds 0-15 of this problem the largest O error is 4.4e-3 to 1.0e-2
    (1.0014e-2 for seed 5, on one of 256,000 elements: an output of 2.79 whose rounding to
    bf16 alone costs 5.6e-3); the same sweep at d = 128 reaches 8.6e-3.  The 1e-2 bound
    leaves little room for outputs above 2 in magnitude."""
    import mask_aware_sparse_amd as fm
    w = workloads.with_head_dim(
        workloads.random_multi_intervals(0, 500, batch=2, heads_q=4, heads_kv=1, n_intervals=4),
        D)
    q, k, v, do = workloads.make_tensors(w, device="cuda")
    s, e = workloads.mask_tensors(w, device="cuda")
    O, L = fm.attn_fwd_multi(q, k, v, s, e)
    dq, dk, dv = fm.attn_bwd_multi(q, k, v, O, L, do, s, e)
    torch.cuda.synchronize()
    ref = oracle.attention_fwd_bwd_multi(*(to_np(x) for x in (q, k, v, do)), w.starts, w.ends)
    check_fwd(O, L, ref[0], ref[1], ctx="d64 multi")
    check_grads(dq, dk, dv, ref[2:], ref[1], ctx="d64 multi")


def test_d64_rank_share_reproduces_global_rows():
    import mask_aware_sparse_amd as fm
    w = workloads.with_head_dim(workloads.random_intervals(6, 1024, batch=1, heads_q=2), D)
    q, k, v, do, vec = gpu_inputs(w)
    O, L = fm.attn_fwd(q, k, v, *vec)
    dq, _, _ = fm.attn_bwd(q, k, v, O, L, do, *vec)
    offs, C = [128, 512, 896], 128
    rows = torch.from_numpy(oracle.rank_rows(offs, C)).cuda()
    lv = fm.localize_mask(*vec, torch.tensor(offs, dtype=torch.int32, device="cuda"), C)
    qr, dor = q[:, :, rows].contiguous(), do[:, :, rows].contiguous()
    Or, Lr = fm.attn_fwd(qr, k, v, *lv)
    dqr, _, _ = fm.attn_bwd(qr, k, v, Or, Lr, dor, *lv)
    torch.cuda.synchronize()
    assert torch.equal(Or, O[:, :, rows]) and torch.equal(Lr, L[:, :, rows])
    assert torch.equal(dqr, dq[:, :, rows])


def test_d64_full_size_sampled():
    """The d = 64 benchmark workload (prefix-LM documents, B=4, 32/8 heads, N=8192) in the
    launch configuration the benchmark times: sampled rows against the oracle."""
    import mask_aware_sparse_amd as fm
    w = workloads.make_workload("v3_prefix_lm_doc_8k_d64")
    q, k, v, do, vec = gpu_inputs(w)
    O, L = fm.attn_fwd(q, k, v, *vec)
    dq, dk, dv = fm.attn_bwd(q, k, v, O, L, do, *vec)
    torch.cuda.synchronize()
    g = w.heads_q // w.heads_kv
    rng = np.random.default_rng(2)
    for b in (0, w.batch - 1):
        rows = sorted({0, w.seqlen - 1} | set(rng.integers(0, w.seqlen, 8).tolist()))
        vb = [x[b:b + 1] for x in w.vectors()]
        for h in (0, w.heads_q - 1):
            sub = lambda t, hh: to_np(t[b:b + 1, hh:hh + 1])
            Or, Lr, dQr = oracle.attention_rows(sub(q, h), sub(k, h // g), sub(v, h // g),
                                                sub(do, h), *vb, 0, 0, rows)
            assert np.abs(to_np(O[b, h, rows]) - Or).max() <= O_TOL
            assert np.abs(to_np(L[b, h, rows]) - Lr).max() <= LSE_TOL
            assert rel_l2(to_np(dq[b, h, rows]), dQr) <= GRAD_TOL
    # gradient-sum invariants at full size: rows of dS sum to 0, so sum_j dK[j] = 0; rows
    # of P sum to 1, so sum_j dV[j] = the group's sum of dO over rows that see a key
    live = torch.isfinite(L).unsqueeze(-1)
    dO_live = (do.double() * live).view(w.batch, w.heads_kv, g, w.seqlen, D).sum((2, 3))
    dk64, dv64 = dk.double(), dv.double()
    eK = (dk64.sum(2).norm(dim=-1) / dk64.pow(2).sum(2).sum(-1).sqrt()).max().item()
    eV = ((dv64.sum(2) - dO_live).norm(dim=-1) / dv64.pow(2).sum(2).sum(-1).sqrt()).max().item()
    assert eK <= 0.05 and eV <= 0.05
