"""GPU forward/backward vs the full fp64 oracle at sizes the oracle finishes in seconds
(several tiles, ragged tails, GQA, rows that see nothing)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import full_parity, gpu_inputs, log, to_np

pytestmark = pytest.mark.gpu

SMALL = {
    "c1_causal_doc_1k": lambda: workloads.causal_doc(0),
    "prefix_lm_doc_1k_gqa": lambda: workloads.prefix_lm_doc(0, n=1024, batch=2, heads_q=4,
                                                            heads_kv=2, lo=128, hi=512),
    "share_question_2k_mqa": lambda: workloads.share_question(0, n=2048, heads_q=4, heads_kv=1,
                                                              prompt_range=(128, 256),
                                                              answer_range=(64, 128)),
    "sliding_window_2k": lambda: workloads.sliding_window_sinks(n=2048, heads_q=2, window=300,
                                                                sinks=10),
    "random_eviction_1k": lambda: workloads.random_eviction(0, n=1024, heads_q=2),
    "random_intervals_700": lambda: workloads.random_intervals(3, 700, batch=2, heads_q=2),
    # query-head groups above 4: several workgroups add into one KV head's dK/dV
    # (two head chunks of 4 and 2 heads)
    "random_intervals_520_g6": lambda: workloads.random_intervals(5, 520, batch=1, heads_q=6,
                                                                  heads_kv=1),
    "prefix_lm_doc_1k_g8": lambda: workloads.prefix_lm_doc(4, n=1024, batch=1, heads_q=16,
                                                           heads_kv=2, lo=128, hi=512),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_workloads(name):
    w = SMALL[name]()
    log(f"parity {name} N={w.seqlen} B={w.batch} Hq={w.heads_q} Hkv={w.heads_kv}")
    res = full_parity(w)
    log(f"  {res}")


@pytest.mark.parametrize("n", [1, 7, 64, 65, 129, 333, 1000])
def test_ragged_lengths(n):
    w = workloads.random_intervals(n, n, batch=1, heads_q=2, heads_kv=1, p_empty=0.4)
    log(f"parity ragged N={n}")
    full_parity(w)


def test_causal_ragged_and_custom_scale():
    w = workloads.causal(777, heads_q=2, heads_kv=2)
    log("parity causal N=777 scale=0.05")
    full_parity(w, scale=0.05)


def test_no_mask_and_all_masked():
    n = 384
    w = workloads.causal(n, heads_q=2)
    w.ute[:] = 0                       # nothing hidden: full attention
    log("parity unmasked N=384")
    full_parity(w)
    w.ute[:] = n                       # every key hidden from every row
    log("parity all-masked N=384")
    import mask_aware_sparse_amd as fm
    q, k, v, do, vec = gpu_inputs(w)
    O, LSE = fm.attn_fwd(q, k, v, *vec)
    dq, dk, dv = fm.attn_bwd(q, k, v, O, LSE, do, *vec)
    torch.cuda.synchronize()
    assert (O == 0).all() and torch.isneginf(LSE).all()
    assert (dq == 0).all() and (dk == 0).all() and (dv == 0).all()


def test_gqa_equals_repeated_heads():
    import mask_aware_sparse_amd as fm
    w = workloads.prefix_lm_doc(2, n=640, batch=1, heads_q=8, heads_kv=2, lo=100, hi=300)
    log("gqa vs repeated heads N=640 Hq=8 Hkv=2")
    q, k, v, do, vec = gpu_inputs(w)
    O, LSE = fm.attn_fwd(q, k, v, *vec)
    dq, dk, dv = fm.attn_bwd(q, k, v, O, LSE, do, *vec)
    kr, vr = k.repeat_interleave(4, 1).contiguous(), v.repeat_interleave(4, 1).contiguous()
    O2, LSE2 = fm.attn_fwd(q, kr, vr, *vec)
    dq2, dk2, dv2 = fm.attn_bwd(q, kr, vr, O2, LSE2, do, *vec)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(LSE, LSE2)
    assert (dq.float() - dq2.float()).abs().max() < 1e-2
    dk2s = dk2.float().view(1, 2, 4, 640, 128).sum(2)
    dv2s = dv2.float().view(1, 2, 4, 640, 128).sum(2)
    assert ((dk.float() - dk2s).norm() / dk2s.norm()) < 1e-2
    assert ((dv.float() - dv2s).norm() / dv2s.norm()) < 1e-2


def test_forward_deterministic_and_order_invariant():
    # Swapping two batch rows (with their vectors) changes the LPT dispatch order; the
    # forward result of each row must not change in any bit.
    import mask_aware_sparse_amd as fm
    w = workloads.prefix_lm_doc(4, n=1024, batch=2, heads_q=4, heads_kv=2, lo=100, hi=700)
    q, k, v, do, vec = gpu_inputs(w)
    O, LSE = fm.attn_fwd(q, k, v, *vec)
    O1, LSE1 = fm.attn_fwd(q, k, v, *vec)
    sw = lambda t: t.flip(0).contiguous()
    Os, LSEs = fm.attn_fwd(sw(q), sw(k), sw(v), *(sw(x) for x in vec))
    torch.cuda.synchronize()
    assert torch.equal(O, O1) and torch.equal(LSE, LSE1)
    assert torch.equal(O, sw(Os)) and torch.equal(LSE, sw(LSEs))


@pytest.mark.parametrize("seed", [1, 2])
def test_c1_other_seeds(seed):
    log(f"parity c1 seed={seed}")
    full_parity(workloads.causal_doc(seed), seed=seed)


def test_partial_path_with_nothing_hidden_is_bit_identical():
    """Every tile classified partial (empty intervals straddling each block) but no cell
    hidden: the masked code path must give exactly the unmasked path's outputs."""
    import mask_aware_sparse_amd as fm
    n = 1000  # ragged: the last KV block is partial in both
    outs = []
    for w in (workloads.full_attention(n, heads_q=4, heads_kv=2),
              workloads.full_attention_partial_tiles(n, heads_q=4, heads_kv=2)):
        log(f"partial-vs-unmasked {w.name} N={n}")
        q, k, v, do, vec = gpu_inputs(w)
        O, LSE = fm.attn_fwd(q, k, v, *vec)
        dq, dk, dv = fm.attn_bwd(q, k, v, O, LSE, do, *vec)
        torch.cuda.synchronize()
        outs.append((O, LSE, dq, dk, dv))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["prefix_lm_doc_1k_gqa", "random_intervals_520_g6",
                                  "sliding_window_2k"])
def test_natural_schedule_same_outputs(name):
    """Index-order dispatch (fm_problem.schedule = natural) against the LPT order: O, LSE and
    dQ bit for bit (each row is written by one workgroup whatever the order); dK/dV up to the
    fp32 summation order (the split plan grants its extra segments in dispatch order, and
    atomic sums follow it)."""
    import mask_aware_sparse_amd as fm
    w = SMALL[name]()
    log(f"natural vs LPT schedule {name}")
    q, k, v, do, vec = gpu_inputs(w)
    outs = []
    for sched in (fm.SCHEDULE_LPT, fm.SCHEDULE_NATURAL):
        O, LSE = fm.attn_fwd(q, k, v, *vec, schedule=sched)
        dq, dk, dv = fm.attn_bwd(q, k, v, O, LSE, do, *vec, schedule=sched)
        torch.cuda.synchronize()
        outs.append((O, LSE, dq, dk, dv))
    (O1, L1, dq1, dk1, dv1), (O2, L2, dq2, dk2, dv2) = outs
    assert torch.equal(O1, O2) and torch.equal(L1, L2) and torch.equal(dq1, dq2)
    for a, b in ((dk1, dk2), (dv1, dv2)):
        assert ((a.float() - b.float()).norm() / b.float().norm()) < 1e-2
