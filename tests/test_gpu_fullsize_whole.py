"""Whole-tensor parity at full size: every element of O, LSE, dQ, dK and dV against the fp64
oracle, on the benchmark's calls.

  c2_prefix_lm_doc_8k        the prefix-LM document workload (B=4, 32/8 heads, N=8192), at
                             seeds 0 and 1 (document lengths and tensors)
  c3_share_question_32k      the share-question workload (B=1, 64 heads on one kv head,
                             N=32768): 64 heads of the oracle, about a minute on the box
  window4096_sinks64_32k_g8  the sliding-window-with-sinks mask at N=32768, 8 query heads on
                             one kv head: the sink block is seen by every row, so the dK/dV
                             split plan cuts its item into segments that add into the fp32
                             accumulators with atomics (two head chunks per KV block)
  window4096_sinks64_32k_g4  the same with 4 query heads: dK/dV stored directly, the sink
                             block's segments written to partial slots and reduced in order
  c3 most-viewed columns     dK/dV of the 12 prompt keys of the share-question workload
                             (N=32768, 64 heads) that the most rows see

Bars: O max-abs 1e-2; LSE max-abs 1e-3 with the -inf rows equal; dQ, dK, dV relative L2
2e-2 per whole tensor (also on the sink block alone), the worst (b, head) reported."""
import numpy as np
import pytest
import torch

import oracle_pool
import workloads
from parity import GRAD_TOL, check_fwd, check_grads, log, rel_l2, to_np

pytestmark = pytest.mark.gpu

WHOLE = {
    "c2_prefix_lm_doc_8k": lambda: workloads.make_workload("c2_prefix_lm_doc_8k"),
    "c2_prefix_lm_doc_8k_seed1": lambda: workloads.make_workload("c2_prefix_lm_doc_8k", 1),
    "c3_share_question_32k": lambda: workloads.make_workload("c3_share_question_32k"),
    "window4096_sinks64_32k_g8": lambda: workloads.sliding_window_sinks(n=32768, heads_q=8,
                                                                         heads_kv=1),
    "window4096_sinks64_32k_g4": lambda: workloads.sliding_window_sinks(n=32768, heads_q=4,
                                                                         heads_kv=1),
}


def _run(w):
    import mask_aware_sparse_amd as fm
    q, k, v, do = workloads.make_tensors(w, device="cuda")
    vec = workloads.mask_tensors(w, device="cuda")
    O, LSE = fm.attn_fwd(q, k, v, *vec)
    dq, dk, dv = fm.attn_bwd(q, k, v, O, LSE, do, *vec)
    torch.cuda.synchronize()
    return (q, k, v, do), (O, LSE, dq, dk, dv)


def worst(x, ref):
    """The largest relative L2 error over the leading (b, head) pairs."""
    e = [rel_l2(x[b, h], ref[b, h]) for b in range(x.shape[0]) for h in range(x.shape[1])]
    return max(e) if e else 0.0


@pytest.mark.parametrize("name", list(WHOLE))
def test_whole_tensors(name):
    w = WHOLE[name]()
    log(f"whole-tensor {name}: B={w.batch} Hq={w.heads_q} Hkv={w.heads_kv} N={w.seqlen}")
    (q, k, v, do), (O, LSE, dq, dk, dv) = _run(w)
    f32 = lambda t: t.float().cpu().numpy()
    O_r, L_r, dQ_r, dK_r, dV_r = oracle_pool.fwd_bwd(f32(q), f32(k), f32(v), f32(do),
                                                     w.vectors())
    fwd = check_fwd(O, LSE, O_r, L_r, ctx=name)
    bwd = check_grads(dq, dk, dv, (dQ_r, dK_r, dV_r), L_r, ctx=name)
    dQg, dKg, dVg = to_np(dq), to_np(dk), to_np(dv)
    log(f"  O max-abs {fwd[0]:.2e}, LSE max-abs {fwd[1]:.2e}, dQ/dK/dV rel-L2 "
        f"{bwd[0]:.2e}/{bwd[1]:.2e}/{bwd[2]:.2e}; worst (b, head) dQ {worst(dQg, dQ_r):.2e} "
        f"dK {worst(dKg, dK_r):.2e} dV {worst(dVg, dV_r):.2e}")
    sinks = w.info.get("sinks")
    if sinks:
        eK = rel_l2(dKg[:, :, :sinks], dK_r[:, :, :sinks])
        eV = rel_l2(dVg[:, :, :sinks], dV_r[:, :, :sinks])
        log(f"  sink keys (seen by every row): dK {eK:.2e} dV {eV:.2e}")
        assert eK <= GRAD_TOL and eV <= GRAD_TOL


def viewers(w, b):
    """Rows that see each key column (UTS = 0, LTE = N in the share-question mask)."""
    assert (w.uts[b] == 0).all() and (w.lte[b] == w.seqlen).all()
    return np.maximum(w.lts[b].astype(np.int64) - w.ute[b], 0)


def test_c3_most_viewed_columns():
    import mask_aware_sparse_amd as fm
    w = workloads.make_workload("c3_share_question_32k")
    vis = viewers(w, 0)
    cols = np.sort(np.argsort(-vis, kind="stable")[:12])
    log(f"c3 most-viewed key columns {cols.tolist()} seen by {vis[cols].min()}-{vis[cols].max()} "
        f"rows x {w.heads_q} heads")
    (q, k, v, do), (O, LSE, dq, dk, dv) = _run(w)
    f32 = lambda t: t.float().cpu().numpy()
    dK_r, dV_r = oracle_pool.cols(f32(q), f32(k), f32(v), f32(do), w.vectors(), 0, 0, cols)
    eK = rel_l2(to_np(dk[0, 0, cols]), dK_r)
    eV = rel_l2(to_np(dv[0, 0, cols]), dV_r)
    log(f"  dK {eK:.2e} dV {eV:.2e}")
    assert eK <= GRAD_TOL and eV <= GRAD_TOL
