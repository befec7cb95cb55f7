"""Split dK/dV work items on the GPU.  A window mask with sink keys makes the sink block's
queue far longer than any other, so the dK/dV plan cuts its pair into queue segments:
fp32 partial sums reduced in segment order where bf16 would be stored directly, fp32
atomics where accumulators are used.  Checked against the fp64 oracle, and the direct
path for run-to-run bit identity (the reduction order is fixed)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_fwd, check_grads, gpu_inputs, log, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("hq,hkv", [(4, 1), (2, 2), (8, 1), (6, 2)])
def test_sink_window_matches_oracle(hq, hkv):
    import mask_aware_sparse_amd as fm
    w = workloads.sliding_window_sinks(n=2048, heads_q=hq, heads_kv=hkv, window=128, sinks=64)
    log(f"split: sink window Hq={hq} Hkv={hkv} N={w.seqlen}")
    q, k, v, do, vec = gpu_inputs(w)
    O, L = fm.attn_fwd(q, k, v, *vec)
    dq, dk, dv = fm.attn_bwd(q, k, v, O, L, do, *vec)
    torch.cuda.synchronize()
    ref = oracle.attention_fwd_bwd(*(to_np(x) for x in (q, k, v, do)), *w.vectors())
    check_fwd(O, L, ref[0], ref[1], ctx="sink window")
    check_grads(dq, dk, dv, ref[2:], ref[1], ctx="sink window")


def test_split_direct_path_is_deterministic():
    import mask_aware_sparse_amd as fm
    w = workloads.sliding_window_sinks(n=4096, heads_q=4, heads_kv=2, window=256, sinks=64)
    q, k, v, do, vec = gpu_inputs(w)
    O, L = fm.attn_fwd(q, k, v, *vec)
    first = fm.attn_bwd(q, k, v, O, L, do, *vec)
    second = fm.attn_bwd(q, k, v, O, L, do, *vec)
    torch.cuda.synchronize()
    for a, b in zip(first, second):
        assert torch.equal(a, b)


def test_split_multi_interval_sinks():
    """The multi-interval form with a sink block (window + random blocks)."""
    import mask_aware_sparse_amd as fm
    w = workloads.block_sparse_window(1, n=2048, heads_q=4, heads_kv=1, window=128,
                                      rand_blocks=2, block=128, sinks=64)
    q, k, v, do = workloads.make_tensors(w, device="cuda")
    s, e = workloads.mask_tensors(w, device="cuda")
    O, L = fm.attn_fwd_multi(q, k, v, s, e)
    dq, dk, dv = fm.attn_bwd_multi(q, k, v, O, L, do, s, e)
    torch.cuda.synchronize()
    ref = oracle.attention_fwd_bwd_multi(*(to_np(x) for x in (q, k, v, do)), w.starts, w.ends)
    check_fwd(O, L, ref[0], ref[1], ctx="multi sinks")
    check_grads(dq, dk, dv, ref[2:], ref[1], ctx="multi sinks")
