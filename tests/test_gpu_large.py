"""Work lists longer than one workgroup sorts (more than 8192 blocks): the LPT order is
then sorted in chunks and merged, and the dK/dV plan runs without splitting.  The
classification and both orders against the oracle at 18,752 blocks per list, and attention
at 9,376 Q-blocks against the oracle on sampled rows and key columns."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import GRAD_TOL, LSE_TOL, O_TOL, gpu_inputs, log, rel_l2, to_np

pytestmark = pytest.mark.gpu


def test_lpt_orders_of_long_lists():
    import mask_aware_sparse_amd as fm
    n, bq, bk = 300_000, 64, 64
    w = workloads.random_intervals(12, n, batch=4, p_empty=0.3)
    log(f"long lists: B=4 N={n} blocks {bq}x{bk}")
    vec = workloads.mask_tensors(w, device="cuda")
    out = fm.classify_tiles(*vec, bq, bk)
    torch.cuda.synchronize()
    cls = oracle.classify(*w.vectors(), bq, bk)
    qq, qc, kq, kc = oracle.queues(cls)
    assert qc.shape[0] * qc.shape[1] > 8192 * 2       # three chunks, two merge passes
    assert np.array_equal(out["q_count"].cpu().numpy(), qc)
    assert np.array_equal(out["k_count"].cpu().numpy(), kc)
    assert np.array_equal(out["q_order"].cpu().numpy(), oracle.lpt_order(oracle.tile_costs(qc)))
    assert np.array_equal(out["k_order"].cpu().numpy(), oracle.lpt_order(oracle.tile_costs(kc)))


def test_attention_beyond_one_workgroup_sort():
    import mask_aware_sparse_amd as fm
    w = workloads.sliding_window_sinks(n=600_064, batch=2, heads_q=2, heads_kv=1, window=256,
                                       sinks=0)
    log(f"long sequence: B=2 N={w.seqlen} window 256")
    q, k, v, do, vec = gpu_inputs(w)
    O, L = fm.attn_fwd(q, k, v, *vec)
    dq, dk, dv = fm.attn_bwd(q, k, v, O, L, do, *vec)
    torch.cuda.synchronize()
    n = w.seqlen
    rng = np.random.default_rng(7)
    rows = sorted({0, 1, 255, 256, n - 1} | set(rng.integers(0, n, 8).tolist()))
    for b in (0, 1):
        vb = [x[b:b + 1] for x in w.vectors()]
        for h in (0, 1):
            sub = lambda t, hh: to_np(t[b:b + 1, hh:hh + 1])
            Or, Lr, dQr = oracle.attention_rows(sub(q, h), sub(k, 0), sub(v, 0), sub(do, h), *vb,
                                                0, 0, rows)
            assert np.abs(to_np(O[b, h, rows]) - Or).max() <= O_TOL
            assert np.abs(to_np(L[b, h, rows]) - Lr).max() <= LSE_TOL
            assert rel_l2(to_np(dq[b, h, rows]), dQr) <= GRAD_TOL
        cols = sorted({0, 300_000, n - 300, n - 1} | set(rng.integers(0, n, 3).tolist()))
        dKr, dVr = oracle.attention_cols(to_np(q[b:b + 1]), to_np(k[b:b + 1]), to_np(v[b:b + 1]),
                                         to_np(do[b:b + 1]), *vb, 0, 0, cols)
        assert rel_l2(to_np(dk[b, 0, cols]), dKr) <= GRAD_TOL
        assert rel_l2(to_np(dv[b, 0, cols]), dVr) <= GRAD_TOL
