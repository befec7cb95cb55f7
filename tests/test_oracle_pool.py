"""The pooled oracle runner (one task per (batch row, query head), summed dK/dV) gives the
oracle's own results: a harness check, not a pin of the oracle."""
import numpy as np

import oracle
import oracle_pool
import workloads


def test_pool_matches_direct_oracle():
    w = workloads.random_intervals(4, 300, batch=2, heads_q=6, heads_kv=2, mask_heads=3)
    q, k, v, do = (t.float().numpy() for t in workloads.make_tensors(w))
    ref = oracle.attention_fwd_bwd(q, k, v, do, *w.vectors())
    got = oracle_pool.fwd_bwd(q, k, v, do, w.vectors())
    for a, b in zip(got, ref):
        fin = np.isfinite(b)
        assert np.array_equal(np.isfinite(a), fin)
        assert np.allclose(a[fin], b[fin], rtol=1e-12, atol=1e-12)
    cols = np.array([0, 7, 150, 299])
    dK, dV = oracle_pool.cols(q, k, v, do, w.vectors(), 1, 1, cols)
    dKr, dVr = oracle.attention_cols(q, k, v, do, *w.vectors(), 1, 1, cols)
    assert np.allclose(dK, dKr, rtol=1e-12, atol=1e-12)
    assert np.allclose(dV, dVr, rtol=1e-12, atol=1e-12)
    assert np.allclose(dK, ref[3][1, 1, cols], rtol=1e-10, atol=1e-12)
