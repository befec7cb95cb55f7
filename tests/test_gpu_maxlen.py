"""The largest length the library accepts, N = 2^22 rows and keys (B = 1, one head, a causal
window of 256): the Q-block queues of 32,768 x 65,536 tiles (8 GiB of forward workspace,
24 GiB backward), sorted lists of 32,768-131,072 blocks (chunked sort and merge passes), and
32-bit offsets near their range.  Sampled rows and key columns against the oracle, and the
gradient-sum invariants.  One more row is rejected before anything is launched (CPU)."""
import ctypes

import numpy as np
import pytest
import torch

import mask_aware_sparse_amd as fm
import oracle
import workloads
from parity import GRAD_TOL, LSE_TOL, O_TOL, gpu_inputs, log, rel_l2, to_np

NMAX = 1 << 22


def test_one_row_past_the_limit_is_rejected():
    n = ctypes.c_size_t()
    for N, ok in ((NMAX, 0), (NMAX + 1, -2)):
        p = fm.Problem(1, 1, 1, N, 128, 0.0)
        assert fm.library().fm_workspace_size(ctypes.byref(p), fm.OP_FWD, 0, 0, ctypes.byref(n)) == ok


@pytest.mark.gpu
def test_maximum_length():
    w = workloads.sliding_window_sinks(n=NMAX, heads_q=1, heads_kv=1, window=256, sinks=0)
    log(f"maximum length N={w.seqlen}: workspaces fwd "
        f"{fm.workspace_size(1, 1, 1, NMAX, fm.OP_FWD) / 2**30:.1f} GiB, bwd "
        f"{fm.workspace_size(1, 1, 1, NMAX, fm.OP_BWD) / 2**30:.1f} GiB")
    q, k, v, do, vec = gpu_inputs(w)
    O, L = fm.attn_fwd(q, k, v, *vec)
    dq, dk, dv = fm.attn_bwd(q, k, v, O, L, do, *vec)
    torch.cuda.synchronize()
    n = w.seqlen
    rng = np.random.default_rng(22)
    rows = sorted({0, 1, 256, n // 2, n - 1} | set(rng.integers(0, n, 2).tolist()))
    sub = lambda t: t[:, :1].float().cpu().numpy()
    Or, Lr, dQr = oracle.attention_rows(sub(q), sub(k), sub(v), sub(do), *w.vectors(), 0, 0, rows)
    eo = np.abs(to_np(O[0, 0, rows]) - Or).max()
    el = np.abs(to_np(L[0, 0, rows]) - Lr).max()
    eq = rel_l2(to_np(dq[0, 0, rows]), dQr)
    log(f"  rows {len(rows)}: O {eo:.2e} LSE {el:.2e} dQ {eq:.2e}")
    assert eo <= O_TOL and el <= LSE_TOL and eq <= GRAD_TOL
    cols = [0, n // 3, n - 1]
    f32 = lambda t: t.float().cpu().numpy()
    dKr, dVr = oracle.attention_cols(f32(q), f32(k), f32(v), f32(do), *w.vectors(), 0, 0, cols,
                                     row_block=64)
    ek = rel_l2(to_np(dk[0, 0, cols]), dKr)
    ev = rel_l2(to_np(dv[0, 0, cols]), dVr)
    log(f"  cols {cols}: dK {ek:.2e} dV {ev:.2e}")
    assert ek <= GRAD_TOL and ev <= GRAD_TOL
    # sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i (every row sees its own key)
    sk = (dk[0, 0].double().sum(0).norm() / dk[0, 0].double().norm()).item()
    sv = ((dv[0, 0].double().sum(0) - do[0, 0].double().sum(0)).norm() /
          dv[0, 0].double().norm()).item()
    log(f"  invariants: sum dK {sk:.2e}, sum dV - sum dO {sv:.2e}")
    assert sk <= 0.05 and sv <= 0.05
