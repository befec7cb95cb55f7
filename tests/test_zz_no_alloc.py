"""fm_attn_fwd_static: the forward on the library's fixed device workspace, for callers
that cannot allocate.  Its outputs must equal fm_attn_fwd's (same kernels, same inputs) bit
for bit, on two calls in a row where the second problem is smaller and its workspace is the
first call's leftovers; both also meet the oracle bars."""
import ctypes

import numpy as np
import pytest
import torch

import mask_aware_sparse_amd as fm
import oracle
import workloads
from parity import check_fwd, gpu_inputs, log, to_np


def test_static_workspace_size_declared():
    text = open(fm.__file__.replace("mask_aware_sparse_amd/__init__.py", "include/fm.h")).read()
    assert "#define FM_STATIC_WORKSPACE_BYTES (16u << 20)" in text
    assert fm.STATIC_WORKSPACE_BYTES == 16 << 20


def test_oversized_problem_refused_before_launch():
    """A forward workspace beyond the static size: FM_ERR_WORKSPACE from the C entry point
    (nothing is dereferenced: the check precedes every launch) and a ValueError from the
    binding."""
    p = fm.Problem(1, 1, 1, 1 << 20, 128, 0.0, 0, 0, 0)       # 1M keys: ~512 MiB of queues
    assert fm.workspace_size(1, 1, 1, 1 << 20, fm.OP_FWD) > fm.STATIC_WORKSPACE_BYTES
    fake = ctypes.c_void_p(0x100000)
    m = fm.Mask(0x100000, 0x100000, 0x100000, 0x100000)
    st = fm.library().fm_attn_fwd_static(ctypes.byref(p), fake, fake, fake, ctypes.byref(m),
                                         fake, fake, None, None)
    assert st == -3                                            # FM_ERR_WORKSPACE
    q = torch.zeros((1, 1, 1 << 20, 128), dtype=torch.bfloat16, device="meta")
    vec = [torch.zeros((1, 1 << 20), dtype=torch.int32) for _ in range(4)]
    with pytest.raises(ValueError, match="static workspace"):
        fm.attn_fwd_static(q, q, q, *vec)


def test_invalid_problem_rejected():
    p = fm.Problem(1, 3, 2, 256, 128, 0.0, 0, 0, 0)            # H_q % H_kv != 0
    fake = ctypes.c_void_p(0x100000)
    m = fm.Mask(0x100000, 0x100000, 0x100000, 0x100000)
    assert fm.library().fm_attn_fwd_static(ctypes.byref(p), fake, fake, fake, ctypes.byref(m),
                                           fake, fake, None, None) == -1


def _static_vs_fwd(w, seed):
    q, k, v, do, vec = gpu_inputs(w, seed)
    O1, L1 = fm.attn_fwd(q, k, v, *vec)
    o = torch.empty_like(q)
    lse = torch.empty(O1.shape[:3], dtype=torch.float32, device=q.device)
    O2, L2 = fm.attn_fwd_static(q, k, v, *vec, out=o, lse=lse)
    torch.cuda.synchronize()
    assert O2.data_ptr() == o.data_ptr() and L2.data_ptr() == lse.data_ptr()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    O_r, L_r = oracle.attention_fwd(*(to_np(t) for t in (q, k, v)), *w.vectors())
    return check_fwd(O2, L2, O_r, L_r, ctx=w.name)


@pytest.mark.gpu
def test_static_forward_matches_fwd_on_two_calls_second_smaller():
    big = workloads.prefix_lm_doc(3, n=2048, batch=2, heads_q=4, heads_kv=2, lo=200, hi=700)
    small = workloads.causal_doc(5, n=777, heads_q=2, heads_kv=1)
    for w, seed in ((big, 0), (small, 1)):
        log(f"static fwd {w.name} N={w.seqlen} B={w.batch} Hq={w.heads_q}")
        log(f"  {_static_vs_fwd(w, seed)}")


@pytest.mark.gpu
def test_static_forward_at_the_size_limit_then_small():
    """The 128K-key sliding window (8.6 MiB of workspace, 2 heads) and then a small causal
    problem: the second call runs on the first call's leftovers."""
    big = workloads.sliding_window_sinks(n=131072, heads_q=2, heads_kv=1)
    need = fm.workspace_size(1, 2, 1, 131072, fm.OP_FWD)
    assert 8 << 20 < need <= fm.STATIC_WORKSPACE_BYTES
    q, k, v, do, vec = gpu_inputs(big)
    O1, L1 = fm.attn_fwd(q, k, v, *vec)
    O2, L2 = fm.attn_fwd_static(q, k, v, *vec)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    small = workloads.causal(333, heads_q=2, heads_kv=2)
    log(f"  after the limit: {_static_vs_fwd(small, 2)}")
