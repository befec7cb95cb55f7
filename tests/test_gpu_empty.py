"""Empty problems through the binding on the device: zero batch rows, zero length, and a
query share of zero rows against a non-empty key set.  Every call returns outputs of the
right (empty) shapes without launching anything that could touch them."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, Nq, Nk, d=128):
    g = torch.Generator(device="cpu").manual_seed(0)
    t = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16).cuda()
    q, do = t(B, Hq, Nq, d), t(B, Hq, Nq, d)
    k, v = t(B, Hkv, Nk, d), t(B, Hkv, Nk, d)
    j = torch.arange(Nk, dtype=torch.int32)
    vec = [torch.full((B, Nk), Nq, dtype=torch.int32), torch.full((B, Nk), Nq, dtype=torch.int32),
           torch.zeros((B, Nk), dtype=torch.int32), j.repeat(B, 1).clamp(max=Nq)]
    return q, k, v, do, [x.contiguous().cuda() for x in vec]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk", [(0, 2, 1, 64, 64), (1, 2, 1, 0, 0), (2, 4, 1, 0, 96)])
def test_empty_problem(B, Hq, Hkv, Nq, Nk):
    import mask_aware_sparse_amd as fm
    q, k, v, do, vec = _inputs(B, Hq, Hkv, Nq, Nk)
    O, L = fm.attn_fwd(q, k, v, *vec)
    dq, dk, dv = fm.attn_bwd(q, k, v, O, L, do, *vec)
    torch.cuda.synchronize()
    assert O.shape == q.shape and L.shape == (B, Hq, Nq)
    assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
    # no query row: every key's gradient is zero
    if B > 0 and Nq == 0:
        assert (dk == 0).all() and (dv == 0).all()
