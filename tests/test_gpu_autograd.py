"""flashmask_attention, the autograd wrapper over fm_attn_fwd / fm_attn_bwd, on the GPU:

  * gradients taken by torch.autograd equal the direct calls bit for bit (same kernels;
    problems whose dK/dV items store directly, so the backward is deterministic), in the
    natural key order and with keys regrouped;
  * the guide's two-vector form (key j visible to rows FMS_j..FME_j inclusive; FlashMask
    Guide, "Mathematical Formalization of Column-Wise Sparsity") through the conversion the
    wrapper documents, against the fp64 oracle at the parity tolerances."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_fwd, check_grads, gpu_inputs, log, to_np

pytestmark = pytest.mark.gpu


def _leaf(t):
    return t.detach().clone().requires_grad_(True)


CASES = {
    "prefix_lm_doc_1k_gqa": (lambda: workloads.prefix_lm_doc(0, n=1024, batch=2, heads_q=4,
                                                             heads_kv=2, lo=128, hi=512), 0),
    # keys regrouped in super-blocks (key_order = 1): the 256-key dK/dV kernel
    "random_eviction_4k_sorted": (lambda: workloads.random_eviction(1, n=4096, heads_q=2), 1),
}


@pytest.mark.parametrize("name", list(CASES))
def test_autograd_equals_direct_calls(name):
    import mask_aware_sparse_amd as fm
    make, key_order = CASES[name]
    w = make()
    log(f"autograd vs direct calls: {name} N={w.seqlen} B={w.batch} Hq={w.heads_q} "
        f"Hkv={w.heads_kv} key_order={key_order}")
    q, k, v, do, vec = gpu_inputs(w)
    ql, kl, vl = _leaf(q), _leaf(k), _leaf(v)
    o = fm.flashmask_attention(ql, kl, vl, *vec, key_order=key_order)
    # d(sum(o * do)) / do = do, exactly representable in bf16
    (o.float() * do.float()).sum().backward()
    O, LSE = fm.attn_fwd(q, k, v, *vec, key_order=key_order)
    dq, dk, dv = fm.attn_bwd(q, k, v, O, LSE, do, *vec, key_order=key_order)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), O)
    assert torch.equal(ql.grad, dq) and torch.equal(kl.grad, dk) and torch.equal(vl.grad, dv)


@pytest.mark.parametrize("causal", [True, False])
def test_two_vector_form_against_oracle(causal):
    import mask_aware_sparse_amd as fm
    lengths = [300, 180, 411, 133]
    n = sum(lengths)
    fms, fme = oracle.mask.encode_packed(lengths, causal=causal)
    log(f"two-vector form: packed documents {lengths} causal={causal}, Hq=4 Hkv=1")
    # the conversion stated in flashmask_attention's docstring, on the device
    fms_t = torch.from_numpy(np.asarray(fms, dtype=np.int32)).cuda()[None]
    fme_t = torch.from_numpy(np.asarray(fme, dtype=np.int32)).cuda()[None]
    lts = (fme_t + 1).contiguous()
    lte = torch.full_like(fms_t, n)
    uts = torch.zeros_like(fms_t)
    ute = fms_t.contiguous()
    g = torch.Generator(device="cuda").manual_seed(11)
    shp_q, shp_k = (1, 4, n, 128), (1, 1, n, 128)
    q, do = (torch.randn(shp_q, generator=g, device="cuda").bfloat16() for _ in range(2))
    k, v = (torch.randn(shp_k, generator=g, device="cuda").bfloat16() for _ in range(2))
    ql, kl, vl = _leaf(q), _leaf(k), _leaf(v)
    o = fm.flashmask_attention(ql, kl, vl, lts, lte, uts, ute)
    (o.float() * do.float()).sum().backward()
    O_dev, LSE_dev = fm.attn_fwd(q, k, v, lts, lte, uts, ute)
    torch.cuda.synchronize()
    # the oracle's own two-vector conversion, pinned on the CPU
    vecs = [x[None] for x in oracle.mask.visible_interval_to_vectors(fms, fme, n)]
    O_r, L_r, dQ_r, dK_r, dV_r = oracle.attention_fwd_bwd(to_np(q), to_np(k), to_np(v),
                                                          to_np(do), *vecs)
    fwd = check_fwd(o.detach(), LSE_dev, O_r, L_r, ctx="two-vector form")
    bwd = check_grads(ql.grad, kl.grad, vl.grad, (dQ_r, dK_r, dV_r), L_r, ctx="two-vector form")
    assert torch.equal(o.detach(), O_dev)
    log(f"  O max-abs {fwd[0]:.2e}, LSE max-abs {fwd[1]:.2e}, dQ/dK/dV rel-L2 "
        f"{bwd[0]:.2e}/{bwd[1]:.2e}/{bwd[2]:.2e}")
