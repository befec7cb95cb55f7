"""The Python binding rejects every malformed tensor argument before it calls the C ABI.

The kernels address each buffer from its base pointer with the problem's strides, so a
wrong shape, dtype, layout or device would become out-of-bounds device accesses.  Shape
and dtype checks run before the device check, so the CPU suite reaches each of them with
host tensors; the last case of each entry point (right shapes, host memory) is refused
for its device."""
import pytest
import torch

import mask_aware_sparse_amd as fm

B, HQ, HKV, N, D = 1, 4, 2, 256, 128


def inputs(n=N):
    bf = dict(dtype=torch.bfloat16)
    q = torch.zeros((B, HQ, n, D), **bf)
    k = torch.zeros((B, HKV, n, D), **bf)
    v = torch.zeros((B, HKV, n, D), **bf)
    vec = [torch.zeros((B, n), dtype=torch.int32) for _ in range(4)]
    return q, k, v, vec


def bwd_inputs():
    q, k, v, vec = inputs()
    o, do = torch.zeros_like(q), torch.zeros_like(q)
    lse = torch.zeros((B, HQ, N), dtype=torch.float32)
    return q, k, v, o, lse, do, vec


def test_fwd_host_tensors_refused_for_their_device():
    q, k, v, vec = inputs()
    with pytest.raises(ValueError, match="on the GPU"):
        fm.attn_fwd(q, k, v, *vec)


@pytest.mark.parametrize("case", ["v_shape", "v_dtype", "out_shape", "out_dtype", "lse_shape",
                                  "lse_dtype", "q_layout", "mask_dtype", "mask_batch",
                                  "mask_keys", "mask_shapes_differ", "head_dim_mismatch"])
def test_fwd_shape_and_dtype_checks(case):
    q, k, v, vec = inputs()
    kw = {}
    msg = None
    if case == "v_shape":
        v = torch.zeros((B, HKV, N - 1, D), dtype=torch.bfloat16); msg = "v must have shape"
    elif case == "v_dtype":
        v = v.float(); msg = "v must be"
    elif case == "out_shape":
        kw["out"] = torch.zeros((B, HQ, N, D // 2), dtype=torch.bfloat16); msg = "out must have"
    elif case == "out_dtype":
        kw["out"] = torch.zeros((B, HQ, N, D), dtype=torch.float16); msg = "out must be"
    elif case == "lse_shape":
        kw["lse"] = torch.zeros((B, HQ, N + 1)); msg = "lse must have"
    elif case == "lse_dtype":
        kw["lse"] = torch.zeros((B, HQ, N), dtype=torch.float64); msg = "lse must be"
    elif case == "q_layout":
        q = torch.zeros((B, N, HQ, D), dtype=torch.bfloat16).transpose(1, 2); msg = "contiguous"
    elif case == "mask_dtype":
        vec[2] = vec[2].long(); msg = "int32"
    elif case == "mask_batch":
        vec = [torch.zeros((B + 1, N), dtype=torch.int32) for _ in range(4)]; msg = "batch"
    elif case == "mask_keys":
        vec = [torch.zeros((B, N + 128), dtype=torch.int32) for _ in range(4)]; msg = "key length"
    elif case == "mask_shapes_differ":
        vec[3] = torch.zeros((B, N + 1), dtype=torch.int32); msg = "one shape"
    elif case == "head_dim_mismatch":
        k = torch.zeros((B, HKV, N, D // 2), dtype=torch.bfloat16); msg = "disagree"
    with pytest.raises(ValueError, match=msg):
        fm.attn_fwd(q, k, v, *vec, **kw)


@pytest.mark.parametrize("case", ["o_shape", "dout_shape", "lse_shape", "lse_dtype", "dq_shape",
                                  "dk_shape", "dv_dtype", "grads_len", "host"])
def test_bwd_checks(case):
    q, k, v, o, lse, do, vec = bwd_inputs()
    grads = None
    msg = None
    if case == "o_shape":
        o = torch.zeros((B, HQ, N - 64, D), dtype=torch.bfloat16); msg = "o must have"
    elif case == "dout_shape":
        do = torch.zeros((B, HQ + 1, N, D), dtype=torch.bfloat16); msg = "dout must have"
    elif case == "lse_shape":
        lse = torch.zeros((B, HQ, N // 2)); msg = "lse must have"
    elif case == "lse_dtype":
        lse = torch.zeros((B, HQ, N), dtype=torch.bfloat16); msg = "lse must be"
    elif case == "dq_shape":
        grads = (torch.zeros_like(k), torch.zeros_like(k), torch.zeros_like(v)); msg = "dq must"
    elif case == "dk_shape":
        grads = (torch.zeros_like(q), torch.zeros_like(q), torch.zeros_like(v)); msg = "dk must"
    elif case == "dv_dtype":
        grads = (torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v).float())
        msg = "dv must be"
    elif case == "grads_len":
        grads = (torch.zeros_like(q), torch.zeros_like(k)); msg = "grads must be"
    elif case == "host":
        msg = "on the GPU"
    with pytest.raises(ValueError, match=msg):
        fm.attn_bwd(q, k, v, o, lse, do, *vec, grads=grads)


def test_classify_checks():
    _, _, _, vec = inputs()
    with pytest.raises(ValueError, match="on the GPU"):
        fm.classify_tiles(*vec, 128, 64)
    with pytest.raises(ValueError, match="positive"):
        fm.classify_tiles(*vec, 0, 64)
    shapes = fm._tile_shapes(B, N // 128, N // 64)
    out = {n: torch.zeros(shp, dtype=dt) for n, (shp, dt) in shapes.items()}
    out["q_queue"] = torch.zeros((B, N // 128, N // 64 + 1), dtype=torch.int32)
    with pytest.raises(ValueError, match="q_queue must have"):
        fm.classify_tiles(*vec, 128, 64, out=out)
    del out["q_queue"]
    with pytest.raises(ValueError, match="lacks"):
        fm.classify_tiles(*vec, 128, 64, out=out)


def test_expand_localize_and_key_order_checks():
    _, _, _, vec = inputs()
    with pytest.raises(ValueError, match="on the GPU"):
        fm.debug_expand_mask(*vec, 0, 0, 16)
    with pytest.raises(ValueError, match="row0 <= row1"):
        fm.debug_expand_mask(*vec, 0, 16, 0)
    offs = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="on the GPU"):
        fm.localize_mask(*vec, offs, 64)
    bad_out = tuple(torch.zeros((B, N + 1), dtype=torch.int32) for _ in range(4))
    with pytest.raises(ValueError, match=r"out\[0\] must have"):
        fm.localize_mask(*vec, offs, 64, out=bad_out)
    with pytest.raises(ValueError, match="offsets"):
        fm.localize_mask(*vec, offs.long(), 64)
    with pytest.raises(ValueError, match="on the GPU"):
        fm.key_order(*vec)


def test_workspace_checks():
    q, k, v, vec = inputs()
    ws = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="too small"):
        fm._workspace(1 << 20, q.device, ws)
    with pytest.raises(ValueError, match="contiguous"):
        fm._workspace(8, q.device, torch.zeros((8, 8), dtype=torch.uint8).t())


@pytest.mark.gpu
def test_mixed_devices_refused_on_the_gpu():
    """Q on the GPU with host mask vectors, outputs or workspaces: refused before launch."""
    q, k, v, vec = inputs()
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    with pytest.raises(ValueError, match="mask tensor 0 must be on"):
        fm.attn_fwd(q, k, v, *vec)
    gvec = [t.cuda() for t in vec]
    with pytest.raises(ValueError, match="out must be on"):
        fm.attn_fwd(q, k, v, *gvec, out=torch.zeros((B, HQ, N, D), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="workspace must be on"):
        fm.attn_fwd(q, k, v, *gvec, ws=torch.zeros(1 << 24, dtype=torch.uint8))
    with pytest.raises(ValueError, match="k must be on"):
        fm.attn_fwd(q, k.cpu(), v, *gvec)


def test_flashmask_attention_checks_like_attn_fwd():
    """The autograd wrapper validates through attn_fwd: the same refusals, before any call."""
    q, k, v, vec = inputs()
    assert "flashmask_attention" in fm.__all__
    with pytest.raises(ValueError, match="on the GPU"):
        fm.flashmask_attention(q.clone().requires_grad_(True), k, v, *vec)
    with pytest.raises(ValueError):
        fm.flashmask_attention(q, k, v[:, :, :-1].contiguous(), *vec)
    with pytest.raises(ValueError):
        fm.flashmask_attention(q, k, v, *vec[:3], vec[3].to(torch.int64))
