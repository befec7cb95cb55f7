"""Key reordering (fm_key_order and fm_problem.key_order = FM_KEYS_SORTED).

The permutation and the permuted vectors bit for bit against the oracle's rule (index
work), on masks that sort (random eviction), keep the natural order (sliding window with
sinks, causal documents) or mix both (random intervals), with ragged super-blocks, bounds
past N_q and several mask rows; the attention outputs with sorted keys against the fp64
oracle in the caller's key order (direct dK/dV stores and fp32 accumulators, GQA,
per-head sets, ragged tails), the tiles of the permuted vectors against the oracle's
classification, and the sorted path on the full-size random-eviction workload (sampled
rows and columns, gradient-sum invariants)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import (GRAD_TOL, LSE_TOL, O_TOL, check_fwd, check_grads, full_parity, gpu_inputs,
                    log, rel_l2, to_np)

pytestmark = pytest.mark.gpu

SPAN, GROUP = 2048, 64


def _vec_tensors(vecs):
    return [torch.as_tensor(np.ascontiguousarray(x), dtype=torch.int32).cuda() for x in vecs]


def _orders():
    w1 = workloads.random_eviction(1, n=8192, batch=2, heads_q=1)
    w2 = workloads.random_eviction(2, n=5000, heads_q=1)            # ragged super-block
    w3 = workloads.sliding_window_sinks(0, n=9000, heads_q=1, window=1024)
    w4 = workloads.random_intervals(3, 6500, batch=2, p_empty=0.3)
    w5 = workloads.causal_doc(0, n=4096)
    return {"random_eviction_2x8192": (w1.vectors(), w1.seqlen),
            "random_eviction_5000": (w2.vectors(), w2.seqlen),
            "random_intervals_2x6500": (w4.vectors(), w4.seqlen),
            "causal_doc_4096": (w5.vectors(), w5.seqlen),
            "random_eviction_nq_3000": (w2.vectors(), 3000),              # bounds past N_q
            "random_eviction_per_head": (
                [np.stack([a[0], b[0]])[None] for a, b in zip(w1.vectors(),
                                                               workloads.random_eviction(
                                                                   4, n=8192).vectors())],
                8192),
            "sliding_window_sinks_9000": (w3.vectors(), w3.seqlen)}


@pytest.mark.parametrize("name", sorted(_orders()))
def test_permutation_bit_exact(name):
    import mask_aware_sparse_amd as fm
    vecs, nq = _orders()[name]
    t = _vec_tensors(vecs)
    perm, pv = fm.key_order(*t, seqlen_q=nq, permuted=True)
    torch.cuda.synchronize()
    ref = oracle.key_order_rows(*vecs, nq, SPAN, GROUP)
    got = perm.cpu().numpy()
    assert np.array_equal(got, ref), name
    nk = ref.shape[-1]
    flat = ref.reshape(-1, nk)
    for x, y in zip(vecs, pv):
        xr = np.asarray(x).reshape(-1, nk)
        want = np.stack([xr[r][flat[r]] for r in range(flat.shape[0])]).reshape(ref.shape)
        assert np.array_equal(y.cpu().numpy(), want)
    moved = int((flat != np.arange(nk)).any(axis=0).sum())
    log(f"key order {name}: {moved} of {nk} positions moved")
    if name.startswith("random_eviction"):
        assert moved >= SPAN
    if name.startswith(("causal_doc", "sliding")):
        assert moved == 0


@pytest.mark.parametrize("name,hq,hkv,n", [
    ("direct_gqa", 4, 2, 4096),        # dK/dV stored by one item per block, 2 kv heads
    ("acc_mqa8_ragged", 8, 1, 4500),   # fp32 accumulators (8 heads per kv head), ragged
])
def test_attention_sorted_keys_match_oracle(name, hq, hkv, n):
    w = workloads.random_eviction(5, n=n, heads_q=hq, heads_kv=hkv)
    log(f"sorted keys {name}: Hq={hq} Hkv={hkv} N={n}")
    full_parity(w, key_order=1)


def test_attention_sorted_keys_natural_mask():
    # a mask whose order is kept: the gathers are identities, so O, LSE and dQ are the
    # natural path's bit for bit; dK and dV come from 256-key workgroups with sorted keys
    # at d = 128 (another summation order), checked against the oracle
    import mask_aware_sparse_amd as fm
    w = workloads.causal_doc(0, n=4096, ndocs=6)
    q, k, v, do, vec = gpu_inputs(w)
    a = fm.attn_fwd(q, k, v, *vec)
    b = fm.attn_fwd(q, k, v, *vec, key_order=1)
    ga = fm.attn_bwd(q, k, v, a[0], a[1], do, *vec)
    gb = fm.attn_bwd(q, k, v, b[0], b[1], do, *vec, key_order=1)
    torch.cuda.synchronize()
    for x, y in zip(a + ga[:1], b + gb[:1]):
        assert torch.equal(x, y)
    ref = oracle.attention_fwd_bwd(*(to_np(x) for x in (q, k, v, do)), *w.vectors())
    check_grads(gb[0], gb[1], gb[2], ref[2:], ref[1], ctx="natural mask, sorted keys")


def test_attention_sorted_keys_per_head_sets():
    import mask_aware_sparse_amd as fm
    w = workloads.random_eviction(6, n=4096, heads_q=4, heads_kv=2)
    other = workloads.random_eviction(7, n=4096).vectors()
    vecs = [np.stack([a[0], b[0]])[None] for a, b in zip(w.vectors(), other)]
    q, k, v, do, _ = gpu_inputs(w)
    vt = _vec_tensors(vecs)
    O, L = fm.attn_fwd(q, k, v, *vt, key_order=1)
    dq, dk, dv = fm.attn_bwd(q, k, v, O, L, do, *vt, key_order=1)
    torch.cuda.synchronize()
    ref = oracle.attention_fwd_bwd(*(to_np(x) for x in (q, k, v, do)), *vecs)
    check_fwd(O, L, ref[0], ref[1], ctx="per-head sorted")
    check_grads(dq, dk, dv, ref[2:], ref[1], ctx="per-head sorted")


def test_permuted_tiles_match_oracle_classification():
    # the classes of the permuted vectors (what the kernels run over) against the oracle's
    # classification of the oracle's permuted vectors, and their cost against the natural
    import mask_aware_sparse_amd as fm
    w = workloads.random_eviction(8, n=16384, heads_q=1)
    vecs = w.vectors()
    perm, pv = fm.key_order(*_vec_tensors(vecs), permuted=True)
    out = fm.classify_tiles(*pv, 128, 64)
    torch.cuda.synchronize()
    ref_perm = oracle.key_order_rows(*vecs, w.seqlen)
    pvr = [np.take_along_axis(np.asarray(x), ref_perm, axis=-1) for x in vecs]
    cls = oracle.classify(*pvr, 128, 64)
    assert np.array_equal(out["tile_class"].cpu().numpy(), cls)
    nat = oracle.classify(*vecs, 128, 64)
    cost = lambda c: 11 * int((c == 1).sum()) + 10 * int((c == 2).sum())
    log(f"forward tile cost natural {cost(nat)} sorted {cost(cls)}")
    assert cost(cls) < 0.65 * cost(nat)


@pytest.mark.parametrize("d", [64, 256])
def test_attention_sorted_keys_other_head_dims(d):
    w = workloads.with_head_dim(workloads.random_eviction(9, n=4096, heads_q=2, heads_kv=1), d)
    log(f"sorted keys d={d}: N={w.seqlen}")
    full_parity(w, key_order=1)


def test_attention_sorted_keys_split_plan():
    # one head, 8K keys: 64 KV blocks for 512 workgroup slots, so the long queues are cut
    # into segments whose fp32 partial sums are reduced before the scatter
    w = workloads.random_eviction(10, n=8192, heads_q=1, heads_kv=1)
    full_parity(w, key_order=1)


def test_attention_sorted_keys_query_share():
    # one context-parallel rank's rows against all keys (N_q < N_k), vectors localized to
    # the rank's rows: the key order clips bounds at N_q
    import mask_aware_sparse_amd as fm
    w = workloads.random_eviction(11, n=8192, heads_q=2, heads_kv=1)
    q, k, v, do, vec = gpu_inputs(w)
    C = 1024
    offs = [1024, 4096, 6144]
    rows = torch.from_numpy(oracle.rank_rows(offs, C)).to(q.device)
    qr, dor = q[:, :, rows].contiguous(), do[:, :, rows].contiguous()
    lv = fm.localize_mask(*vec, torch.tensor(offs, dtype=torch.int32, device=q.device), C)
    O, L = fm.attn_fwd(qr, k, v, *lv, key_order=1)
    dq, dk, dv = fm.attn_bwd(qr, k, v, O, L, dor, *lv, key_order=1)
    torch.cuda.synchronize()
    lvn = [x.cpu().numpy() for x in lv]
    ref = oracle.attention_fwd_bwd(*(to_np(x) for x in (qr, k, v, dor)), *lvn)
    check_fwd(O, L, ref[0], ref[1], ctx="query share sorted")
    check_grads(dq, dk, dv, ref[2:], ref[1], ctx="query share sorted")
    perm = fm.key_order(*lv, seqlen_q=len(rows))
    torch.cuda.synchronize()
    assert np.array_equal(perm.cpu().numpy(), oracle.key_order_rows(*lvn, len(rows)))
