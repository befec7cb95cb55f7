"""Per-head mask sets: vectors [B][H_m][N], query head h uses set h // (H_q / H_m).

The kernels against the fp64 oracle on small problems covering every way query heads,
kv heads and sets can relate (sets coarser than, equal to and finer than the kv heads;
dK/dV stored directly or summed over several work items), the classification per mask
row against the oracle's, and the variant's full-size workload on sampled rows and
columns.  Heads that see nothing, ragged tails and per-head all-hidden sets included."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import (GRAD_TOL, LSE_TOL, O_TOL, check_fwd, check_grads, gpu_inputs, log, rel_l2,
                    to_np)

pytestmark = pytest.mark.gpu

# (H_q, H_kv, H_m, N): what each case exercises
CASES = {
    "sets_per_query_head_g2": (4, 2, 4, 384),      # finer than kv heads: 2 writers per block
    "sets_per_kv_head_g4": (8, 2, 2, 320),         # = kv heads, direct bf16 stores, ragged
    "sets_coarser_than_kv": (8, 4, 2, 256),        # two kv heads per set
    "sets_split_group_of_8": (8, 1, 2, 448),       # one kv head, 2 sets of 4 heads
    "sets_per_query_head_g8": (8, 1, 8, 200),      # 8 writers per block, ragged
    "one_set_mqa_6": (6, 1, 1, 256),               # the shared case through 3-d vectors
}


def _problem(name, seed=0):
    hq, hkv, hm, n = CASES[name]
    return workloads.random_intervals(seed, n, batch=2, heads_q=hq, heads_kv=hkv, p_empty=0.3,
                                      mask_heads=hm)


def _hide_set(w, b, m):
    """Make set m of batch row b hide every row (its heads see nothing)."""
    lts, lte, uts, ute = w.vectors()
    lts[b, m] = 0
    lte[b, m] = w.seqlen


@pytest.mark.parametrize("name", list(CASES))
def test_per_head_matches_oracle(name):
    import mask_aware_sparse_amd as fm
    w = _problem(name)
    if w.mask_heads > 1:
        _hide_set(w, 1, w.mask_heads - 1)
    log(f"per-head {name}: Hq={w.heads_q} Hkv={w.heads_kv} Hm={w.mask_heads} N={w.seqlen}")
    q, k, v, do, vec = gpu_inputs(w)
    O, L = fm.attn_fwd(q, k, v, *vec)
    dq, dk, dv = fm.attn_bwd(q, k, v, O, L, do, *vec)
    torch.cuda.synchronize()
    ref = oracle.attention_fwd_bwd(*(to_np(x) for x in (q, k, v, do)), *w.vectors())
    check_fwd(O, L, ref[0], ref[1], ctx=name)
    check_grads(dq, dk, dv, ref[2:], ref[1], ctx=name)
    if w.mask_heads > 1:
        per = w.heads_q // w.mask_heads
        dead = slice(w.heads_q - per, w.heads_q)
        assert bool((O[1, dead] == 0).all()) and bool(torch.isneginf(L[1, dead]).all())
        assert bool((dq[1, dead] == 0).all())


@pytest.mark.parametrize("name", ["sets_per_query_head_g2", "sets_per_kv_head_g4",
                                  "sets_per_query_head_g8"])
def test_equal_sets_reproduce_the_shared_run(name):
    """Every set equal to one shared set: O, LSE and dQ are the shared run's bit for bit
    (the same tiles in the same order per head); dK/dV too when both store directly,
    else within the gradient tolerance (fp32 sums in another order)."""
    import mask_aware_sparse_amd as fm
    hq, hkv, hm, n = CASES[name]
    w = workloads.random_intervals(4, n, batch=2, heads_q=hq, heads_kv=hkv, p_empty=0.3)
    q, k, v, do, vec = gpu_inputs(w)
    vec3 = tuple(x[:, None, :].expand(-1, hm, -1).contiguous() for x in vec)
    a = fm.attn_fwd(q, k, v, *vec)
    b = fm.attn_fwd(q, k, v, *vec3)
    ga = fm.attn_bwd(q, k, v, *a, do, *vec)
    gb = fm.attn_bwd(q, k, v, *b, do, *vec3)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(ga[0], gb[0])
    g = hq // hkv
    direct = hm <= hkv and g <= 4
    for x, y in zip(ga[1:], gb[1:]):
        if direct:
            assert torch.equal(x, y)
        else:
            assert rel_l2(to_np(y), to_np(x)) <= GRAD_TOL


@pytest.mark.parametrize("bq,bk", [(128, 64), (32, 128), (64, 64)])
def test_classification_per_mask_row(bq, bk):
    import mask_aware_sparse_amd as fm
    w = workloads.random_intervals(9, 1000, batch=2, heads_q=6, mask_heads=3)
    vec = workloads.mask_tensors(w, device="cuda")
    out = fm.classify_tiles(*vec, bq, bk)
    torch.cuda.synchronize()
    flat = [x.reshape(-1, w.seqlen) for x in w.vectors()]       # mask rows b * H_m + m
    cls = oracle.classify(*flat, bq, bk)
    qq, qc, kq, kc = oracle.queues(cls)
    assert np.array_equal(out["tile_class"].cpu().numpy(), cls)
    assert np.array_equal(out["q_queue"].cpu().numpy(), qq)
    assert np.array_equal(out["q_count"].cpu().numpy(), qc)
    assert np.array_equal(out["k_queue"].cpu().numpy(), kq)
    assert np.array_equal(out["k_count"].cpu().numpy(), kc)
    assert np.array_equal(out["q_order"].cpu().numpy(),
                          oracle.lpt_order(oracle.tile_costs(qc)))
    assert np.array_equal(out["k_order"].cpu().numpy(),
                          oracle.lpt_order(oracle.tile_costs(kc)))


def test_localize_per_head_sets():
    import mask_aware_sparse_amd as fm
    w = workloads.random_intervals(2, 512, batch=2, heads_q=4, mask_heads=4)
    vec = workloads.mask_tensors(w, device="cuda")
    offs = [64, 256, 448]
    got = fm.localize_mask(*vec, torch.tensor(offs, dtype=torch.int32, device="cuda"), 64)
    for g, r in zip(got, oracle.localize_vectors(w.vectors(), offs, 64)):
        assert g.shape == vec[0].shape
        assert np.array_equal(g.cpu().numpy(), r)


def test_debug_expand_per_mask_row():
    import mask_aware_sparse_amd as fm
    w = workloads.random_intervals(6, 300, batch=2, heads_q=2, mask_heads=2)
    vec = workloads.mask_tensors(w, device="cuda")
    for b in range(2):
        for m in range(2):
            got = fm.debug_expand_mask(*vec, b * 2 + m, 0, 300).cpu().numpy().astype(bool)
            assert np.array_equal(got, oracle.dense_mask(*(x[b, m] for x in w.vectors())))


def test_full_size_variant_sampled():
    """The variant's benchmark workload (per-head windows, N = 32K, 32 query heads, 8 kv
    heads, 8 sets) in the launch configuration the benchmark times: sampled rows of every
    set against the oracle, and sampled key columns' dK/dV of two kv heads."""
    import mask_aware_sparse_amd as fm
    w = workloads.make_workload("v1_per_head_windows_32k")
    log(f"full-size per-head windows: Hq={w.heads_q} Hkv={w.heads_kv} Hm={w.mask_heads} "
        f"N={w.seqlen}")
    q, k, v, do, vec = gpu_inputs(w)
    O, L = fm.attn_fwd(q, k, v, *vec)
    dq, dk, dv = fm.attn_bwd(q, k, v, O, L, do, *vec)
    torch.cuda.synchronize()
    g = w.heads_q // w.heads_kv
    per = w.heads_q // w.mask_heads
    n = w.seqlen
    rng = np.random.default_rng(3)
    rows = sorted({0, 1, 63, 64, n - 1} | set(rng.integers(0, n, 5).tolist()))
    sub = lambda t, hh: to_np(t[:1, hh:hh + 1])
    for m in range(w.mask_heads):
        h = m * per + int(rng.integers(0, per))
        kvh = h // g
        vm = [x[:, m] for x in w.vectors()]
        Or, Lr, dQr = oracle.attention_rows(sub(q, h), sub(k, kvh), sub(v, kvh), sub(do, h),
                                            *vm, 0, 0, rows)
        assert np.abs(to_np(O[0, h, rows]) - Or).max() <= O_TOL, (m, h)
        assert np.abs(to_np(L[0, h, rows]) - Lr).max() <= LSE_TOL, (m, h)
        assert rel_l2(to_np(dq[0, h, rows]), dQr) <= GRAD_TOL, (m, h)
    # key columns near the end are seen by few rows in every set: cheap to recompute
    cols = [n - 300, n - 129, n - 64, n - 1]
    for kvh in (0, w.heads_kv - 1):
        dKr, dVr = oracle.attention_cols(to_np(q[:1]), to_np(k[:1]), to_np(v[:1]),
                                         to_np(do[:1]), *w.vectors(), 0, kvh, cols)
        assert rel_l2(to_np(dk[0, kvh, cols]), dKr) <= GRAD_TOL, kvh
        assert rel_l2(to_np(dv[0, kvh, cols]), dVr) <= GRAD_TOL, kvh
