"""GPU tile classification vs the oracle: bit-exact (classes, queues, counts, block
min/max, LPT orders) and the dense mask expansion byte-exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import log

pytestmark = pytest.mark.gpu


def gpu_classify(w, bq, bk):
    import mask_aware_sparse_amd as fm
    vec = workloads.mask_tensors(w, device="cuda")
    out = fm.classify_tiles(*vec, bq, bk, heads_q=w.heads_q, heads_kv=w.heads_kv)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def oracle_minmax(w, bk):
    parts = [oracle.block_minmax(x, bk) for x in w.vectors()]
    return np.stack([a for mm in parts for a in mm], axis=-1).astype(np.int32)


def compare(w, bq, bk):
    log(f"classify {w.name} N={w.seqlen} B={w.batch} tile={bq}x{bk}")
    g = gpu_classify(w, bq, bk)
    cls = oracle.classify(*w.vectors(), bq, bk)
    qq, qc, kq, kc = oracle.queues(cls)
    assert np.array_equal(g["block_minmax"], oracle_minmax(w, bk))
    assert np.array_equal(g["tile_class"], cls)
    assert np.array_equal(g["q_queue"], qq)
    assert np.array_equal(g["q_count"], qc)
    assert np.array_equal(g["k_queue"], kq)
    assert np.array_equal(g["k_count"], kc)
    assert np.array_equal(g["q_order"], oracle.lpt_order(oracle.tile_costs(qc)))
    assert np.array_equal(g["k_order"], oracle.lpt_order(oracle.tile_costs(kc)))


@pytest.mark.parametrize("name", workloads.CONFIG_NAMES)
@pytest.mark.parametrize("tile", [(128, 64), (64, 128), (128, 128)])
def test_configs_bit_exact(name, tile):
    compare(workloads.make_workload(name), *tile)


# Long queue lists: 2, 4 or 8 Q-blocks of one mask row per classification workgroup (more
# than 4096, 8192 or 16384 queue rows), with a Q-block count that R does not divide.
@pytest.mark.parametrize("batch,n,bq,bk", [(3, 1499 * 16 - 5, 16, 128),
                                           (5, 1999 * 16 - 3, 16, 256),
                                           (3, 5555 * 16 - 7, 16, 256)])
def test_rows_per_workgroup(batch, n, bq, bk):
    w = workloads.random_intervals(21 + batch, n, batch=batch, p_empty=0.3)
    compare(w, bq, bk)


@pytest.mark.parametrize("seed", range(6))
def test_adversarial_and_ragged(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 3000))
    bq, bk = (int(x) for x in rng.choice([8, 16, 32, 64, 128, 256], 2))
    w = workloads.random_intervals(seed, n, batch=int(rng.integers(1, 4)), p_empty=0.3)
    compare(w, bq, bk)


def test_seeds_1_2():
    for seed in (1, 2):
        for name in workloads.CONFIG_NAMES:
            compare(workloads.make_workload(name, seed), 128, 64)


@pytest.mark.parametrize("name", workloads.CONFIG_NAMES[:3])
def test_dense_expansion_full(name):
    import mask_aware_sparse_amd as fm
    w = workloads.make_workload(name)
    vec = workloads.mask_tensors(w, device="cuda")
    for b in range(w.batch):
        dense = fm.debug_expand_mask(*vec, b, 0, w.seqlen).cpu().numpy()
        ref = oracle.dense_mask(*(x[b] for x in w.vectors()))
        assert np.array_equal(dense.astype(bool), ref), (name, b)


@pytest.mark.parametrize("name", workloads.CONFIG_NAMES[3:])
def test_dense_expansion_sampled_blocks(name):
    import mask_aware_sparse_amd as fm
    w = workloads.make_workload(name)
    vec = workloads.mask_tensors(w, device="cuda")
    rng = np.random.default_rng(0)
    # 256 distinct seeded 128-row blocks, the first and the last among them
    nb = w.seqlen // 128
    picks = np.r_[0, nb - 1, rng.choice(np.arange(1, nb - 1), 254, replace=False)]
    for r0 in np.sort(picks) * 128:
        dense = fm.debug_expand_mask(*vec, 0, int(r0), int(r0) + 128).cpu().numpy()
        ref = oracle.masked_rows(*(x[0] for x in w.vectors()), int(r0), int(r0) + 128)
        assert np.array_equal(dense.astype(bool), ref), (name, r0)


def test_dense_expansion_unaligned_rows():
    import mask_aware_sparse_amd as fm
    w = workloads.random_intervals(5, 301, batch=2)
    vec = workloads.mask_tensors(w, device="cuda")
    dense = fm.debug_expand_mask(*vec, 1, 7, 250).cpu().numpy()
    ref = oracle.masked_rows(*(x[1] for x in w.vectors()), 7, 250)
    assert np.array_equal(dense.astype(bool), ref)
