"""fm_check_mask counts the row bounds outside [0, N_q]: zero on every benchmark workload's
vectors, and exactly the number planted on adversarial vectors (values below 0 and above N_q
in each of the four vectors, per-head sets, a query share with N_q < N_k, multi-interval)."""
import numpy as np
import pytest
import torch

import mask_aware_sparse_amd as fm
import workloads
from parity import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", workloads.CONFIG_NAMES)
def test_benchmark_vectors_are_in_range(name):
    w = workloads.make_workload(name)
    vec = workloads.mask_tensors(w, device="cuda")
    assert fm.check_mask(*vec) == 0


def planted(seed, shape, nq):
    rng = np.random.default_rng(seed)
    vec = [rng.integers(0, nq + 1, shape).astype(np.int32) for _ in range(4)]
    n_bad = 0
    for x in vec:
        flat = x.reshape(-1)
        idx = rng.choice(flat.size, size=min(flat.size, int(rng.integers(1, 40))), replace=False)
        bad = np.where(rng.random(idx.size) < 0.5, rng.integers(-5000, 0, idx.size),
                       rng.integers(nq + 1, nq + 5000, idx.size)).astype(np.int32)
        flat[idx] = bad
        n_bad += idx.size
    return vec, n_bad


@pytest.mark.parametrize("seed,shape,nq", [(0, (2, 1000), 1000), (1, (1, 3, 777), 777),
                                            (2, (2, 4096), 512), (3, (1, 1), 1)])
def test_planted_out_of_range_values_counted(seed, shape, nq):
    vec, n_bad = planted(seed, shape, nq)
    t = [torch.from_numpy(x).cuda() for x in vec]
    got = fm.check_mask(*t, seqlen_q=nq)
    log(f"check_mask shape={shape} N_q={nq}: planted {n_bad}, counted {got}")
    assert got == n_bad
    # the boundary values 0 and N_q are in range
    ok = [torch.full(shape, v, dtype=torch.int32, device="cuda") for v in (0, nq, 0, nq)]
    assert fm.check_mask(*ok, seqlen_q=nq) == 0


def test_multi_interval_counted():
    w = workloads.random_multi_intervals(4, 500, batch=2, n_intervals=3)
    st, en = (torch.from_numpy(x).cuda() for x in w.intervals())
    assert fm.check_mask_multi(st, en) == 0
    st[1, 2, 7] = -1
    en[0, 0, 499] = 501
    en[1, 1, 0] = 10 ** 6
    assert fm.check_mask_multi(st, en) == 3
