"""Running the fp64 oracle on large parity cases, one (batch row, query head) per task, in a
pool of fresh worker processes.

Each task calls the oracle unchanged on a single-head slice of the problem: Q and dO of head
h, K and V of its kv head h // (H_q / H_kv), the vectors of its batch row (or of its mask
set).  O, LSE and dQ of the slice are that head's rows of the whole result; the slice's dK
and dV are that head's contribution, and the contributions of a kv head's query heads are
summed here (the same sum the oracle forms, in another order: the results agree to fp64
rounding).  Workers are spawned (fresh interpreters that import numpy and the oracle only,
never the GPU), each with one BLAS thread, at most 16 of them."""
import multiprocessing as mp
import os

import numpy as np

import oracle

MAX_WORKERS = 16


def _fwd_bwd_task(args):
    from threadpoolctl import threadpool_limits
    q, k, v, do, vecs, scale = args
    with threadpool_limits(1):
        return oracle.attention_fwd_bwd(q, k, v, do, *vecs, scale=scale)


def _cols_task(args):
    from threadpoolctl import threadpool_limits
    q, k, v, do, vecs, cols, scale = args
    with threadpool_limits(1):
        return oracle.attention_cols(q, k, v, do, *vecs, 0, 0, cols, scale=scale)


def _pool_map(fn, tasks):
    n = max(1, min(MAX_WORKERS, os.cpu_count() or 1, len(tasks)))
    with mp.get_context("spawn").Pool(n) as pool:
        return pool.map(fn, tasks, chunksize=1)


def _head_vectors(vecs, b, h, heads_q):
    """The vectors of (b, h): [1][N] from [B][N], or its mask set's from [B][H_m][N]."""
    out = []
    for x in vecs:
        x = np.asarray(x)
        out.append(x[b:b + 1] if x.ndim == 2 else x[b:b + 1, h // (heads_q // x.shape[1])])
    return out


def fwd_bwd(q, k, v, do, vecs, scale=None):
    """(O, LSE, dQ, dK, dV) of the whole problem in float64, as oracle.attention_fwd_bwd."""
    B, Hq, N, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    tasks, keys = [], []
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            tasks.append((q[b:b + 1, h:h + 1], k[b:b + 1, kv:kv + 1], v[b:b + 1, kv:kv + 1],
                          do[b:b + 1, h:h + 1], _head_vectors(vecs, b, h, Hq), scale))
            keys.append((b, h, kv))
    res = _pool_map(_fwd_bwd_task, tasks)
    O = np.zeros((B, Hq, N, d)); LSE = np.full((B, Hq, N), -np.inf)
    dQ = np.zeros((B, Hq, N, d)); dK = np.zeros((B, Hkv, Nk, d)); dV = np.zeros((B, Hkv, Nk, d))
    for (b, h, kv), (o, lse, dq, dk, dv) in zip(keys, res):
        O[b, h], LSE[b, h], dQ[b, h] = o[0, 0], lse[0, 0], dq[0, 0]
        dK[b, kv] += dk[0, 0]
        dV[b, kv] += dv[0, 0]
    return O, LSE, dQ, dK, dV


def cols(q, k, v, do, vecs, b, kv, columns, scale=None):
    """dK and dV [len(columns)][d] of kv head `kv` of batch row b, as oracle.attention_cols."""
    Hq, Hkv = q.shape[1], k.shape[1]
    g = Hq // Hkv
    tasks = [(q[b:b + 1, h:h + 1], k[b:b + 1, kv:kv + 1], v[b:b + 1, kv:kv + 1],
              do[b:b + 1, h:h + 1], _head_vectors(vecs, b, h, Hq), np.asarray(columns), scale)
             for h in range(kv * g, (kv + 1) * g)]
    res = _pool_map(_cols_task, tasks)
    return sum(r[0] for r in res), sum(r[1] for r in res)
