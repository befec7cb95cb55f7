#!/usr/bin/env python3
"""Benchmark: mask-aware attention forward + backward on one MI355X.

One step = fm_attn_fwd + fm_attn_bwd (classification, LPT order, attention kernels,
backward pre/post kernels) over one batch of seeded synthetic inputs resident in HBM.

Metric: effective TFLOP/s counting attended (q, k) pairs only, 4*d flop per pair in
the forward and 10*d in the backward (14*d = 1792 flop per pair at d = 128), over the
whole step time (wall clock over the timed steps).  The roofline entry covers the
dominant (longest) attention kernel: algorithmic flop per launch / its average duration,
measured with HIP events recorded around that kernel on the stream it runs on, in every
other timed step.  Its `traffic` is the HBM bytes per launch
from a committed rocprofv3 counter summary (profiles/traffic_<kernel>_<workload>.txt),
reported only while the kernel sources still hash to the value recorded there.

The default run times the random-eviction workload (128K keys, keys sorted) and then the
share-question (32K) and sliding-window (128K) workloads, reported under "also".  `peak` is
the published dense bf16 MFMA figure; beside it the line gives the device's CU count, the
GFX clock sampled (amdsmi) during the timed steps and the MFMA peak at that clock.
`--schedule natural` dispatches work items in index order instead of LPT order.

Prints ONE JSON line.  `--gpus N` with N > 1 exits: the benchmark runs on one GPU.
`--calibrate-copy MIB` instead runs a plain device-to-device copy of that size (for
scaling the FETCH_SIZE / WRITE_SIZE counters) and prints its byte count.
`--classify-bandwidth` instead times fm_classify_tiles (block min/max, classes, both queue
sets, costs, both LPT orders) on the c5 vectors replicated over 4 batch rows (the most the
single-workgroup LPT sort takes at the forward tile: 4 x 2048 KV blocks), against the
HBM roofline.
`--cp P` instead emulates context parallelism over P ranks on the one GPU: the query
axis of the workload is cut into 2P chunks, assigned to ranks either contiguously or by
fm_ipo_balance on the chunks' tile costs; each rank's share (its chunks' rows against
all keys, vectors renumbered by fm_localize_mask) runs fwd+bwd in turn, and the per-rank
times, their max/mean and the rate of a job bounded by the slowest rank are reported.
`--ipo-table` instead runs the host chunk balancer (fm_ipo_balance, HCC-IPO stage 1) on
seeded instances of the FlashMask-3 page's IPO ablation configurations and prints the
share of instances above the lower bound after LPT, P2 and P3, the mean gaps and times.
`--measure-alpha` instead times the relative cost of a partial tile (the alpha_p : alpha_u
of the FlashMask-3 page's tile cost, §3.3): full attention classified all-unmasked
against the same attention classified all-partial (empty intervals, nothing hidden).
"""
import hashlib
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

MFMA_BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16: 256 CU x 2.4 GHz x 4096 flop/clk/CU
MFMA_BF16_FLOP_PER_CLK_CU = 4096
# The headline runs on the largest single-GPU configuration (random eviction, 128K keys);
# the other long-context configurations are timed in the same run and reported beside it.
DEFAULT_WORKLOAD = "c5_random_eviction_128k"
ALSO_WORKLOADS = ("c3_share_question_32k", "c4_sliding_window_128k")
# workloads timed with their keys reordered (fm_problem.key_order = FM_KEYS_SORTED) unless
# --key-order says otherwise: the random-eviction mask, whose columns end at scattered rows
SORTED_KEY_WORKLOADS = {"c5_random_eviction_128k"}


def attended_pairs(w):
    """Attended (q, k) pairs summed over batch rows and query heads, by interval
    arithmetic on the column vectors (N_q = w.seqlen rows minus the union of the two
    hidden intervals, per key column).  Per-head vectors [B][H_m][N] count each set once
    per query head that uses it (H_q / H_m heads)."""
    vecs = [np.asarray(x, dtype=np.int64) for x in w.vectors()]
    if vecs[0].ndim == 2:
        vecs = [x[:, None, :] for x in vecs]
    hm = vecs[0].shape[1]
    total = 0
    n = w.seqlen
    for b in range(w.batch):
        for m in range(hm):
            lts, lte, uts, ute = (x[b, m] for x in vecs)
            a1, b1 = np.clip(lts, 0, n), np.clip(lte, 0, n)
            a2, b2 = np.clip(uts, 0, n), np.clip(ute, 0, n)
            l1, l2 = np.maximum(b1 - a1, 0), np.maximum(b2 - a2, 0)
            inter = np.maximum(np.minimum(b1, b2) - np.maximum(a1, a2), 0)
            inter = np.where((l1 > 0) & (l2 > 0), inter, 0)
            total += int((n - (l1 + l2 - inter)).sum())
    return total * (w.heads_q // hm)


def attended_pairs_multi(w):
    """Attended pairs of a multi-interval workload: per key column, the length of the union
    of its visible intervals clipped to [0, N_q), times the query heads that use the set."""
    st = np.clip(np.asarray(w.starts, dtype=np.int64), 0, w.seqlen)
    en = np.clip(np.asarray(w.ends, dtype=np.int64), 0, w.seqlen)
    if st.ndim == 3:
        st, en = st[:, None], en[:, None]
    en = np.maximum(en, st)                      # empty intervals have no length
    order = np.argsort(st, axis=2, kind="stable")
    st = np.take_along_axis(st, order, axis=2)
    en = np.take_along_axis(en, order, axis=2)
    covered = np.zeros(st.shape[:2] + st.shape[3:], dtype=np.int64)
    reach = np.zeros_like(covered)               # end of the union so far
    for m in range(st.shape[2]):
        covered += np.maximum(en[:, :, m] - np.maximum(st[:, :, m], reach), 0)
        reach = np.maximum(reach, en[:, :, m])
    return int(covered.sum()) * (w.heads_q // st.shape[1])


def attended_pairs_blocks(w):
    """Attended pairs of a block-sparse workload: the area of every visible 128 x 128 block
    (cut at N), times the query heads that use the grid."""
    g = np.asarray(w.blocks, dtype=np.int64)
    if g.ndim == 3:
        g = g[:, None]
    n, blk = w.seqlen, 128
    edge = np.minimum(np.arange(g.shape[-1]) * blk + blk, n) - np.arange(g.shape[-1]) * blk
    area = int(np.einsum('bmij,i,j->', g, edge[:g.shape[-2]], edge))
    return area * (w.heads_q // g.shape[1])


def head_vectors(w, b, h):
    """The four vectors [1][N] query head h of batch row b uses."""
    if w.lts.ndim == 2:
        return [x[b:b + 1] for x in w.vectors()]
    m = h // (w.heads_q // w.mask_heads)
    return [x[b:b + 1, m] for x in w.vectors()]


def source_digest():
    """sha256 over the library's kernel sources and headers (what the counters measured)."""
    h = hashlib.sha256()
    for d in ("mask_aware_sparse_amd/csrc", "include"):
        for f in sorted(os.listdir(os.path.join(ROOT, d))):
            if f.endswith((".hip", ".h", ".cpp")):
                with open(os.path.join(ROOT, d, f), "rb") as fh:
                    h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def stored_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter summary,
    or None when there is none or the sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.lstrip().startswith("#"):
                key, val = line.split("=", 1)
                kv[key.strip()] = val.strip()
    if kv.get("source_sha256") != source_digest():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calibrate_copy(mib):
    """A plain copy of `mib` MiB (read once, written once) for counter calibration."""
    import torch
    n = mib * 2**20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}))


HBM_PEAK_GBS = 8000.0   # MI355X HBM3E


def classify_bandwidth(steps, warmup, batch=4, block_q=128, block_k=64):
    """fm_classify_tiles on the c5 (random eviction, N = 131072) vectors replicated to
    `batch` rows, at the forward's tile shape.  Bytes: the algorithmic traffic (vectors
    read once; block min/max, classes, one int32 per queued tile per direction, counts,
    costs and orders written once) and the bytes this layout actually writes (queue rows
    are fixed-length, filled with -1 past the count)."""
    import torch
    import mask_aware_sparse_amd as fm
    w = workloads.make_workload("c5_random_eviction_128k", 0)
    n = w.seqlen
    vec = [torch.from_numpy(np.ascontiguousarray(np.repeat(x[:1], batch, 0))).cuda()
           for x in w.vectors()]
    nqb, nkb = -(-n // block_q), -(-n // block_k)
    ws = torch.empty(fm.workspace_size(batch, 1, 1, n, fm.OP_CLASSIFY, block_q, block_k),
                     dtype=torch.uint8, device="cuda")
    out = fm.classify_tiles(*vec, block_q, block_k, ws=ws)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(warmup + steps):
        e = ev[i - warmup] if i >= warmup else None
        if e:
            e[0].record()
        fm.classify_tiles(*vec, block_q, block_k, out=out, ws=ws)
        if e:
            e[1].record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    queued = int((out["tile_class"] != 0).sum())
    read = 16 * batch * n
    small = 32 * batch * nkb + 8 * batch * (nqb + nkb) + 8 * batch * (nqb + nkb)  # mm, counts, costs+orders
    alg = read + small + batch * nqb * nkb + 2 * 4 * queued
    layout = read + small + batch * nqb * nkb + 2 * 4 * batch * nqb * nkb
    gbs = lambda b: b / (ms * 1e-3) / 1e9
    print(json.dumps({
        "measure": "fm_classify_tiles bandwidth",
        "config": {"vectors": "c5_random_eviction_128k replicated", "batch": batch,
                   "seq_len": n, "block_q": block_q, "block_k": block_k,
                   "queued_tiles": queued, "steps": steps, "warmup": warmup},
        "ms_median": round(ms, 4),
        "algorithmic_bytes": alg, "layout_bytes": layout,
        "roofline": {"bound": "hbm", "achieved": round(gbs(alg), 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs(alg) / HBM_PEAK_GBS, 4)},
        "layout_gbs": round(gbs(layout), 1)}))


def cp_emulation(workload, P, steps, warmup, kappa=2):
    import torch
    import mask_aware_sparse_amd as fm
    w = workloads.make_workload(workload, 0)
    n = w.seqlen
    nch = P * kappa
    if n % nch or (n // nch) % 128:
        raise SystemExit(f"--cp {P}: N = {n} does not split into {nch} chunks of whole Q-blocks")
    C = n // nch
    q, k, v, do = workloads.make_tensors(w, device="cuda")
    vec = workloads.mask_tensors(w, device="cuda")
    # chunk loads: the forward tile costs of the chunk's Q-blocks, summed over the batch
    bq, bk = fm.tile_shape(fm.OP_FWD)
    t = fm.classify_tiles(*vec, bq, bk)
    qc = t["q_count"].cpu().numpy().astype(np.int64)          # [B][nQB][2]
    cost = (11 * qc[..., 0] + 10 * qc[..., 1]).sum(axis=0)     # [nQB]
    wchunk = cost.reshape(nch, C // bq).sum(axis=1)
    plans = {"contiguous": [list(range(r * kappa, (r + 1) * kappa)) for r in range(P)]}
    owner, rep = fm.ipo_balance(wchunk, P, 3)
    plans["ipo"] = [[int(c) for c in np.nonzero(owner == r)[0]] for r in range(P)]
    A_all = attended_pairs(w)
    out = {"measure": f"context parallelism over {P} ranks emulated on one GPU",
           "config": {"workload": workload, "ranks": P, "chunks": nch, "chunk_rows": C,
                      "steps": steps, "warmup": warmup},
           "ipo_report": {k_: (int(v_) if not isinstance(v_, bool) else v_)
                          for k_, v_ in rep.items()}, "plans": {}}
    for name, plan in plans.items():
        ranks = []
        for r, chunks in enumerate(plan):
            offs = [c * C for c in sorted(chunks)]
            rows = torch.cat([torch.arange(o, o + C, device="cuda") for o in offs])
            qr, dor = q[:, :, rows].contiguous(), do[:, :, rows].contiguous()
            lv = fm.localize_mask(*vec, torch.tensor(offs, dtype=torch.int32, device="cuda"), C)
            o = torch.empty_like(qr)
            lse = torch.empty((w.batch, w.heads_q, qr.shape[2]), dtype=torch.float32,
                              device="cuda")
            grads = (torch.empty_like(qr), torch.empty_like(k), torch.empty_like(v))
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            for i in range(warmup + steps):
                e = ev[i - warmup] if i >= warmup else None
                if e:
                    e[0].record()
                fm.attn_fwd(qr, k, v, *lv, out=o, lse=lse)
                fm.attn_bwd(qr, k, v, o, lse, dor, *lv, grads=grads)
                if e:
                    e[1].record()
            torch.cuda.synchronize()
            ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
            lw = workloads.Workload(w.name, w.batch, w.heads_q, w.heads_kv, qr.shape[2],
                                    w.head_dim, *[x.cpu().numpy() for x in lv], w.seed)
            pairs = attended_pairs(lw)  # N_q local rows, vectors over all N_k keys
            ranks.append({"rank": r, "chunks": sorted(chunks), "ms": round(ms, 3),
                          "load": int(wchunk[sorted(chunks)].sum()),
                          "tflops": round(14 * w.head_dim * pairs / (ms * 1e-3) / 1e12, 1)})
        t_ms = [x["ms"] for x in ranks]
        out["plans"][name] = {
            "ranks": ranks, "max_ms": max(t_ms), "mean_ms": round(float(np.mean(t_ms)), 3),
            "max_over_mean": round(max(t_ms) / float(np.mean(t_ms)), 3),
            "job_tflops_if_parallel": round(14 * w.head_dim * A_all / (max(t_ms) * 1e-3) / 1e12, 1)}
    print(json.dumps(out))


def ipo_table(instances=200, seed=0):
    """fm_ipo_balance on the ablation table's configurations (n, P, kappa, w_max).  The
    page does not give its instance distributions; the stand-ins are: uniform integer
    weights in [1, w_max]; 'causal' chunk i carrying (i + 1) steps of ceil(w_max / n)
    plus a uniform jitter below one step (the load of a causal query chunk grows with
    its position).  Host code: no GPU is touched."""
    import random
    import mask_aware_sparse_amd as fm
    rng = random.Random(seed)
    cfgs = [("uniform", 64, 16, 4, 1000), ("uniform_wide", 64, 16, 4, 10**4),
            ("causal", 64, 8, 8, 200), ("uniform_128", 128, 16, 8, 200)]
    out = []
    for name, n, P, kappa, wmax in cfgs:
        rows = []
        for _ in range(instances if n == 64 else instances // 2):
            if name == "causal":
                step = -(-wmax // n)
                w = [(i + 1) * step + rng.randrange(step) for i in range(n)]
            else:
                w = [rng.randint(1, wmax) for _ in range(n)]
            t0 = time.perf_counter()
            _, r = fm.ipo_balance(w, P, 3)
            dt = time.perf_counter() - t0
            rows.append((r["lpt"] > r["lb"], r["p2"] > r["lb"], r["final"] > r["lb"],
                         (r["lpt"] - r["lb"]) / r["lb"], (r["p2"] - r["lb"]) / r["lb"],
                         (r["final"] - r["lb"]) / r["lb"], dt))
        a = np.array(rows, dtype=float)
        out.append({"config": {"name": name, "n": n, "P": P, "kappa": kappa, "w_max": wmax,
                               "instances": len(rows)},
                    "above_lb": {"lpt": a[:, 0].mean(), "p2": a[:, 1].mean(),
                                 "p2_p3": a[:, 2].mean()},
                    "mean_gap_pct": {"lpt": 100 * a[:, 3].mean(), "p2": 100 * a[:, 4].mean(),
                                     "p2_p3": 100 * a[:, 5].mean()},
                    "ms_per_instance": {"mean": 1e3 * a[:, 6].mean(), "max": 1e3 * a[:, 6].max()}})
    print(json.dumps({"measure": "HCC-IPO stage 1 (host) on the IPO ablation configurations",
                      "results": out}))


def measure_alpha(steps, warmup, n=8192, heads=64):
    """Per-kernel time of all-partial vs all-unmasked tiles on identical work (MQA,
    B = 1, the given N and query heads).  Also checks that both give bit-identical
    outputs, since nothing is hidden in either."""
    import torch
    import mask_aware_sparse_amd as fm
    runs = {}
    outs = {}
    for tag, w in (("unmasked", workloads.full_attention(n, heads_q=heads)),
                   ("partial", workloads.full_attention_partial_tiles(n, heads_q=heads))):
        q, k, v, do = workloads.make_tensors(w, seed=0, device="cuda")
        vec = workloads.mask_tensors(w, device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty((1, heads, n), dtype=torch.float32, device="cuda")
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        ws_f = torch.empty(fm.workspace_size(1, heads, 1, n, fm.OP_FWD), dtype=torch.uint8,
                           device="cuda")
        ws_b = torch.empty(fm.workspace_size(1, heads, 1, n, fm.OP_BWD), dtype=torch.uint8,
                           device="cuda")
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
        for i in range(warmup + steps):
            e = ev[i - warmup] if i >= warmup else None
            fm.attn_fwd(q, k, v, *vec, ws=ws_f, out=o, lse=lse,
                        events=None if e is None else (e[0], e[1]))
            fm.attn_bwd(q, k, v, o, lse, do, *vec, ws=ws_b, grads=grads,
                        events=None if e is None else (e[2], e[3], e[4], e[5]))
        torch.cuda.synchronize()
        runs[tag] = {kname: float(np.median([e[a].elapsed_time(e[b]) for e in ev]))
                     for kname, a, b in (("k_attn_fwd", 0, 1), ("k_attn_bwd_dkdv", 2, 3),
                                         ("k_attn_bwd_dq", 4, 5))}
        outs[tag] = (o.clone(), lse.clone()) + tuple(g.clone() for g in grads)
    # O, LSE, dQ are written once per element; dK/dV of MQA groups are summed with fp32
    # atomics in arbitrary order, so only their difference is reported
    same = all(torch.equal(a, b) for a, b in zip(outs["unmasked"][:3], outs["partial"][:3]))
    dkdv_diff = max(float((a.float() - b.float()).abs().max())
                    for a, b in zip(outs["unmasked"][3:], outs["partial"][3:]))
    ratio = {kname: round(runs["partial"][kname] / runs["unmasked"][kname], 4)
             for kname in runs["unmasked"]}
    print(json.dumps({"measure": "alpha_p / alpha_u (partial vs unmasked tile time)",
                      "config": {"batch": 1, "heads_q": heads, "heads_kv": 1, "seq_len": n,
                                 "head_dim": 128, "steps": steps, "warmup": warmup},
                      "ms_median": runs, "ratio": ratio, "o_lse_dq_bit_identical": same,
                      "dk_dv_max_abs_diff": dkdv_diff}))


CPU_SAMPLE_ROWS = 8192


def cpu_baseline(w, q, k, v, do, budget_s):
    """Time the fp64 oracle on a bounded sample of the same workload, until the budget is
    spent: whole (b, h) problems for the multi-interval and block forms; for the
    four-vector form, units of at most CPU_SAMPLE_ROWS query rows of one (b, h) against
    every key (the rows' vectors renumbered into the unit's rows, as one context-parallel
    rank's share), taken b = 0.., h = 0.., row chunks in a seeded order so that one long
    head does not exceed the budget.  Reported in the metric's unit over the sample's
    attended pairs."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count()
    g = w.heads_q // w.heads_kv
    n = w.seqlen
    four = not isinstance(w, (workloads.BlockWorkload, workloads.MultiWorkload))
    chunk = min(n, CPU_SAMPLE_ROWS) if four else n
    n_chunks = -(-n // chunk)
    chunk_order = np.random.default_rng(0).permutation(n_chunks)
    units, rows, pairs, t_total = 0, 0, 0, 0.0
    f = lambda t, b, hh, r0=0, r1=None: \
        t[b:b + 1, hh:hh + 1, r0:r1].float().cpu().numpy().astype(np.float64)
    for b in range(w.batch):
        for h in range(w.heads_q):
            kvh = h // g
            for c in (chunk_order if four else [0]):
                r0, r1 = int(c) * chunk, min(int(c) * chunk + chunk, n)
                if isinstance(w, workloads.BlockWorkload):
                    m = h // (w.heads_q // w.mask_heads)
                    grid = w.blocks[b:b + 1] if w.blocks.ndim == 3 else w.blocks[b:b + 1, m]
                    args = (f(q, b, h), f(k, b, kvh), f(v, b, kvh), f(do, b, h))
                    t0 = time.perf_counter()
                    oracle.attention_fwd_bwd_blocks(*args, grid)
                    t_total += time.perf_counter() - t0
                    one = workloads.BlockWorkload(w.name, 1, 1, 1, n, w.head_dim,
                                                  np.ascontiguousarray(grid), w.seed)
                    pairs += attended_pairs_blocks(one)
                elif isinstance(w, workloads.MultiWorkload):
                    m = h // (w.heads_q // w.mask_heads)
                    st, en = ((x[b:b + 1] if x.ndim == 3 else x[b:b + 1, m])
                              for x in w.intervals())
                    args = (f(q, b, h), f(k, b, kvh), f(v, b, kvh), f(do, b, h))
                    t0 = time.perf_counter()
                    oracle.attention_fwd_bwd_multi(*args, st, en)
                    t_total += time.perf_counter() - t0
                    one = workloads.MultiWorkload(w.name, 1, 1, 1, n, w.head_dim,
                                                  st.copy(), en.copy(), w.seed)
                    pairs += attended_pairs_multi(one)
                else:
                    sub = head_vectors(w, b, h)
                    local = oracle.localize_vectors(sub, [r0], r1 - r0)
                    args = (f(q, b, h, r0, r1), f(k, b, kvh), f(v, b, kvh), f(do, b, h, r0, r1))
                    t0 = time.perf_counter()
                    oracle.attention_fwd_bwd(*args, *local)
                    t_total += time.perf_counter() - t0
                    one = workloads.Workload(w.name, 1, 1, 1, r1 - r0, w.head_dim,
                                             *[np.ascontiguousarray(x) for x in local], w.seed)
                    pairs += attended_pairs(one)
                units += 1
                rows += r1 - r0
                if t_total >= budget_s:
                    break
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    flop = 14 * w.head_dim * pairs
    what = (f"{units} units of <= {chunk} query rows of one (b,h) ({rows} rows of "
            f"{w.batch * w.heads_q * n})" if four else
            f"{units} of {w.batch * w.heads_q} (b,h) problems")
    return {"value": flop / t_total / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{what} of {w.name}, fp64 numpy fwd+bwd, {t_total:.1f} s"}


class ClockSampler:
    """The GFX clock (MHz) sampled by amdsmi every `period` seconds in a thread, between
    start() and stop(); mean() is None where amdsmi is unavailable."""

    def __init__(self, period=0.02):
        import threading
        self.period, self.samples, self._stop = period, [], threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            self._read()
        except Exception:
            self._smi = None

    def _read(self):
        return float(self._smi.amdsmi_get_clock_info(self._h, self._smi.AmdSmiClkType.GFX)["clk"])

    def _loop(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception:
                return
            self._stop.wait(self.period)

    def start(self):
        import threading
        if self._smi is not None:
            self._thread = threading.Thread(target=self._loop, daemon=True)
            self._thread.start()

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        if self._smi is not None:
            try:
                self._smi.amdsmi_shut_down()
            except Exception:
                pass

    # below this many samples (0.2 s of timed steps at the default period) the readings
    # catch the clock ramping up or idle between launches and say nothing of the kernels'
    MIN_SAMPLES = 10

    def mean(self):
        """Mean of the samples, or None with fewer than MIN_SAMPLES of them."""
        return float(np.mean(self.samples)) if len(self.samples) >= self.MIN_SAMPLES else None


def run_workload(name, seed, steps, warmup, key_order_opt, schedule, clock=None, graph=False):
    """Time `steps` fwd+bwd steps of workload `name` after `warmup` untimed ones.  Returns a
    dict of the figures and the input tensors (for the CPU baseline).  With `graph`, the
    timed steps are replays of one HIP graph holding a whole step (both calls: every
    classification, sort and attention kernel), captured after the eager steps, which still
    give the per-kernel times; the eager wall time per step is reported beside it."""
    import torch
    import mask_aware_sparse_amd as fm

    dev = "cuda"
    w = workloads.make_workload(name, seed)
    q, k, v, do = workloads.make_tensors(w, device=dev)
    vec = workloads.mask_tensors(w, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.batch, w.heads_q, w.seqlen), dtype=torch.float32, device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    multi = isinstance(w, workloads.MultiWorkload)
    blocks = isinstance(w, workloads.BlockWorkload)
    sorted_keys = (key_order_opt == "sorted" or
                   (key_order_opt == "auto" and name in SORTED_KEY_WORKLOADS))
    if sorted_keys and (multi or blocks):
        sys.exit("bench.py: --key-order sorted applies to four-vector masks only")
    key_order = fm.KEYS_SORTED if sorted_keys else fm.KEYS_NATURAL
    sched = fm.SCHEDULE_NATURAL if schedule == "natural" else fm.SCHEDULE_LPT
    ws_f = torch.empty(fm.workspace_size(w.batch, w.heads_q, w.heads_kv, w.seqlen, fm.OP_FWD,
                                         head_dim=w.head_dim, mask_heads=w.mask_heads,
                                         key_order=key_order),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(fm.workspace_size(w.batch, w.heads_q, w.heads_kv, w.seqlen, fm.OP_BWD,
                                         head_dim=w.head_dim, mask_heads=w.mask_heads,
                                         key_order=key_order),
                       dtype=torch.uint8, device=dev)
    A = attended_pairs_blocks(w) if blocks else (attended_pairs_multi(w) if multi
                                                 else attended_pairs(w))
    d = w.head_dim
    attn_fwd = fm.attn_fwd_blocks if blocks else (fm.attn_fwd_multi if multi else fm.attn_fwd)
    attn_bwd = fm.attn_bwd_blocks if blocks else (fm.attn_bwd_multi if multi else fm.attn_bwd)
    opt = {"schedule": sched}
    if not (multi or blocks):
        opt["key_order"] = key_order

    # per instrumented step: 0 start, 1/2 fwd kernel, 8 between the calls, 3/4 dK/dV
    # kernel, 6/7 dQ kernel, 5 end (all on the current stream, which the library launches
    # on).  Every other timed step is instrumented: a timing event costs the stream some
    # tens of microseconds, which would otherwise be charged to every step's wall time.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(9)]
          for _ in range((steps + 1) // 2)]

    def step(e=None):
        if e is not None:
            e[0].record()
        attn_fwd(q, k, v, *vec, ws=ws_f, out=o, lse=lse,
                 events=None if e is None else (e[1], e[2]), **opt)
        if e is not None:
            e[8].record()
        attn_bwd(q, k, v, o, lse, do, *vec, ws=ws_b, grads=grads,
                 events=None if e is None else (e[3], e[4], e[6], e[7]), **opt)
        if e is not None:
            e[5].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if clock is not None and not graph:
        clock.start()
    t0 = time.perf_counter()
    for i in range(steps):
        step(ev[i // 2] if i % 2 == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eager_ms = wall * 1e3 / steps
    if graph:
        # the library allocates nothing, issues no memset and never synchronizes inside a
        # call, so one step captures whole (the same buffers, replayed on the same stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        if clock is not None:
            clock.start()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    if clock is not None:
        clock.stop()

    el = lambda a, b: np.array([e[a].elapsed_time(e[b]) for e in ev])
    step_ms, call_fwd_ms, call_bwd_ms = el(0, 5), el(0, 8), el(8, 5)
    fwd_ms, dkdv_ms, dq_ms = el(1, 2), el(3, 4), el(6, 7)
    ms = wall * 1e3 / steps
    value = 14 * d * A / (ms * 1e-3) / 1e12
    # algorithmic flop per attended pair of each attention kernel: forward 4d (QK, PV);
    # dK/dV kernel 8d (S and dP recomputed once for the backward, dV, dK); dQ kernel 2d
    # (its second recomputation of S and dP is not algorithmic work)
    kernels = {
        "k_attn_fwd": (float(fwd_ms.mean()), 4 * d * A),
        "k_attn_bwd_dkdv": (float(dkdv_ms.mean()), 8 * d * A),
        "k_attn_bwd_dq": (float(dq_ms.mean()), 2 * d * A),
    }
    tflops = {kname: f / (t * 1e-3) / 1e12 for kname, (t, f) in kernels.items()}
    dom = max(kernels, key=lambda kname: kernels[kname][0])
    config = {"workload": name, "batch": w.batch, "heads_q": w.heads_q,
              "heads_kv": w.heads_kv, "mask_heads": w.mask_heads,
              "mask_intervals": w.n_intervals if multi else None,
              "mask_blocks": "128x128" if blocks else None, "seq_len": w.seqlen,
              "head_dim": d, "attended_pairs": A, "seed": seed,
              "key_order": "sorted" if sorted_keys else "natural", "schedule": schedule,
              "launch": "hip_graph" if graph else "eager"}
    return {
        "w": w, "tensors": (q, k, v, do), "value": value, "ms": ms, "config": config,
        "kernels": {kname: {"ms": round(t, 4), "algorithmic_tflops": round(tflops[kname], 2)}
                    for kname, (t, _) in kernels.items()},
        "event_ms_per_step": round(float(step_ms.mean()), 4),
        "eager_ms_per_step": round(eager_ms, 4),
        # whole calls, classification and LPT sort included: 4d*A / t_fwd and 10d*A / t_bwd
        "fwd": {"ms": round(float(call_fwd_ms.mean()), 4),
                "tflops": round(4 * d * A / (call_fwd_ms.mean() * 1e-3) / 1e12, 2)},
        "bwd": {"ms": round(float(call_bwd_ms.mean()), 4),
                "tflops": round(10 * d * A / (call_bwd_ms.mean() * 1e-3) / 1e12, 2)},
        "roofline": {"kernel": dom, "bound": "mfma",
                     "achieved": round(tflops[dom], 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops[dom] / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": stored_traffic(dom, name + ("_sorted_keys" if sorted_keys
                                                            else ""))},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=workloads.CONFIG_NAMES + workloads.VARIANT_NAMES)
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads timed after the headline one (default: "
                         "c3 and c4 with the default workload, none otherwise; '' for none)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the cpu_baseline sample (0 = skip)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run only a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--classify-bandwidth", action="store_true",
                    help="time fm_classify_tiles on replicated c5 vectors (HBM roofline)")
    ap.add_argument("--classify-batch", type=int, default=4,
                    help="batch rows of the replicated c5 vectors for --classify-bandwidth")
    ap.add_argument("--cp", type=int, default=0, metavar="P",
                    help="emulate context parallelism over P ranks (query shares in turn)")
    ap.add_argument("--ipo-table", action="store_true",
                    help="host chunk balancer on the IPO ablation configurations")
    ap.add_argument("--measure-alpha", action="store_true",
                    help="time partial against unmasked tiles on identical work")
    ap.add_argument("--key-order", choices=["auto", "natural", "sorted"], default="auto",
                    help="key order of the four-vector entry points (auto: sorted for the "
                         "random-eviction workload, natural otherwise)")
    ap.add_argument("--schedule", choices=["lpt", "natural"], default="lpt",
                    help="dispatch order of the attention kernels' work items")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one HIP graph holding a whole step (launch gaps "
                         "removed; per-kernel times still come from eager steps)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: the benchmark runs on one GPU only; multi-GPU runs are not supported",
              file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy > 0:
        calibrate_copy(args.calibrate_copy)
        return
    if args.measure_alpha:
        measure_alpha(args.steps, args.warmup)
        return
    if args.ipo_table:
        ipo_table()
        return
    if args.cp > 0:
        cp_emulation(args.workload, args.cp, min(args.steps, 3), min(args.warmup, 1))
        return
    if args.classify_bandwidth:
        classify_bandwidth(args.steps, args.warmup, batch=args.classify_batch)
        return

    import torch

    if args.also is None:
        also = list(ALSO_WORKLOADS) if args.workload == DEFAULT_WORKLOAD else []
    else:
        also = [x for x in args.also.split(",") if x]
    clock = ClockSampler()
    r = run_workload(args.workload, args.seed, args.steps, args.warmup, args.key_order,
                     args.schedule, clock, graph=args.graph)
    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_baseline(r["w"], *r["tensors"], args.cpu_budget)
    r["tensors"] = None
    torch.cuda.empty_cache()
    cu = int(torch.cuda.get_device_properties(0).multi_processor_count)
    mhz = clock.mean()
    peak_at_clock = cu * MFMA_BF16_FLOP_PER_CLK_CU * mhz * 1e6 / 1e12 if mhz else None
    extra = {}
    for name in also:
        x = run_workload(name, args.seed, args.steps, args.warmup, args.key_order,
                         args.schedule, graph=args.graph)
        x["tensors"] = None
        torch.cuda.empty_cache()
        extra[name] = {"value": round(x["value"], 3), "unit": "TFLOP/s",
                       "ms_per_step": round(x["ms"], 4),
                       "eager_ms_per_step": x["eager_ms_per_step"],
                       "pct_mfma_peak": round(100 * x["value"] / MFMA_BF16_PEAK_TFLOPS, 2),
                       "key_order": x["config"]["key_order"], "kernels": x["kernels"],
                       "fwd": x["fwd"], "bwd": x["bwd"],
                       "roofline": {k_: x["roofline"][k_] for k_ in ("kernel", "achieved", "frac",
                                                                     "traffic")}}
    out = {
        "metric": "effective TFLOP/s (attended pairs only) fwd+bwd, bf16 d=128; % MFMA peak",
        "value": round(r["value"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": r["config"],
        "pct_mfma_peak": round(100 * r["value"] / MFMA_BF16_PEAK_TFLOPS, 2),
        "device": {"compute_units": cu, "gfx_clock_mhz_mean": round(mhz, 1) if mhz else None,
                   "clock_samples": len(clock.samples),
                   "mfma_bf16_peak_at_clock_tflops": round(peak_at_clock, 1)
                   if peak_at_clock else None,
                   "pct_mfma_peak_at_clock": round(100 * r["value"] / peak_at_clock, 2)
                   if peak_at_clock else None},
        "kernels": r["kernels"],
        "event_ms_per_step": r["event_ms_per_step"],
        "eager_ms_per_step": r["eager_ms_per_step"],
        "fwd": r["fwd"],
        "bwd": r["bwd"],
        "roofline": r["roofline"],
        "cpu_baseline": cpu,
        "also": extra,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
