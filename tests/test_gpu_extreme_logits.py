"""Forward/backward parity with scores far from zero (|s| * log2(e) up to about 260).

The forward keeps one exponent offset per row and forms p = 2^(s c - offset).  A row
that no key of its first queued tile reaches has no offset when later tiles arrive; it
must take its offset from the first tile in which it sees a key, whatever the
magnitude of its scores there (Flash MSA guide, "The Flash Core": the running row max
starts from the first visible score).  With scores near -255 (log2 units) against an
offset of 0, every p would underflow; with scores near +255 every p would overflow.

Inputs (workloads.extreme_logit_tensors): half of each key row is one shared +-1 pattern,
the other half exact small random values; queries put a factor of +-32 on the shared
half, so every q.k is exact in fp32.  The masks
put rows of diagonal Q-blocks above their first queued tile (queues run right to left) at
the forward's tile for their heads (128 rows, or 32 rows of four packed query heads):
causal documents, share-question packing, prefix-LM documents (also packed) and plain
causal with a ragged tail.  Bars as everywhere: O max-abs 1e-2, LSE max-abs 1e-3 with -inf rows equal,
dQ/dK/dV relative L2 2e-2."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_fwd, check_grads, log, to_np

FWD_BK = 64   # keys per forward tile


def fwd_bq(w):
    """Query rows per forward tile: 32 where four query heads of one kv head and mask set
    share a workgroup (head groups of four), else 128."""
    g, qpm = w.heads_q // w.heads_kv, w.heads_q // max(getattr(w, "mask_heads", 0) or 1, 1)
    return 32 if g % 4 == 0 and qpm % 4 == 0 else 128

MASKS = {
    "causal_doc_1k": lambda: workloads.causal_doc(0, heads_q=2, heads_kv=1),
    "share_question_2k_mqa": lambda: workloads.share_question(0, n=2048, heads_q=2, heads_kv=1,
                                                              prompt_range=(128, 256),
                                                              answer_range=(64, 128)),
    # four query heads per kv head: the forward's packed 32-row tiles, where the rows above
    # a document boundary see nothing of the next document's bidirectional prefix
    "prefix_lm_doc_1k_mqa4_packed": lambda: workloads.prefix_lm_doc(1, n=1024, batch=2,
                                                                    heads_q=4, heads_kv=1,
                                                                    lo=128, hi=512),
    "prefix_lm_doc_1k_gqa": lambda: workloads.prefix_lm_doc(1, n=1024, batch=2, heads_q=4,
                                                            heads_kv=2, lo=128, hi=512),
    "causal_777": lambda: workloads.causal(777, heads_q=2, heads_kv=2),
}
KINDS = ("low", "high", "mixed")


def rows_hidden_in_first_tile(w):
    """Rows that see some key but none of their Q-block's first queued forward tile."""
    bq = fwd_bq(w)
    cls = oracle.classify(*w.vectors(), bq, FWD_BK)
    out = []
    for b in range(w.batch):
        hid = oracle.masked_rows(*(x[b] for x in w.vectors()), 0, w.seqlen)
        for qb in range(cls.shape[1]):
            live = np.nonzero(cls[b, qb])[0]
            if live.size == 0:
                continue
            kb = live.max()                                    # queues run right to left
            r0, r1 = qb * bq, min(qb * bq + bq, w.seqlen)
            k0, k1 = kb * FWD_BK, min(kb * FWD_BK + FWD_BK, w.seqlen)
            sub = hid[r0:r1]
            rows = np.nonzero(sub[:, k0:k1].all(1) & ~sub.all(1))[0] + r0
            out += [(b, int(r)) for r in rows]
    return out


@pytest.mark.parametrize("name", list(MASKS))
def test_masks_exercise_rows_without_first_tile(name):
    """Each mask puts rows that see keys outside their first queued tile (CPU check of
    the inputs, so the GPU cases below test what they mean to)."""
    assert len(rows_hidden_in_first_tile(MASKS[name]())) > 0


def test_extreme_inputs_have_the_stated_scores():
    w = workloads.causal_doc(0, heads_q=2, heads_kv=1)
    c = 1.0 / np.sqrt(128) / np.log(2.0)
    for kind, lo, hi in (("low", -2192, -1904), ("high", 1904, 2192), ("mixed", -2192, 2192)):
        q, k, v, do = workloads.extreme_logit_tensors(w, kind)
        s = to_np(q[0, 1]) @ to_np(k[0, 0]).T
        assert s.min() >= lo and s.max() <= hi, kind
        assert np.array_equal(4 * s, np.round(4 * s))    # multiples of 1/4: exact in fp32
        if kind != "mixed":
            assert abs(s).min() * c > 240                 # |s| log2(e)/sqrt(d) above 240
        # the keys' weights differ: spread of a row's scores of several log2 units
        assert (s.max(1) - s.min(1)).mean() * c > 4


@pytest.mark.gpu
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("name", list(MASKS))
def test_extreme_logits_parity(name, kind):
    import mask_aware_sparse_amd as fm
    w = MASKS[name]()
    log(f"extreme logits {name} kind={kind} N={w.seqlen} B={w.batch} Hq={w.heads_q} "
        f"Hkv={w.heads_kv}")
    q, k, v, do = workloads.extreme_logit_tensors(w, kind, device="cuda")
    vec = workloads.mask_tensors(w, device="cuda")
    O, LSE = fm.attn_fwd(q, k, v, *vec)
    dq, dk, dv = fm.attn_bwd(q, k, v, O, LSE, do, *vec)
    torch.cuda.synchronize()
    O_r, L_r, dQ_r, dK_r, dV_r = oracle.attention_fwd_bwd(*(to_np(t) for t in (q, k, v, do)),
                                                          *w.vectors())
    # rows that see keys never come back as -inf (the -inf sets must coincide)
    fwd = check_fwd(O, LSE, O_r, L_r, ctx=f"{name}/{kind}")
    hidden_first = rows_hidden_in_first_tile(w)
    Lg = to_np(LSE)
    for b, r in hidden_first:
        assert np.isfinite(Lg[b, :, r]).all(), (name, kind, b, r)
    bwd = check_grads(dq, dk, dv, (dQ_r, dK_r, dV_r), L_r, ctx=f"{name}/{kind}")
    log(f"  O/LSE {fwd}, dQ/dK/dV {bwd}, rows outside their first tile: {len(hidden_first)}")
