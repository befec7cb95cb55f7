"""Masked softmax attention, forward and analytic backward, in float64 (oracle).

Test infrastructure only.  What is computed (the method reaches exactly this, up
to rounding order, because skipped tiles are fully hidden and contribute 0):

  S = scale * Q K^T with S_ij = -inf where the column mask hides (i, j)
  (FlashMask Guide, dense additive-mask formula S = QK^T/sqrt(d) + M);
  O = softmax(S) V, computed here as the plain two-pass softmax (row max, then
  exp and sum), not the online form, so that the GPU's online form is checked
  against it (Flash MSA guide, "Why Standard Attention Broke" and "The Flash
  Core"); LSE_i = m_i + ln l_i, the statistics the forward keeps for the backward
  (same guide, "The Backward Pass").

  Backward by the chain rule (Flash MSA guide, "The Backward Pass"; the page drops
  the softmax scale in dQ and dK, restored here):
  P_ij = exp(S_ij - LSE_i); dV = P^T dO; dP = dO V^T;
  D_i = sum_j P_ij dP_ij; dS = P o (dP - D); dQ = scale dS K; dK = scale dS^T Q.

Readings: a row whose every key is hidden gets O = 0, LSE = -inf, dQ = 0 and adds
nothing to dK/dV.  Query head h uses kv head h // (H_q / H_kv) (GQA: K/V heads are
shared by contiguous groups of query heads, Flash MSA guide FAQ).  dK/dV of a kv
head sum over the query heads of its group.

Mask vectors are one set per batch row, [B][N_k], shared by every head (FlashMask-3
page, Overview), or -- the per-head variant its list of extensions names without
defining -- [B][H_m][N_k] with H_m dividing H_q, where query head h uses set
h // (H_q / H_m) (contiguous groups, as for GQA; H_m = H_q is one set per head).

The multi-interval form (FlashMask Guide, "Multi-Interval Sparse Masks"; the *_multi
functions) gives each column M <= 4 active intervals instead: starts and ends
[B][M][N_k] or [B][H_m][M][N_k], row i seeing key j iff some interval holds it.

Rows are processed in blocks; each block expands only its own rows of the mask
(never the full N x N matrix) and restricts its products to the columns that at
least one of its rows can see, which is exact because hidden columns contribute 0.
"""
import numpy as np

from .mask import hidden_block_rows, hidden_multi_rows, masked_rows


class _FourVectors:
    """The four-vector form of one (b, h): hidden iff in [LTS, LTE) or [UTS, UTE)."""

    def __init__(self, vecs):
        self.v = vecs

    def rows(self, r0, r1):
        return masked_rows(*self.v, r0, r1)

    def column(self, c, n):
        return masked_rows(*(x[c:c + 1] for x in self.v), 0, n)[:, 0]


class _Intervals:
    """The multi-interval form of one (b, h): visible iff in some [start_m, end_m)."""

    def __init__(self, starts, ends):
        self.s, self.e = starts, ends

    def rows(self, r0, r1):
        return hidden_multi_rows(self.s, self.e, r0, r1)

    def column(self, c, n):
        return hidden_multi_rows(self.s[:, c:c + 1], self.e[:, c:c + 1], 0, n)[:, 0]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _scale(d, scale):
    return 1.0 / np.sqrt(d) if scale is None or scale <= 0 else float(scale)


class _Blocks:
    """The block-sparse form of one (b, h): visible iff its 128 x 128 block is."""

    def __init__(self, blocks, nk):
        self.blk, self.nk = blocks, nk

    def rows(self, r0, r1):
        return hidden_block_rows(self.blk, r0, r1, self.nk)

    def column(self, c, n):
        return hidden_block_rows(self.blk, 0, n, self.nk)[:, c]


def _row_block(qh, kh, vh, mask, r0, r1, scale, dOh=None):
    """Forward (and, if dOh is given, backward) for rows [r0, r1) of one (b, h) whose
    mask is `mask` (_FourVectors or _Intervals).

    Returns O [R][d], LSE [R], and if dOh: dQ [R][d], cols, dK_part, dV_part where
    the parts are [len(cols)][d] contributions to the key columns `cols`."""
    hid = mask.rows(r0, r1)                                   # [R][N]
    cols = np.nonzero(~hid.all(axis=0))[0]
    R, d = r1 - r0, qh.shape[1]
    O = np.zeros((R, d))
    lse = np.full(R, -np.inf)
    if dOh is not None:
        dQ = np.zeros((R, d))
        empty = np.zeros((0, d))
    if cols.size == 0:
        if dOh is None:
            return O, lse
        return O, lse, dQ, cols, empty, empty
    q = qh[r0:r1]
    k = kh[cols]
    v = vh[cols]
    h = hid[:, cols]
    S = scale * (q @ k.T)
    S[h] = -np.inf
    m = S.max(axis=1)                                          # -inf for all-hidden rows
    live = np.isfinite(m)
    e = np.zeros_like(S)
    e[live] = np.exp(S[live] - m[live, None])                  # exp(-inf) = 0 where hidden
    l = e.sum(axis=1)
    O[live] = (e[live] / l[live, None]) @ v
    lse[live] = m[live] + np.log(l[live])
    if dOh is None:
        return O, lse
    do = dOh[r0:r1]
    P = np.zeros_like(S)
    P[live] = np.exp(S[live] - lse[live, None])
    dP = do @ v.T
    D = (P * dP).sum(axis=1)
    dS = P * (dP - D[:, None])
    dQ = scale * (dS @ k)
    dK_part = scale * (dS.T @ q)
    dV_part = P.T @ do
    return O, lse, dQ, cols, dK_part, dV_part


def _check(q, k, v):
    """Q [B][H_q][N_q][d], K and V [B][H_kv][N_k][d]; N_q = N_k for self-attention,
    N_q < N_k for one rank's share of the query rows under context parallelism with
    localized vectors.  Returns (B, H_q, H_kv, N_q, d, g)."""
    B, Hq, N, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    assert (B, d) == (Bk, dk) and v.shape == k.shape
    assert Hq % Hkv == 0
    return B, Hq, Hkv, N, d, Hq // Hkv


def _vectors_of(vecs, B, Hq, Nk):
    """Mask getter (b, h) -> _FourVectors for vectors [B][N_k] or [B][H_m][N_k] (row
    bounds in [0, N_q])."""
    arrs = [np.asarray(x) for x in vecs]
    shape = arrs[0].shape
    assert all(x.shape == shape for x in arrs)
    if len(shape) == 2:
        assert shape == (B, Nk)
        return lambda b, h: _FourVectors(tuple(x[b] for x in arrs))
    assert len(shape) == 3 and shape[0] == B and shape[2] == Nk and Hq % shape[1] == 0
    per = Hq // shape[1]                      # query heads per mask head
    return lambda b, h: _FourVectors(tuple(x[b, h // per] for x in arrs))


def _intervals_of(starts, ends, B, Hq, Nk):
    """Mask getter (b, h) -> _Intervals for starts/ends [B][M][N_k] or [B][H_m][M][N_k]."""
    s, e = np.asarray(starts), np.asarray(ends)
    assert s.shape == e.shape and s.shape[-1] == Nk and s.shape[0] == B
    if s.ndim == 3:
        assert 1 <= s.shape[1] <= 4
        return lambda b, h: _Intervals(s[b], e[b])
    assert s.ndim == 4 and Hq % s.shape[1] == 0 and 1 <= s.shape[2] <= 4
    per = Hq // s.shape[1]
    return lambda b, h: _Intervals(s[b, h // per], e[b, h // per])


def _fwd(q, k, v, mask_of, scale, row_block):
    B, Hq, Hkv, N, d, g = _check(q, k, v)
    sc = _scale(d, scale)
    O = np.zeros((B, Hq, N, d))
    LSE = np.full((B, Hq, N), -np.inf)
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            mk = mask_of(b, h)
            for r0 in range(0, N, row_block):
                r1 = min(r0 + row_block, N)
                O[b, h, r0:r1], LSE[b, h, r0:r1] = _row_block(q[b, h], k[b, kv], v[b, kv],
                                                              mk, r0, r1, sc)
    return O, LSE


def _fwd_bwd(q, k, v, do, mask_of, scale, row_block):
    B, Hq, Hkv, N, d, g = _check(q, k, v)
    sc = _scale(d, scale)
    O = np.zeros((B, Hq, N, d))
    LSE = np.full((B, Hq, N), -np.inf)
    dQ = np.zeros((B, Hq, N, d))
    dK = np.zeros((B, Hkv, k.shape[2], d))
    dV = np.zeros((B, Hkv, k.shape[2], d))
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            mk = mask_of(b, h)
            for r0 in range(0, N, row_block):
                r1 = min(r0 + row_block, N)
                o, lse, dq, cols, dkp, dvp = _row_block(q[b, h], k[b, kv], v[b, kv], mk,
                                                        r0, r1, sc, dOh=do[b, h])
                O[b, h, r0:r1], LSE[b, h, r0:r1], dQ[b, h, r0:r1] = o, lse, dq
                dK[b, kv, cols] += dkp
                dV[b, kv, cols] += dvp
    return O, LSE, dQ, dK, dV


def _rows(q, k, v, do, mk, b, h, rows, scale):
    Hq, Hkv = q.shape[1], k.shape[1]
    kv = h // (Hq // Hkv)
    d = q.shape[3]
    sc = _scale(d, scale)
    qh, kh, vh = _f64(q[b, h]), _f64(k[b, kv]), _f64(v[b, kv])
    dOh = None if do is None else _f64(do[b, h])
    O = np.zeros((len(rows), d)); LSE = np.zeros(len(rows)); dQ = np.zeros((len(rows), d))
    for t, r in enumerate(rows):
        res = _row_block(qh, kh, vh, mk, int(r), int(r) + 1, sc, dOh=dOh)
        O[t], LSE[t] = res[0][0], res[1][0]
        if dOh is not None:
            dQ[t] = res[2][0]
    return O, LSE, (dQ if dOh is not None else None)


def _cols(q, k, v, do, mask_of, b, kv, cols, scale, row_block):
    Hq, Hkv = q.shape[1], k.shape[1]
    g = Hq // Hkv
    d = q.shape[3]
    sc = _scale(d, scale)
    N = q.shape[2]
    cols = np.asarray(cols)
    kh, vh = _f64(k[b, kv]), _f64(v[b, kv])
    dK = np.zeros((len(cols), d)); dV = np.zeros((len(cols), d))
    for h in range(kv * g, (kv + 1) * g):
        mk = mask_of(b, h)
        # rows that see at least one selected column
        need = np.zeros(N, dtype=bool)
        for c in cols:
            need |= ~mk.column(int(c), N)
        # Rows that see none of the selected columns contribute exactly 0 to them, so
        # whole row blocks that contain at least one needed row can be computed.
        starts = sorted({int(r) // row_block * row_block for r in np.nonzero(need)[0]})
        qh, dOh = _f64(q[b, h]), _f64(do[b, h])
        for r0 in starts:
            r1 = min(r0 + row_block, N)
            _, _, _, cs, dkp, dvp = _row_block(qh, kh, vh, mk, r0, r1, sc, dOh=dOh)
            where = np.searchsorted(cs, cols)
            hit = (where < len(cs)) & (cs[np.minimum(where, len(cs) - 1)] == cols) \
                if len(cs) else np.zeros(len(cols), dtype=bool)
            dK[hit] += dkp[where[hit]]
            dV[hit] += dvp[where[hit]]
    return dK, dV


# ---- four-vector form (LTS/LTE/UTS/UTE) ----------------------------------------------

def attention_fwd(q, k, v, lts, lte, uts, ute, scale=None, row_block=256):
    """O [B][H_q][N][d] and LSE [B][H_q][N] (natural log) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    of = _vectors_of((lts, lte, uts, ute), q.shape[0], q.shape[1], k.shape[2])
    return _fwd(q, k, v, of, scale, row_block)


def attention_fwd_bwd(q, k, v, do, lts, lte, uts, ute, scale=None, row_block=256):
    """(O, LSE, dQ, dK, dV) in float64; the backward recomputes the softmax from
    its definition (no statistic comes from anywhere but this function)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    of = _vectors_of((lts, lte, uts, ute), q.shape[0], q.shape[1], k.shape[2])
    return _fwd_bwd(q, k, v, do, of, scale, row_block)


def attention_bwd(q, k, v, do, lts, lte, uts, ute, scale=None, row_block=256):
    """(dQ, dK, dV) in float64."""
    _, _, dQ, dK, dV = attention_fwd_bwd(q, k, v, do, lts, lte, uts, ute, scale, row_block)
    return dQ, dK, dV


def attention_rows(q, k, v, do, lts, lte, uts, ute, b, h, rows, scale=None):
    """O, LSE and dQ of selected query rows of one (b, h).  Each row is computed
    on its own from the full key axis, so any row of a full-size problem can be
    checked.  `do` may be None (then dQ is None)."""
    mk = _vectors_of((lts, lte, uts, ute), q.shape[0], q.shape[1], k.shape[2])(b, h)
    return _rows(q, k, v, do, mk, b, h, rows, scale)


def attention_cols(q, k, v, do, lts, lte, uts, ute, b, kv, cols, scale=None, row_block=256):
    """dK and dV of selected key columns of one (b, kv head).  Every query row of
    the group that sees any selected column is computed in full (its softmax needs
    the whole row), so this is cheap only where the selected columns are seen by
    few rows."""
    of = _vectors_of((lts, lte, uts, ute), q.shape[0], q.shape[1], k.shape[2])
    return _cols(q, k, v, do, of, b, kv, cols, scale, row_block)


def _blocks_of(blocks, B, Hq, Nq, Nk):
    """Mask getter (b, h) -> _Blocks for a block grid [B][nQB][nKB] or [B][H_m][nQB][nKB]
    (nQB = ceil(N_q / 128), nKB = ceil(N_k / 128))."""
    from .mask import BLOCK
    g = np.asarray(blocks)
    nqb, nkb = -(-Nq // BLOCK), -(-Nk // BLOCK)
    if g.ndim == 3:
        assert g.shape == (B, nqb, nkb)
        return lambda b, h: _Blocks(g[b], Nk)
    assert g.ndim == 4 and g.shape[0] == B and g.shape[2:] == (nqb, nkb) and Hq % g.shape[1] == 0
    per = Hq // g.shape[1]
    return lambda b, h: _Blocks(g[b, h // per], Nk)


# ---- block-sparse form (blocks [B][nQB][nKB] or [B][H_m][nQB][nKB], 128 x 128 blocks) -----

def attention_fwd_blocks(q, k, v, blocks, scale=None, row_block=256):
    q, k, v = _f64(q), _f64(k), _f64(v)
    of = _blocks_of(blocks, q.shape[0], q.shape[1], q.shape[2], k.shape[2])
    return _fwd(q, k, v, of, scale, row_block)


def attention_fwd_bwd_blocks(q, k, v, do, blocks, scale=None, row_block=256):
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    of = _blocks_of(blocks, q.shape[0], q.shape[1], q.shape[2], k.shape[2])
    return _fwd_bwd(q, k, v, do, of, scale, row_block)


def attention_rows_blocks(q, k, v, do, blocks, b, h, rows, scale=None):
    mk = _blocks_of(blocks, q.shape[0], q.shape[1], q.shape[2], k.shape[2])(b, h)
    return _rows(q, k, v, do, mk, b, h, rows, scale)


def attention_cols_blocks(q, k, v, do, blocks, b, kv, cols, scale=None, row_block=256):
    of = _blocks_of(blocks, q.shape[0], q.shape[1], q.shape[2], k.shape[2])
    return _cols(q, k, v, do, of, b, kv, cols, scale, row_block)


# ---- multi-interval form (starts/ends [B][M][N_k] or [B][H_m][M][N_k]) -------------------

def attention_fwd_multi(q, k, v, starts, ends, scale=None, row_block=256):
    q, k, v = _f64(q), _f64(k), _f64(v)
    of = _intervals_of(starts, ends, q.shape[0], q.shape[1], k.shape[2])
    return _fwd(q, k, v, of, scale, row_block)


def attention_fwd_bwd_multi(q, k, v, do, starts, ends, scale=None, row_block=256):
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    of = _intervals_of(starts, ends, q.shape[0], q.shape[1], k.shape[2])
    return _fwd_bwd(q, k, v, do, of, scale, row_block)


def attention_rows_multi(q, k, v, do, starts, ends, b, h, rows, scale=None):
    mk = _intervals_of(starts, ends, q.shape[0], q.shape[1], k.shape[2])(b, h)
    return _rows(q, k, v, do, mk, b, h, rows, scale)


def attention_cols_multi(q, k, v, do, starts, ends, b, kv, cols, scale=None, row_block=256):
    of = _intervals_of(starts, ends, q.shape[0], q.shape[1], k.shape[2])
    return _cols(q, k, v, do, of, b, kv, cols, scale, row_block)
