"""Host-side checks of the C ABI: the library loads, exports every declared entry
point, and rejects bad arguments before launching anything (no GPU needed)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import mask_aware_sparse_amd as fm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fm.h")

FM_OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fm_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = fm.library()
    names = declared_functions()
    assert {"fm_classify_tiles", "fm_attn_fwd", "fm_attn_bwd", "fm_workspace_size",
            "fm_tile_shape", "fm_debug_expand_mask", "fm_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fm.library_path()],
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (fm_\w+)", out))
    assert set(names) <= exported


def prob(B=1, Hq=4, Hkv=2, N=256, d=128, scale=0.0):
    return fm.Problem(B, Hq, Hkv, N, d, scale)


FAKE = ctypes.c_void_p(0x100000)   # never dereferenced: every case fails validation first


def fake_mask():
    return fm.Mask(0x100000, 0x100000, 0x100000, 0x100000)


def fwd(p, ws_bytes=1 << 40, q=FAKE, mask=None):
    m = fake_mask() if mask is None else mask
    return fm.library().fm_attn_fwd(ctypes.byref(p), q, FAKE, FAKE, ctypes.byref(m), FAKE, FAKE,
                                    FAKE, ctypes.c_size_t(ws_bytes), None, None)


def bwd(p, ws_bytes=1 << 40, dq=FAKE):
    m = fake_mask()
    return fm.library().fm_attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    ctypes.byref(m), dq, FAKE, FAKE, FAKE,
                                    ctypes.c_size_t(ws_bytes), None, None)


def test_status_strings():
    for s in (FM_OK, INVALID, UNSUPPORTED, WORKSPACE, -4):
        assert fm.status_string(s).startswith("FM_")


def test_tile_shapes():
    assert fm.tile_shape(fm.OP_FWD) == (128, 64)
    assert fm.tile_shape(fm.OP_BWD) == (32, 128)
    with pytest.raises(fm.FMError):
        fm.tile_shape(fm.OP_CLASSIFY)


def split_plan_bytes(pairs, per, acc):
    """Workspace of the dK/dV split plan: unit tables over pairs + extra units, the split
    pair tables, two counters, and (without fp32 accumulators) 2 x 2 x extra x per partial
    slots of 128 keys x 128 dims (fp32, dK and dV)."""
    al = lambda x: (x + 255) // 256 * 256
    extra = min(512 // per, pairs)
    b = 2 * al((pairs + extra) * 4) + 2 * al(extra * 4) + al(8)
    return b if acc else b + al(2 * 2 * extra * per * 128 * 128 * 4)


def test_workspace_sizes():
    # forward: minmax (16 int32 per block: room for 4 intervals) + queue + counts + cost +
    # order, each 256-byte aligned
    B, N = 2, 1000
    nqb, nkb = 8, 16
    al = lambda x: (x + 255) // 256 * 256
    want = al(B * nkb * 64) + al(B * nqb * nkb * 4) + al(B * nqb * 8) + 2 * al(B * nqb * 4) + \
        al(B * N * 4)                              # + all-zero vectors for block-sparse masks
    assert fm.workspace_size(B, 4, 2, N, fm.OP_FWD) == want
    assert fm.workspace_size(B, 4, 2, N, fm.OP_CLASSIFY, 64, 32) == al(B * 16 * 4) + al(B * 32 * 4)
    # backward: fp32 dK/dV accumulators exist only for query-head groups above 4 heads;
    # without them the split plan keeps fp32 partial slots instead (same Hq, so the same
    # D / LSE buffers; tiles depend on B and N only; 16 pairs of 2 workgroups each)
    with_acc = fm.workspace_size(B, 8, 1, N, fm.OP_BWD)
    without = fm.workspace_size(B, 8, 2, N, fm.OP_BWD)
    assert with_acc - without == 2 * al(B * 1 * N * 128 * 4) + \
        split_plan_bytes(16, 2, True) - split_plan_bytes(16, 2, False)


@pytest.mark.parametrize("bad,code", [
    (dict(Hq=3, Hkv=2), INVALID),
    (dict(Hkv=0), INVALID),
    (dict(N=-1), INVALID),
    (dict(B=-2), INVALID),
    (dict(d=96), UNSUPPORTED),
    (dict(d=512), UNSUPPORTED),
    (dict(d=32), UNSUPPORTED),
    (dict(N=1 << 30), UNSUPPORTED),
    (dict(B=1100, N=1 << 21), UNSUPPORTED),  # more than 2^24 KV blocks to sort
])
def test_invalid_problems(bad, code):
    p = prob(**bad)
    assert fwd(p) == code
    assert bwd(p) == code
    n = ctypes.c_size_t()
    assert fm.library().fm_workspace_size(ctypes.byref(p), 1, 0, 0, ctypes.byref(n)) == code


def test_null_and_misaligned_pointers():
    assert fm.library().fm_attn_fwd(None, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 0, None,
                                    None) == INVALID
    assert fwd(prob(), q=ctypes.c_void_p(0)) == INVALID
    assert fwd(prob(), q=ctypes.c_void_p(0x100002)) == INVALID
    assert bwd(prob(), dq=ctypes.c_void_p(0)) == INVALID
    assert fwd(prob(), mask=fm.Mask(0, 0x100000, 0x100000, 0x100000)) == INVALID


def test_workspace_too_small():
    p = prob()
    need = fm.workspace_size(1, 4, 2, 256, fm.OP_FWD)
    assert fwd(p, ws_bytes=need - 1) == WORKSPACE
    need = fm.workspace_size(1, 4, 2, 256, fm.OP_BWD)
    assert bwd(p, ws_bytes=need - 1) == WORKSPACE


def test_empty_problems_are_noops():
    # nothing to do: returns FM_OK without touching any pointer
    for kw in (dict(B=0), dict(N=0), dict(Hq=0, Hkv=1)):
        p = prob(**kw)
        assert fwd(p, ws_bytes=0) == FM_OK
        assert bwd(p, ws_bytes=0) == FM_OK


def test_classify_tile_shape_checks():
    p = prob(N=100)
    m = fake_mask()
    t = fm.Tiles(*([0x100000] * 8))
    lib = fm.library()
    for bq, bk in ((12, 64), (4, 64), (512, 64), (64, 0)):
        assert lib.fm_classify_tiles(ctypes.byref(p), ctypes.byref(m), bq, bk, ctypes.byref(t),
                                     FAKE, ctypes.c_size_t(1 << 30), None) == INVALID
    assert lib.fm_classify_tiles(ctypes.byref(p), ctypes.byref(m), 64, 64, ctypes.byref(t),
                                 FAKE, ctypes.c_size_t(0), None) == WORKSPACE


def test_expand_mask_argument_checks():
    p = prob(B=2, N=100)
    m = fake_mask()
    lib = fm.library()
    for b, r0, r1 in ((2, 0, 10), (-1, 0, 10), (0, 5, 4), (0, 0, 101)):
        assert lib.fm_debug_expand_mask(ctypes.byref(p), ctypes.byref(m), b, r0, r1, FAKE,
                                        None) == INVALID
    assert lib.fm_debug_expand_mask(ctypes.byref(p), ctypes.byref(m), 0, 7, 7, None, None) == FM_OK


def test_missing_library_fails_loudly():
    code = ("import os; os.environ['FM_LIBRARY']='/nonexistent/libfm.so'\n"
            "import mask_aware_sparse_amd as fm\n"
            "try:\n    fm.library()\nexcept RuntimeError as e:\n    print('raised', e)\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert "raised" in out.stdout


def prob_kv(B=1, Hq=4, Hkv=2, Nq=256, Nk=1024):
    p = fm.Problem(B, Hq, Hkv, Nq, 128, 0.0)
    p.seqlen_kv = Nk
    return p


def test_query_share_problem_checks():
    assert fwd(prob_kv(Nk=-1)) == INVALID
    assert bwd(prob_kv(Nk=-1)) == INVALID
    assert fwd(prob_kv(Nk=(1 << 22) + 1)) == UNSUPPORTED
    # N_q = N_k = 0 is nothing to do; N_q = 0 with keys is not (dK/dV must be zeroed)
    assert fwd(prob_kv(Nq=0, Nk=0), ws_bytes=0) == FM_OK
    assert bwd(prob_kv(Nq=0, Nk=0), ws_bytes=0) == FM_OK
    assert bwd(prob_kv(Nq=0, Nk=512), ws_bytes=0) == WORKSPACE


def test_query_share_workspace_sizes():
    # forward tiles: nQB = N_q / 128 Q-blocks by nKB = N_k / 64 KV blocks
    al = lambda x: (x + 255) // 256 * 256
    nqb, nkb = 2, 16
    want = al(nkb * 64) + al(nqb * nkb * 4) + al(nqb * 8) + 2 * al(nqb * 4) + al(1024 * 4)
    assert fm.workspace_size(1, 4, 2, 256, fm.OP_FWD, seqlen_kv=1024) == want
    square = fm.workspace_size(1, 4, 2, 256, fm.OP_BWD)
    assert fm.workspace_size(1, 4, 2, 256, fm.OP_BWD, seqlen_kv=1024) > square


def test_localize_argument_checks():
    lib = fm.library()
    p = prob_kv(B=2, Nq=0, Nk=100)
    m = fake_mask()
    out = fm.MaskOut(0x100000, 0x100000, 0x100000, 0x100000)
    call = lambda p_, n, c, offs=FAKE, mm=m, o=out: lib.fm_localize_mask(
        None if p_ is None else ctypes.byref(p_), None if mm is None else ctypes.byref(mm),
        offs, n, c, None if o is None else ctypes.byref(o), None)
    assert call(None, 1, 8) == INVALID
    assert call(p, 1, 8, mm=None) == INVALID
    assert call(p, 1, 8, o=None) == INVALID
    assert call(p, 0, 8) == INVALID
    assert call(p, 1, 0) == INVALID
    assert call(p, 4097, 8) == UNSUPPORTED
    assert call(p, 1, 8, offs=None) == INVALID
    assert call(prob_kv(B=0, Nq=0, Nk=100), 1, 8) == FM_OK     # no columns: nothing to do


# ---- per-head mask sets (fm_problem.mask_heads) -------------------------------------

def prob_hm(Hq, Hkv, Hm, B=1, N=256):
    p = fm.Problem(B, Hq, Hkv, N, 128, 0.0)
    p.mask_heads = Hm
    return p


@pytest.mark.parametrize("Hq,Hkv,Hm", [(8, 4, 3), (12, 4, 6), (4, 2, 8), (4, 2, -1)])
def test_mask_heads_that_do_not_fit_are_rejected(Hq, Hkv, Hm):
    # H_m must divide H_q and divide H_kv or be a multiple of it
    p = prob_hm(Hq, Hkv, Hm)
    assert fwd(p) == INVALID
    assert bwd(p) == INVALID
    n = ctypes.c_size_t()
    assert fm.library().fm_workspace_size(ctypes.byref(p), 1, 0, 0, ctypes.byref(n)) == INVALID


@pytest.mark.parametrize("Hq,Hkv,Hm", [(8, 4, 2), (8, 4, 4), (8, 4, 8), (8, 1, 2), (6, 3, 1),
                                       (6, 3, 0)])
def test_mask_heads_that_fit_are_accepted(Hq, Hkv, Hm):
    n = ctypes.c_size_t()
    p = prob_hm(Hq, Hkv, Hm)
    for op in (fm.OP_FWD, fm.OP_BWD):
        assert fm.library().fm_workspace_size(ctypes.byref(p), op, 0, 0, ctypes.byref(n)) == FM_OK


def test_mask_heads_workspace_sizes():
    al = lambda x: (x + 255) // 256 * 256
    B, N, Hm = 2, 1000, 4
    R = B * Hm                                   # tile structures per mask row
    nqb, nkb = 8, 16
    want = al(R * nkb * 64) + al(R * nqb * nkb * 4) + al(R * nqb * 8) + 2 * al(R * nqb * 4) + \
        al(R * N * 4)
    assert fm.workspace_size(B, 8, 4, N, fm.OP_FWD, mask_heads=Hm) == want
    # dK/dV accumulators appear when sets split a kv head's group (two writers per block):
    # 8 query heads, 4 kv heads (groups of 2), 8 sets -> accumulators; 4 sets -> none
    al_acc = 2 * al(B * 4 * N * 128 * 4)
    split = fm.workspace_size(B, 8, 4, N, fm.OP_BWD, mask_heads=8)
    whole = fm.workspace_size(B, 8, 4, N, fm.OP_BWD, mask_heads=4)
    tiles_k = al(B * 4 * 8 * 64) + al(B * 4 * 8 * 32 * 4) + al(B * 4 * 8 * 8) + 2 * al(B * 4 * 8 * 4)
    tiles_q = al(B * 4 * nkb * 64) + al(B * 4 * nqb * nkb * 4) + al(B * 4 * nqb * 8) + \
        2 * al(B * 4 * nqb * 4)
    # 8 sets: twice the tile rows, accumulators, and the plan of 128 pairs without partial
    # slots against 64 pairs with them
    assert split - whole == al_acc + tiles_k + tiles_q + split_plan_bytes(128, 1, True) - \
        split_plan_bytes(64, 1, False) + al(16 * N * 4) - al(8 * N * 4)


def test_mask_heads_sort_limit():
    # at most 2^24 work blocks per sorted list: B * H_m * nKB at the forward's 64-key blocks
    n = ctypes.c_size_t()
    ok = prob_hm(64, 8, 64, N=1 << 22)            # 64 sets * 65536 KV blocks = 2^22
    assert fm.library().fm_workspace_size(ctypes.byref(ok), fm.OP_FWD, 0, 0,
                                          ctypes.byref(n)) == FM_OK
    big = prob_hm(64, 8, 64, B=5, N=1 << 22)      # 5 * 2^22 > 2^24
    assert fm.library().fm_workspace_size(ctypes.byref(big), fm.OP_FWD, 0, 0,
                                          ctypes.byref(n)) == UNSUPPORTED


# ---- multi-interval masks (fm_mask_multi) --------------------------------------------

def fwd_multi(p, m, ws_bytes=1 << 40):
    return fm.library().fm_attn_fwd_multi(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(m),
                                          FAKE, FAKE, FAKE, ctypes.c_size_t(ws_bytes), None, None)


def bwd_multi(p, m, ws_bytes=1 << 40):
    return fm.library().fm_attn_bwd_multi(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          ctypes.byref(m), FAKE, FAKE, FAKE, FAKE,
                                          ctypes.c_size_t(ws_bytes), None, None)


@pytest.mark.parametrize("n", [0, 5, -1])
def test_multi_interval_count_checked(n):
    m = fm.MaskMulti(0x100000, 0x100000, n)
    assert fwd_multi(prob(), m) == INVALID
    assert bwd_multi(prob(), m) == INVALID
    t = fm.Tiles(*([0x100000] * 8))
    assert fm.library().fm_classify_tiles_multi(ctypes.byref(prob()), ctypes.byref(m), 64, 64,
                                                ctypes.byref(t), FAKE, ctypes.c_size_t(1 << 30),
                                                None) == INVALID
    assert fm.library().fm_localize_mask_multi(ctypes.byref(prob()), ctypes.byref(m), FAKE, 1, 8,
                                               FAKE, FAKE, None) == INVALID


def test_multi_null_pointers_and_workspace():
    assert fwd_multi(prob(), fm.MaskMulti(0, 0x100000, 2)) == INVALID
    assert bwd_multi(prob(), fm.MaskMulti(0x100000, 0, 2)) == INVALID
    m = fm.MaskMulti(0x100000, 0x100000, 4)
    need = fm.workspace_size(1, 4, 2, 256, fm.OP_FWD)
    assert fwd_multi(prob(), m, ws_bytes=need - 1) == WORKSPACE
    need = fm.workspace_size(1, 4, 2, 256, fm.OP_BWD)
    assert bwd_multi(prob(), m, ws_bytes=need - 1) == WORKSPACE
    # empty problems are no-ops for the multi form too
    assert fwd_multi(prob(B=0), m, ws_bytes=0) == FM_OK
    assert bwd_multi(prob(N=0), m, ws_bytes=0) == FM_OK


def test_multi_localize_argument_checks():
    lib = fm.library()
    p = prob_kv(B=2, Nq=0, Nk=100)
    m = fm.MaskMulti(0x100000, 0x100000, 3)
    call = lambda n, c, offs=FAKE, ls=FAKE, le=FAKE: lib.fm_localize_mask_multi(
        ctypes.byref(p), ctypes.byref(m), offs, n, c, ls, le, None)
    assert call(0, 8) == INVALID
    assert call(1, 0) == INVALID
    assert call(1, 8, offs=None) == INVALID
    assert call(1, 8, ls=None) == INVALID
    assert call(4097, 8) == UNSUPPORTED


# ---- block-sparse masks (fm_mask_blocks) ----------------------------------------------

def test_blocks_null_grid_and_workspace():
    lib = fm.library()
    null = fm.MaskBlocks(0)
    assert lib.fm_attn_fwd_blocks(ctypes.byref(prob()), FAKE, FAKE, FAKE, ctypes.byref(null), FAKE,
                                  FAKE, FAKE, ctypes.c_size_t(1 << 40), None, None) == INVALID
    m = fm.MaskBlocks(0x100000)
    need = fm.workspace_size(1, 4, 2, 256, fm.OP_FWD)
    assert lib.fm_attn_fwd_blocks(ctypes.byref(prob()), FAKE, FAKE, FAKE, ctypes.byref(m), FAKE,
                                  FAKE, FAKE, ctypes.c_size_t(need - 1), None, None) == WORKSPACE
    need = fm.workspace_size(1, 4, 2, 256, fm.OP_BWD)
    assert lib.fm_attn_bwd_blocks(ctypes.byref(prob()), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  ctypes.byref(m), FAKE, FAKE, FAKE, FAKE,
                                  ctypes.c_size_t(need - 1), None, None) == WORKSPACE
    # an empty problem needs no grid
    assert lib.fm_attn_fwd_blocks(ctypes.byref(prob(N=0)), FAKE, FAKE, FAKE, ctypes.byref(null),
                                  FAKE, FAKE, FAKE, ctypes.c_size_t(0), None, None) == FM_OK


def test_blocks_binding_checks_the_grid_shape():
    import torch
    with pytest.raises(ValueError):
        fm._mask_blocks(torch.zeros((1, 2, 3), dtype=torch.uint8), 300, 300)   # needs 3 x 3
    with pytest.raises(ValueError):
        fm._mask_blocks(torch.zeros((1, 3, 3), dtype=torch.int32), 300, 300)   # uint8 only
    m, B, Hm = fm._mask_blocks(torch.zeros((2, 4, 3, 3), dtype=torch.uint8), 300, 257)
    assert (B, Hm) == (2, 4)


# ---- key order (fm_problem.key_order, fm_key_order) ------------------------------------
def test_key_order_values_checked():
    p = prob()
    p.key_order = 2
    assert fwd(p) == INVALID
    assert bwd(p) == INVALID
    n = ctypes.c_size_t()
    assert fm.library().fm_workspace_size(ctypes.byref(p), 1, 0, 0, ctypes.byref(n)) == INVALID


def test_key_order_unsupported_forms():
    lib = fm.library()
    p = prob()
    p.key_order = fm.KEYS_SORTED
    mm = fm.MaskMulti(0x100000, 0x100000, 1)
    assert lib.fm_attn_fwd_multi(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(mm), FAKE,
                                 FAKE, FAKE, ctypes.c_size_t(1 << 40), None, None) == UNSUPPORTED
    mb = fm.MaskBlocks(0x100000)
    assert lib.fm_attn_bwd_blocks(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  ctypes.byref(mb), FAKE, FAKE, FAKE, FAKE,
                                  ctypes.c_size_t(1 << 40), None, None) == UNSUPPORTED
    # a kv head shared by two mask sets would need two key orders
    ph = fm.Problem(1, 4, 2, 256, 128, 0.0, 0, 4, fm.KEYS_SORTED)
    assert fwd(ph) == UNSUPPORTED
    assert bwd(ph) == UNSUPPORTED
    ph.mask_heads = 2
    assert fwd(ph, ws_bytes=0) == WORKSPACE


def test_key_order_workspace_sizes():
    al = lambda x: (x + 255) // 256 * 256
    B, Hq, Hkv, N, d, Hm = 2, 8, 2, 1000, 128, 2
    nat = {op: fm.workspace_size(B, Hq, Hkv, N, op, mask_heads=Hm) for op in (1, 2)}
    srt = {op: fm.workspace_size(B, Hq, Hkv, N, op, mask_heads=Hm, key_order=fm.KEYS_SORTED)
           for op in (1, 2)}
    cols, rows = al(B * Hm * N * 4), al(B * Hkv * N * d * 2)
    # the permutation and four vectors; K and V (forward), also dK and dV (backward)
    assert srt[1] - nat[1] == 5 * cols + 2 * rows
    # the backward's dK/dV tiles also change shape (256 keys per block at d = 128), so its
    # tile structures differ; at d = 64 they keep 128 keys and only the copies are added
    assert srt[2] - nat[2] >= 4 * rows
    n64 = fm.workspace_size(B, Hq, Hkv, N, 2, mask_heads=Hm, head_dim=64)
    s64 = fm.workspace_size(B, Hq, Hkv, N, 2, mask_heads=Hm, head_dim=64, key_order=1)
    assert s64 - n64 == 5 * cols + 4 * al(B * Hkv * N * 64 * 2)
    # the classifier's workspace ignores the option
    assert fm.workspace_size(B, Hq, Hkv, N, 0, 64, 64, mask_heads=Hm, key_order=1) == \
        fm.workspace_size(B, Hq, Hkv, N, 0, 64, 64, mask_heads=Hm)


def test_key_order_entry_point_checks():
    lib = fm.library()
    m = fake_mask()
    p = fm.Problem(1, 1, 1, 256, 128, 0.0, 0, 0, 0)
    assert lib.fm_key_order(None, ctypes.byref(m), FAKE, None, None) == INVALID
    assert lib.fm_key_order(ctypes.byref(p), None, FAKE, None, None) == INVALID
    assert lib.fm_key_order(ctypes.byref(p), ctypes.byref(m), None, None, None) == INVALID
    bad = fm.Mask(0x100000, 0, 0x100000, 0x100000)
    assert lib.fm_key_order(ctypes.byref(p), ctypes.byref(bad), FAKE, None, None) == INVALID
    p.seqlen = 1 << 23
    assert lib.fm_key_order(ctypes.byref(p), ctypes.byref(m), FAKE, None, None) == UNSUPPORTED
    # nothing to order: no pointer is touched
    e = fm.Problem(0, 1, 1, 256, 128, 0.0, 0, 0, 0)
    assert lib.fm_key_order(ctypes.byref(e), ctypes.byref(m), None, None, None) == FM_OK


def test_workspace_bytes_matches_workspace_size():
    lib = fm.library()
    for args in [(2, 8, 2, 1000, 1, 0, 0), (2, 8, 1, 1000, 2, 0, 0), (1, 4, 2, 300, 0, 64, 32)]:
        B, Hq, Hkv, N, op, bq, bk = args
        p = prob(B=B, Hq=Hq, Hkv=Hkv, N=N)
        assert lib.fm_workspace_bytes(ctypes.byref(p), op, bq, bk) == \
            fm.workspace_size(B, Hq, Hkv, N, op, bq, bk)
    # rejected problems and arguments give 0
    assert lib.fm_workspace_bytes(ctypes.byref(prob(Hq=3, Hkv=2)), 1, 0, 0) == 0
    assert lib.fm_workspace_bytes(ctypes.byref(prob()), 0, 48, 64) == 0
    assert lib.fm_workspace_bytes(None, 1, 0, 0) == 0


def test_schedule_values_checked():
    """fm_problem.schedule: FM_SCHEDULE_LPT (0) or FM_SCHEDULE_NATURAL (1); others rejected
    before anything is launched."""
    for bad in (2, -1):
        p = fm.Problem(1, 4, 2, 256, 128, 0.0, 0, 0, 0, bad)
        assert fwd(p) == INVALID
        assert bwd(p) == INVALID
    n = ctypes.c_size_t()
    ok = fm.Problem(1, 4, 2, 256, 128, 0.0, 0, 0, 0, fm.SCHEDULE_NATURAL)
    assert fm.library().fm_workspace_size(ctypes.byref(ok), fm.OP_FWD, 0, 0, ctypes.byref(n)) == 0
    assert n.value == fm.workspace_size(1, 4, 2, 256, fm.OP_FWD)


def test_check_mask_argument_checks():
    """fm_check_mask / _multi: null problem, mask or count, and a bad interval count, are
    rejected before anything is launched."""
    lib = fm.library()
    p = prob()
    m = fake_mask()
    assert lib.fm_check_mask(None, ctypes.byref(m), FAKE, None) == INVALID
    assert lib.fm_check_mask(ctypes.byref(p), None, FAKE, None) == INVALID
    assert lib.fm_check_mask(ctypes.byref(p), ctypes.byref(m), None, None) == INVALID
    nulls = fm.Mask(0, 0x100000, 0x100000, 0x100000)
    assert lib.fm_check_mask(ctypes.byref(p), ctypes.byref(nulls), FAKE, None) == INVALID
    for n in (0, 5):
        mm = fm.MaskMulti(0x100000, 0x100000, n)
        assert lib.fm_check_mask_multi(ctypes.byref(p), ctypes.byref(mm), FAKE, None) == INVALID
