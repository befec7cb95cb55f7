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
    assert fm.tile_shape(fm.OP_BWD) == (32, 256)
    with pytest.raises(fm.FMError):
        fm.tile_shape(fm.OP_CLASSIFY)


def test_workspace_sizes():
    # forward: minmax + queue + counts + cost + order, each 256-byte aligned
    B, N = 2, 1000
    nqb, nkb = 8, 16
    al = lambda x: (x + 255) // 256 * 256
    want = al(B * nkb * 32) + al(B * nqb * nkb * 4) + al(B * nqb * 8) + 2 * al(B * nqb * 4)
    assert fm.workspace_size(B, 4, 2, N, fm.OP_FWD) == want
    assert fm.workspace_size(B, 4, 2, N, fm.OP_CLASSIFY, 64, 32) == al(B * 16 * 4) + al(B * 32 * 4)
    # backward: fp32 dK/dV accumulators exist only for query-head groups above 4 heads
    # (same Hq, so the same D / LSE buffers; tiles depend on B and N only)
    with_acc = fm.workspace_size(B, 8, 1, N, fm.OP_BWD)
    without = fm.workspace_size(B, 8, 2, N, fm.OP_BWD)
    assert with_acc - without == 2 * al(B * 1 * N * 128 * 4)
    assert without < 2 * B * 8 * N * 4 + 65536


@pytest.mark.parametrize("bad,code", [
    (dict(Hq=3, Hkv=2), INVALID),
    (dict(Hkv=0), INVALID),
    (dict(N=-1), INVALID),
    (dict(B=-2), INVALID),
    (dict(d=64), UNSUPPORTED),
    (dict(N=1 << 30), UNSUPPORTED),
    (dict(B=65, N=16384), UNSUPPORTED),     # more than 8192 Q-blocks to sort
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
