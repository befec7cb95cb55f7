"""Mask-aware (column-interval) attention on AMD MI355X: thin Python binding of libfm.

Every function here marshals arguments and calls the C ABI declared in include/fm.h;
all computation runs in the library's HIP kernels.  torch is used for device memory
(outputs and workspaces are torch tensors) and for the current stream.  There is no
fallback: if libfm.so is missing or fails to load, every call raises.

The operation (FlashMask-3 project page, Overview and §3.1): key column j of batch row
b hides query rows [LTS_j, LTE_j) and [UTS_j, UTE_j); tiles are skipped, masked or run
plain according to the block min/max of those vectors; forward returns O and the
per-row natural-log LSE, backward returns dQ, dK, dV (Flash MSA guide, "The Backward
Pass").
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "FMError", "library", "library_path", "tile_shape", "workspace_size", "classify_tiles",
    "ipo_balance", "fm_ipo_balance", "localize_mask", "fm_localize_mask",
    "attn_fwd", "attn_bwd", "debug_expand_mask", "status_string",
    "fm_tile_shape", "fm_workspace_size", "fm_classify_tiles", "fm_attn_fwd", "fm_attn_bwd",
    "fm_debug_expand_mask", "fm_status_string", "attn_fwd_static", "fm_attn_fwd_static",
    "STATIC_WORKSPACE_BYTES", "check_mask", "check_mask_multi", "fm_check_mask",
    "fm_check_mask_multi",
    "OP_CLASSIFY", "OP_FWD", "OP_BWD", "HEAD_DIM", "key_order", "fm_key_order",
    "KEYS_NATURAL", "KEYS_SORTED", "KEY_ORDER_SPAN", "KEY_ORDER_GROUP", "SCHEDULE_LPT",
    "SCHEDULE_NATURAL", "flashmask_attention",
]

HERE = os.path.dirname(os.path.abspath(__file__))
OP_CLASSIFY, OP_FWD, OP_BWD = 0, 1, 2
KEYS_NATURAL, KEYS_SORTED = 0, 1      # fm_problem.key_order
SCHEDULE_LPT, SCHEDULE_NATURAL = 0, 1  # fm_problem.schedule
KEY_ORDER_SPAN, KEY_ORDER_GROUP = 2048, 64
HEAD_DIM = 128
FM_OK = 0
STATIC_WORKSPACE_BYTES = 16 << 20   # FM_STATIC_WORKSPACE_BYTES


def library_path() -> str:
    return os.environ.get("FM_LIBRARY", os.path.join(HERE, "libfm.so"))


class FMError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32),
                ("heads_kv", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("seqlen_kv", ctypes.c_int32), ("mask_heads", ctypes.c_int32),
                ("key_order", ctypes.c_int32), ("schedule", ctypes.c_int32)]


class MaskOut(ctypes.Structure):
    _fields_ = [("lts", ctypes.c_void_p), ("lte", ctypes.c_void_p),
                ("uts", ctypes.c_void_p), ("ute", ctypes.c_void_p)]


class Mask(ctypes.Structure):
    _fields_ = [("lts", ctypes.c_void_p), ("lte", ctypes.c_void_p),
                ("uts", ctypes.c_void_p), ("ute", ctypes.c_void_p)]


class MaskMulti(ctypes.Structure):
    _fields_ = [("start", ctypes.c_void_p), ("end", ctypes.c_void_p),
                ("n_intervals", ctypes.c_int32)]


class MaskBlocks(ctypes.Structure):
    _fields_ = [("blocks", ctypes.c_void_p)]


class KernelEvents(ctypes.Structure):
    _fields_ = [("start", ctypes.c_void_p), ("stop", ctypes.c_void_p),
                ("start2", ctypes.c_void_p), ("stop2", ctypes.c_void_p)]


class Tiles(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("block_minmax", "tile_class", "q_queue", "q_count", "k_queue", "k_count",
                 "q_order", "k_order")]


_lib = None
_P = ctypes.c_void_p
_STATUS = ctypes.c_int


def library():
    """Load libfm.so once; raises if it is missing (no fallback path exists)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"libfm.so not found at {path}; build it with "
                               "`python -m mask_aware_sparse_amd.build`")
        lib = ctypes.CDLL(path)
        PP, PM, PT = ctypes.POINTER(Problem), ctypes.POINTER(Mask), ctypes.POINTER(Tiles)
        PE = ctypes.POINTER(KernelEvents)
        PX = ctypes.POINTER(MaskMulti)
        PB = ctypes.POINTER(MaskBlocks)
        sig = {
            "fm_status_string": ([_STATUS], ctypes.c_char_p),
            "fm_tile_shape": ([_STATUS, ctypes.POINTER(ctypes.c_int32),
                               ctypes.POINTER(ctypes.c_int32)], _STATUS),
            "fm_workspace_size": ([PP, _STATUS, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.POINTER(ctypes.c_size_t)], _STATUS),
            "fm_workspace_bytes": ([PP, _STATUS, ctypes.c_int32, ctypes.c_int32],
                                   ctypes.c_size_t),
            "fm_classify_tiles": ([PP, PM, ctypes.c_int32, ctypes.c_int32, PT, _P,
                                   ctypes.c_size_t, _P], _STATUS),
            "fm_attn_fwd": ([PP, _P, _P, _P, PM, _P, _P, _P, ctypes.c_size_t, _P, PE], _STATUS),
            "fm_attn_fwd_static": ([PP, _P, _P, _P, PM, _P, _P, _P, PE], _STATUS),
            "fm_attn_bwd": ([PP, _P, _P, _P, _P, _P, _P, PM, _P, _P, _P, _P, ctypes.c_size_t,
                             _P, PE], _STATUS),
            "fm_debug_expand_mask": ([PP, PM, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      _P, _P], _STATUS),
            "fm_localize_mask": ([PP, PM, _P, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.POINTER(MaskOut), _P], _STATUS),
            "fm_key_order": ([PP, PM, _P, ctypes.POINTER(MaskOut), _P], _STATUS),
            "fm_check_mask": ([PP, PM, _P, _P], _STATUS),
            "fm_check_mask_multi": ([PP, PX, _P, _P], _STATUS),
            "fm_classify_tiles_multi": ([PP, PX, ctypes.c_int32, ctypes.c_int32, PT, _P,
                                         ctypes.c_size_t, _P], _STATUS),
            "fm_attn_fwd_multi": ([PP, _P, _P, _P, PX, _P, _P, _P, ctypes.c_size_t, _P, PE],
                                  _STATUS),
            "fm_attn_bwd_multi": ([PP, _P, _P, _P, _P, _P, _P, PX, _P, _P, _P, _P,
                                   ctypes.c_size_t, _P, PE], _STATUS),
            "fm_debug_expand_mask_multi": ([PP, PX, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, _P, _P], _STATUS),
            "fm_localize_mask_multi": ([PP, PX, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P],
                                       _STATUS),
            "fm_classify_tiles_blocks": ([PP, PB, ctypes.c_int32, ctypes.c_int32, PT, _P,
                                          ctypes.c_size_t, _P], _STATUS),
            "fm_attn_fwd_blocks": ([PP, _P, _P, _P, PB, _P, _P, _P, ctypes.c_size_t, _P, PE],
                                   _STATUS),
            "fm_attn_bwd_blocks": ([PP, _P, _P, _P, _P, _P, _P, PB, _P, _P, _P, _P,
                                    ctypes.c_size_t, _P, PE], _STATUS),
            "fm_debug_expand_mask_blocks": ([PP, PB, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, _P, _P], _STATUS),
        }
        for name, (args, res) in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return library().fm_status_string(int(status)).decode()


def _check(status, where):
    if status != FM_OK:
        raise FMError(status, where)


def _problem(batch, heads_q, heads_kv, seqlen, scale=None, head_dim=HEAD_DIM, seqlen_kv=0,
             mask_heads=0, key_order=KEYS_NATURAL, schedule=SCHEDULE_LPT):
    return Problem(int(batch), int(heads_q), int(heads_kv), int(seqlen), int(head_dim),
                   float(scale) if scale is not None else 0.0, int(seqlen_kv), int(mask_heads),
                   int(key_order), int(schedule))


def _mask(lts, lte, uts, ute):
    for t in (lts, lte, uts, ute):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("mask vectors must be contiguous int32 tensors [B][N] or [B][H_m][N]")
        if t.shape != lts.shape:
            raise ValueError("the four mask vectors must have one shape")
    return Mask(lts.data_ptr(), lte.data_ptr(), uts.data_ptr(), ute.data_ptr())


def _on_device(device, named):
    """Every tensor of `named` ((name, tensor or None) pairs) on `device`, a GPU.  Runs
    after the shape and dtype checks, so those are reported first."""
    if device.type != "cuda":
        raise ValueError(f"tensors must be on the GPU (got {device})")
    for name, t in named:
        if t is not None and t.device != device:
            raise ValueError(f"{name} must be on {device} (got {t.device})")


def _expect(t, name, shape, dtype):
    """A caller-supplied tensor: exact shape, dtype and contiguity (the kernels address it
    from its base pointer with the problem's strides)."""
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _keep_alive(stream, device, *tensors):
    """Tensors allocated here and used on a stream other than the current one: tell the
    caching allocator, so that it does not hand their memory out again while the kernels
    queued on `stream` may still use it."""
    if stream is None or stream == torch.cuda.current_stream(device):
        return
    for t in tensors:
        if t is not None and t.numel():
            t.record_stream(stream)


def _mask_dims(lts):
    """(B, H_m, N_k) of vectors [B][N_k] (one set per batch row, H_m = 1) or
    [B][H_m][N_k] (per-head sets: query head h uses set h // (H_q / H_m))."""
    if lts.dim() == 2:
        return lts.shape[0], 1, lts.shape[1]
    if lts.dim() == 3:
        return tuple(lts.shape)
    raise ValueError("mask vectors must be [B][N] or [B][H_m][N]")


def _stream(device, stream=None):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None and t.numel() else 0)


def tile_shape(op: int):
    bq, bk = ctypes.c_int32(), ctypes.c_int32()
    _check(library().fm_tile_shape(int(op), ctypes.byref(bq), ctypes.byref(bk)), "fm_tile_shape")
    return bq.value, bk.value


def workspace_size(batch, heads_q, heads_kv, seqlen, op, block_q=0, block_k=0, head_dim=HEAD_DIM,
                   seqlen_kv=0, mask_heads=0, key_order=KEYS_NATURAL):
    """Workspace bytes for N_q = seqlen query rows, N_k = seqlen_kv keys (0: N_q),
    mask_heads vector sets per batch row (0: 1) and the key order (KEYS_SORTED adds the
    permuted K, V, vectors and, backward, dK, dV)."""
    n = ctypes.c_size_t()
    p = _problem(batch, heads_q, heads_kv, seqlen, head_dim=head_dim, seqlen_kv=seqlen_kv,
                 mask_heads=mask_heads, key_order=key_order)
    _check(library().fm_workspace_size(ctypes.byref(p), int(op), int(block_q), int(block_k),
                                       ctypes.byref(n)), "fm_workspace_size")
    return n.value


def _workspace(nbytes, device, ws=None):
    """(workspace, allocated here?).  A caller's workspace must be contiguous, on the
    device and at least `nbytes` long."""
    if ws is not None:
        if not ws.is_contiguous():
            raise ValueError("workspace tensor must be contiguous")
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace tensor too small")
        _on_device(device, [("workspace", ws)])
        return ws, False
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device), True


class IpoReport(ctypes.Structure):
    _fields_ = [("lb", ctypes.c_int64), ("makespan_lpt", ctypes.c_int64),
                ("makespan_p2", ctypes.c_int64), ("makespan", ctypes.c_int64),
                ("certified", ctypes.c_int32), ("moves", ctypes.c_int32)]


def ipo_balance(weights, ranks, stages=3):
    """fm_ipo_balance on host data: returns (owner int32 array, report dict)."""
    import numpy as np
    w = np.ascontiguousarray(np.asarray(weights, dtype=np.int64))
    owner = np.empty(w.shape[0], dtype=np.int32)
    rep = IpoReport()
    lib = library()
    lib.fm_ipo_balance.restype = _STATUS
    lib.fm_ipo_balance.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(IpoReport)]
    _check(lib.fm_ipo_balance(w.ctypes.data, int(w.shape[0]), int(ranks), int(stages),
                              owner.ctypes.data, ctypes.byref(rep)), "fm_ipo_balance")
    return owner, {"lb": rep.lb, "lpt": rep.makespan_lpt, "p2": rep.makespan_p2,
                   "final": rep.makespan, "certified": bool(rep.certified),
                   "moves": rep.moves}


def _mask_multi(starts, ends):
    """(MaskMulti, B, H_m, M, N_k) for interval starts/ends [B][M][N_k] or [B][H_m][M][N_k]."""
    for t in (starts, ends):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("interval starts/ends must be contiguous int32 tensors")
    if starts.shape != ends.shape:
        raise ValueError("interval starts and ends must have one shape")
    if starts.dim() == 3:
        B, M, N = starts.shape
        Hm = 1
    elif starts.dim() == 4:
        B, Hm, M, N = starts.shape
    else:
        raise ValueError("interval starts/ends must be [B][M][N] or [B][H_m][M][N]")
    return MaskMulti(starts.data_ptr(), ends.data_ptr(), int(M)), B, Hm, M, N


BLOCK = 128  # block edge of the block-sparse form


def _mask_blocks(blocks, seqlen_q, seqlen_k):
    """(MaskBlocks, B, H_m) for a block grid [B][nQB][nKB] or [B][H_m][nQB][nKB] of uint8
    (1 = visible) over 128 x 128 blocks, checked against ceil(N / 128)."""
    if blocks.dtype != torch.uint8 or not blocks.is_contiguous():
        raise ValueError("blocks must be a contiguous uint8 tensor")
    nqb, nkb = -(-int(seqlen_q) // BLOCK), -(-int(seqlen_k) // BLOCK)
    if blocks.dim() == 3:
        B, Hm = blocks.shape[0], 1
    elif blocks.dim() == 4:
        B, Hm = blocks.shape[0], blocks.shape[1]
    else:
        raise ValueError("blocks must be [B][nQB][nKB] or [B][H_m][nQB][nKB]")
    if tuple(blocks.shape[-2:]) != (nqb, nkb):
        raise ValueError(f"blocks must have {nqb} x {nkb} blocks for N_q={seqlen_q}, N_k={seqlen_k}")
    return MaskBlocks(blocks.data_ptr()), B, Hm


def _classify(fn, m, mask_ts, B, Hm, Nk, block_q, block_k, heads_q, heads_kv, stream, out, ws,
              seqlen_q, width, dev):
    if Hm > 1 and heads_q == 1 and heads_kv == 1:
        heads_q = Hm                      # the heads play no part in the classification
    N = Nk if seqlen_q is None else int(seqlen_q)
    if int(block_q) <= 0 or int(block_k) <= 0:
        raise ValueError("tile shape must be positive")
    nqb, nkb = -(-N // block_q), -(-Nk // block_k)
    shapes = _tile_shapes(B * Hm, nqb, nkb, width)
    fresh = out is None
    if fresh:
        out = {n: torch.empty(shp, dtype=dt, device=dev) for n, (shp, dt) in shapes.items()}
    else:
        for n, (shp, dt) in shapes.items():
            if n not in out:
                raise ValueError(f"out lacks {n!r}")
            _expect(out[n], n, shp, dt)
    p = _problem(B, heads_q, heads_kv, N, seqlen_kv=Nk, mask_heads=Hm)
    nbytes = workspace_size(B, heads_q, heads_kv, N, OP_CLASSIFY, block_q, block_k,
                            seqlen_kv=Nk, mask_heads=Hm)
    _on_device(dev, [(f"mask tensor {i}", t) for i, t in enumerate(mask_ts)] +
               [(n, out[n]) for n in shapes])
    ws, own_ws = _workspace(nbytes, dev, ws)
    tiles = Tiles(*(out[n].data_ptr() if out[n].numel() else 0 for n, _ in Tiles._fields_))
    _check(fn(ctypes.byref(p), ctypes.byref(m), int(block_q), int(block_k), ctypes.byref(tiles),
              _ptr(ws), ctypes.c_size_t(nbytes), _stream(dev, stream)), fn.__name__)
    _keep_alive(stream, dev, *([ws] if own_ws else []), *(out.values() if fresh else ()))
    return out


def classify_tiles(lts, lte, uts, ute, block_q, block_k, heads_q=1, heads_kv=1, stream=None,
                   out=None, ws=None, seqlen_q=None):
    """Run fm_classify_tiles; returns a dict of device tensors (see fm_tiles in fm.h).
    The vectors are [B][N_k] or [B][H_m][N_k] (tiles per mask row b * H_m + m); `seqlen_q`
    is N_q (default N_k).  `out` (a dict as returned by an earlier call of the same shape)
    and `ws` (uint8 device tensor of at least workspace_size(..., OP_CLASSIFY, block_q,
    block_k) bytes) may be passed to reuse buffers."""
    B, Hm, Nk = _mask_dims(lts)
    return _classify(library().fm_classify_tiles, _mask(lts, lte, uts, ute),
                     (lts, lte, uts, ute), B, Hm, Nk, block_q, block_k, heads_q, heads_kv, stream,
                     out, ws, seqlen_q, 8, lts.device)


def classify_tiles_multi(starts, ends, block_q, block_k, heads_q=1, heads_kv=1, stream=None,
                         out=None, ws=None, seqlen_q=None):
    """fm_classify_tiles_multi for interval starts/ends [B][M][N_k] or [B][H_m][M][N_k];
    block_minmax is [B*H_m][nKB][4M]."""
    m, B, Hm, M, Nk = _mask_multi(starts, ends)
    return _classify(library().fm_classify_tiles_multi, m, (starts, ends), B, Hm, Nk, block_q,
                     block_k, heads_q, heads_kv, stream, out, ws, seqlen_q, 4 * M, starts.device)


def classify_tiles_blocks(blocks, block_q, block_k, seqlen_q, seqlen_k, heads_q=1, heads_kv=1,
                          stream=None, out=None, ws=None):
    """fm_classify_tiles_blocks for a block grid (see _mask_blocks); block_minmax is not
    written."""
    m, B, Hm = _mask_blocks(blocks, seqlen_q, seqlen_k)
    return _classify(library().fm_classify_tiles_blocks, m, (blocks,), B, Hm, int(seqlen_k),
                     block_q, block_k, heads_q, heads_kv, stream, out, ws, int(seqlen_q), 8,
                     blocks.device)


def _tile_shapes(R, nqb, nkb, width=8):
    """(shape, dtype) of each fm_tiles buffer for R mask rows (see fm_tiles in fm.h)."""
    i32 = torch.int32
    return {
        "block_minmax": ((R, nkb, width), i32),
        "tile_class": ((R, nqb, nkb), torch.uint8),
        "q_queue": ((R, nqb, nkb), i32),
        "q_count": ((R, nqb, 2), i32),
        "k_queue": ((R, nkb, nqb), i32),
        "k_count": ((R, nkb, 2), i32),
        "q_order": ((R * nqb,), i32),
        "k_order": ((R * nkb,), i32),
    }


def _shapes(q, k, mask_shape):
    """(B, H_q, H_kv, N_q, N_k, d, H_m) from Q [B][H_q][N_q][d], K [B][H_kv][N_k][d] and
    the mask's (B, H_m, N_k)."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("expected Q [B][H_q][N_q][d] and K/V [B][H_kv][N_k][d]")
    B, Hq, N, d = q.shape
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("Q and K/V shapes disagree")
    if k.shape[2] == 0 and N > 0:
        # fm_problem.seqlen_kv = 0 means "as many keys as rows"
        raise ValueError("query rows without keys cannot be expressed (seqlen_kv = 0 means N_q)")
    Bm, Hm, Nm = mask_shape
    if Bm != B or Nm != k.shape[2]:
        raise ValueError("the mask's batch and key length must match Q and K")
    return B, Hq, k.shape[1], N, k.shape[2], d, Hm


def _bf16(*named):
    for name, t in named:
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 tensor")


def _events(ev):
    """Up to four torch.cuda.Event objects (start, stop[, start2, stop2]) ->
    fm_kernel_events pointer (or None)."""
    if ev is None:
        return None
    handles = []
    for e in ev:
        if e.cuda_event == 0:          # torch creates the event lazily on first record
            e.record()
        handles.append(e.cuda_event)
    handles += [0] * (4 - len(handles))
    return ctypes.byref(KernelEvents(*handles))


def _fwd(fn, q, k, v, m, mask_ts, mask_shape, scale, ws, out, lse, stream, events,
         key_order=KEYS_NATURAL, schedule=SCHEDULE_LPT):
    _bf16(("q", q), ("k", k), ("v", v))
    B, Hq, Hkv, N, Nk, d, Hm = _shapes(q, k, mask_shape)
    _expect(v, "v", k.shape, torch.bfloat16)
    if out is not None:
        _expect(out, "out", q.shape, torch.bfloat16)
    if lse is not None:
        _expect(lse, "lse", (B, Hq, N), torch.float32)
    dev = q.device
    _on_device(dev, [("k", k), ("v", v), ("out", out), ("lse", lse)] +
               [(f"mask tensor {i}", t) for i, t in enumerate(mask_ts)])
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, Hq, N), dtype=torch.float32, device=dev) if lse is None else lse
    p = _problem(B, Hq, Hkv, N, scale, head_dim=d, seqlen_kv=Nk, mask_heads=Hm,
                 key_order=key_order, schedule=schedule)
    nbytes = workspace_size(B, Hq, Hkv, N, OP_FWD, head_dim=d, seqlen_kv=Nk, mask_heads=Hm,
                            key_order=key_order)
    w, own_ws = _workspace(nbytes, dev, ws)
    _check(fn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(m), _ptr(o), _ptr(lse_t),
              _ptr(w), ctypes.c_size_t(nbytes), _stream(dev, stream), _events(events)),
           fn.__name__)
    _keep_alive(stream, dev, w if own_ws else None, o if out is None else None,
                lse_t if lse is None else None)
    return o, lse_t


def _bwd(fn, q, k, v, o, lse, dout, m, mask_ts, mask_shape, scale, ws, grads, stream, events,
         key_order=KEYS_NATURAL, schedule=SCHEDULE_LPT):
    _bf16(("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout))
    B, Hq, Hkv, N, Nk, d, Hm = _shapes(q, k, mask_shape)
    _expect(v, "v", k.shape, torch.bfloat16)
    _expect(o, "o", q.shape, torch.bfloat16)
    _expect(dout, "dout", q.shape, torch.bfloat16)
    _expect(lse, "lse", (B, Hq, N), torch.float32)
    if grads is not None:
        if len(grads) != 3:
            raise ValueError("grads must be (dq, dk, dv)")
        for name, g, like in zip(("dq", "dk", "dv"), grads, (q, k, k)):
            _expect(g, name, like.shape, torch.bfloat16)
    dev = q.device
    _on_device(dev, [("k", k), ("v", v), ("o", o), ("dout", dout), ("lse", lse)] +
               ([] if grads is None else list(zip(("dq", "dk", "dv"), grads))) +
               [(f"mask tensor {i}", t) for i, t in enumerate(mask_ts)])
    fresh = grads is None
    if fresh:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    p = _problem(B, Hq, Hkv, N, scale, head_dim=d, seqlen_kv=Nk, mask_heads=Hm,
                 key_order=key_order, schedule=schedule)
    nbytes = workspace_size(B, Hq, Hkv, N, OP_BWD, head_dim=d, seqlen_kv=Nk, mask_heads=Hm,
                            key_order=key_order)
    w, own_ws = _workspace(nbytes, dev, ws)
    _check(fn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
              ctypes.byref(m), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(w), ctypes.c_size_t(nbytes),
              _stream(dev, stream), _events(events)), fn.__name__)
    _keep_alive(stream, dev, w if own_ws else None, *(grads if fresh else ()))
    return dq, dk, dv


def attn_fwd(q, k, v, lts, lte, uts, ute, scale=None, ws=None, out=None, lse=None, stream=None,
             events=None, key_order=KEYS_NATURAL, schedule=SCHEDULE_LPT):
    """O (bf16 [B][H_q][N_q][d]) and LSE (fp32 [B][H_q][N_q], natural log) via fm_attn_fwd;
    K/V are [B][H_kv][N_k][d] and the vectors [B][N_k] or, one set per group of H_q / H_m
    query heads, [B][H_m][N_k].
    `events`: optional (start, stop) torch.cuda.Event pair timing the attention kernel.
    `key_order`: KEYS_SORTED runs the kernels over the keys in fm_key_order's order.
    `schedule`: SCHEDULE_LPT (cost-descending dispatch) or SCHEDULE_NATURAL (index order)."""
    return _fwd(library().fm_attn_fwd, q, k, v, _mask(lts, lte, uts, ute), (lts, lte, uts, ute),
                _mask_dims(lts), scale, ws, out, lse, stream, events, key_order, schedule)


def attn_fwd_static(q, k, v, lts, lte, uts, ute, scale=None, out=None, lse=None, stream=None,
                    events=None):
    """fm_attn_fwd_static: attn_fwd on the library's own fixed device workspace (no
    workspace argument; for callers that cannot allocate).  Pass `out` and `lse` to make the
    call allocate nothing at all.  Problems whose forward workspace exceeds
    STATIC_WORKSPACE_BYTES are refused.  Calls that overlap on one GPU (different streams)
    race on the shared workspace."""
    m = _mask(lts, lte, uts, ute)
    mask_ts = (lts, lte, uts, ute)
    _bf16(("q", q), ("k", k), ("v", v))
    B, Hq, Hkv, N, Nk, d, Hm = _shapes(q, k, _mask_dims(lts))
    _expect(v, "v", k.shape, torch.bfloat16)
    if out is not None:
        _expect(out, "out", q.shape, torch.bfloat16)
    if lse is not None:
        _expect(lse, "lse", (B, Hq, N), torch.float32)
    need = workspace_size(B, Hq, Hkv, N, OP_FWD, head_dim=d, seqlen_kv=Nk, mask_heads=Hm)
    if need > STATIC_WORKSPACE_BYTES:
        raise ValueError(f"the forward workspace of this problem ({need} bytes) exceeds the "
                         f"static workspace ({STATIC_WORKSPACE_BYTES} bytes); use attn_fwd")
    dev = q.device
    _on_device(dev, [("k", k), ("v", v), ("out", out), ("lse", lse)] +
               [(f"mask tensor {i}", t) for i, t in enumerate(mask_ts)])
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, Hq, N), dtype=torch.float32, device=dev) if lse is None else lse
    p = _problem(B, Hq, Hkv, N, scale, head_dim=d, seqlen_kv=Nk, mask_heads=Hm)
    _check(library().fm_attn_fwd_static(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                        ctypes.byref(m), _ptr(o), _ptr(lse_t),
                                        _stream(dev, stream), _events(events)),
           "fm_attn_fwd_static")
    _keep_alive(stream, dev, o if out is None else None, lse_t if lse is None else None)
    return o, lse_t


def attn_fwd_multi(q, k, v, starts, ends, scale=None, ws=None, out=None, lse=None, stream=None,
                   events=None, schedule=SCHEDULE_LPT):
    """fm_attn_fwd_multi: as attn_fwd with the multi-interval mask, starts/ends
    [B][M][N_k] or [B][H_m][M][N_k] (key j visible to row i iff some interval holds i)."""
    m, B, Hm, M, Nk = _mask_multi(starts, ends)
    return _fwd(library().fm_attn_fwd_multi, q, k, v, m, (starts, ends), (B, Hm, Nk), scale,
                ws, out, lse, stream, events, schedule=schedule)


def attn_fwd_blocks(q, k, v, blocks, scale=None, ws=None, out=None, lse=None, stream=None,
                    events=None, schedule=SCHEDULE_LPT):
    """fm_attn_fwd_blocks: as attn_fwd with a block-sparse mask, a uint8 grid [B][nQB][nKB]
    or [B][H_m][nQB][nKB] over 128 x 128 blocks (1 = visible)."""
    m, B, Hm = _mask_blocks(blocks, q.shape[2], k.shape[2])
    return _fwd(library().fm_attn_fwd_blocks, q, k, v, m, (blocks,), (B, Hm, k.shape[2]),
                scale, ws, out, lse, stream, events, schedule=schedule)


def attn_bwd_blocks(q, k, v, o, lse, dout, blocks, scale=None, ws=None, grads=None, stream=None,
                    events=None, schedule=SCHEDULE_LPT):
    """fm_attn_bwd_blocks: as attn_bwd with a block-sparse mask."""
    m, B, Hm = _mask_blocks(blocks, q.shape[2], k.shape[2])
    return _bwd(library().fm_attn_bwd_blocks, q, k, v, o, lse, dout, m, (blocks,),
                (B, Hm, k.shape[2]), scale, ws, grads, stream, events, schedule=schedule)


def attn_bwd(q, k, v, o, lse, dout, lts, lte, uts, ute, scale=None, ws=None, grads=None,
             stream=None, events=None, key_order=KEYS_NATURAL, schedule=SCHEDULE_LPT):
    """(dQ, dK, dV) in bf16 via fm_attn_bwd.  `events`: optional (start, stop, start2,
    stop2) torch.cuda.Event objects timing the dK/dV kernel and the dQ kernel.
    `key_order`: as for attn_fwd; dK and dV come back in the caller's key order."""
    return _bwd(library().fm_attn_bwd, q, k, v, o, lse, dout, _mask(lts, lte, uts, ute),
                (lts, lte, uts, ute), _mask_dims(lts), scale, ws, grads, stream, events,
                key_order, schedule)


def attn_bwd_multi(q, k, v, o, lse, dout, starts, ends, scale=None, ws=None, grads=None,
                   stream=None, events=None, schedule=SCHEDULE_LPT):
    """fm_attn_bwd_multi: as attn_bwd with the multi-interval mask."""
    m, B, Hm, M, Nk = _mask_multi(starts, ends)
    return _bwd(library().fm_attn_bwd_multi, q, k, v, o, lse, dout, m, (starts, ends),
                (B, Hm, Nk), scale, ws, grads, stream, events, schedule=schedule)


def _expand(fn, m, mask_ts, B, Hm, N, b, row0, row1, stream, seqlen_q, dev):
    if not 0 <= int(row0) <= int(row1):
        raise ValueError("need 0 <= row0 <= row1")
    _on_device(dev, [(f"mask tensor {i}", t) for i, t in enumerate(mask_ts)])
    dense = torch.empty((row1 - row0, N), dtype=torch.uint8, device=dev)
    p = _problem(B, Hm, 1, N if seqlen_q is None else int(seqlen_q), seqlen_kv=N, mask_heads=Hm)
    _check(fn(ctypes.byref(p), ctypes.byref(m), int(b), int(row0), int(row1), _ptr(dense),
              _stream(dev, stream)), fn.__name__)
    _keep_alive(stream, dev, dense)
    return dense


def debug_expand_mask(lts, lte, uts, ute, b, row0, row1, stream=None, seqlen_q=None):
    """uint8 [row1-row0][N_k] dense expansion (1 = hidden) by the kernels' predicate, of
    mask row b (batch row * H_m + set for per-head vectors)."""
    B, Hm, N = _mask_dims(lts)
    return _expand(library().fm_debug_expand_mask, _mask(lts, lte, uts, ute),
                   (lts, lte, uts, ute), B, Hm, N, b, row0, row1, stream, seqlen_q, lts.device)


def debug_expand_mask_multi(starts, ends, b, row0, row1, stream=None, seqlen_q=None):
    """Dense expansion of mask row b of the multi-interval form (1 = hidden)."""
    m, B, Hm, M, N = _mask_multi(starts, ends)
    return _expand(library().fm_debug_expand_mask_multi, m, (starts, ends), B, Hm, N, b, row0,
                   row1, stream, seqlen_q, starts.device)


def debug_expand_mask_blocks(blocks, b, row0, row1, seqlen_q, seqlen_k, stream=None):
    """Dense expansion of mask row b of a block grid (1 = hidden)."""
    m, B, Hm = _mask_blocks(blocks, seqlen_q, seqlen_k)
    return _expand(library().fm_debug_expand_mask_blocks, m, (blocks,), B, Hm, int(seqlen_k), b,
                   row0, row1, stream, int(seqlen_q), blocks.device)


def _offsets(offsets):
    if offsets.dtype != torch.int32 or not offsets.is_contiguous() or offsets.dim() != 1:
        raise ValueError("offsets must be a contiguous int32 tensor [n_chunks]")


def localize_mask(lts, lte, uts, ute, offsets, chunk_len, out=None, stream=None):
    """fm_localize_mask: the vectors [B][N_k] renumbered into the rows of a rank that owns
    the query chunks [offsets[i], offsets[i] + chunk_len) (offsets: int32 device tensor,
    ascending, non-overlapping).  Returns four int32 tensors of the vectors' shape ([B][N_k]
    or [B][H_m][N_k])."""
    B, Hm, N = _mask_dims(lts)
    m = _mask(lts, lte, uts, ute)
    _offsets(offsets)
    fresh = out is None
    if not fresh:
        if len(out) != 4:
            raise ValueError("out must hold four tensors")
        for i, t in enumerate(out):
            _expect(t, f"out[{i}]", lts.shape, torch.int32)
    _on_device(lts.device, [("lte", lte), ("uts", uts), ("ute", ute), ("offsets", offsets)] +
               ([] if fresh else [(f"out[{i}]", t) for i, t in enumerate(out)]))
    if fresh:
        out = tuple(torch.empty_like(lts) for _ in range(4))
    p = _problem(B, 1, 1, 0, seqlen_kv=N, mask_heads=Hm)
    mo = MaskOut(*(t.data_ptr() for t in out))
    _check(library().fm_localize_mask(ctypes.byref(p), ctypes.byref(m), _ptr(offsets),
                                      int(offsets.numel()), int(chunk_len), ctypes.byref(mo),
                                      _stream(lts.device, stream)), "fm_localize_mask")
    _keep_alive(stream, lts.device, *(out if fresh else ()))
    return out


def key_order(lts, lte, uts, ute, seqlen_q=None, permuted=False, stream=None):
    """fm_key_order: the key permutation of each mask row (int32, the vectors' shape;
    position p holds key perm[p]) and, with permuted=True, also the four vectors in that
    order.  seqlen_q: N_q (default: N_k)."""
    B, Hm, N = _mask_dims(lts)
    m = _mask(lts, lte, uts, ute)
    _on_device(lts.device, [("lte", lte), ("uts", uts), ("ute", ute)])
    perm = torch.empty_like(lts)
    out = tuple(torch.empty_like(lts) for _ in range(4)) if permuted else None
    p = _problem(B, 1, 1, N if seqlen_q is None else int(seqlen_q), seqlen_kv=N, mask_heads=Hm)
    mo = ctypes.byref(MaskOut(*(t.data_ptr() for t in out))) if permuted else None
    _check(library().fm_key_order(ctypes.byref(p), ctypes.byref(m), _ptr(perm), mo,
                                  _stream(lts.device, stream)), "fm_key_order")
    _keep_alive(stream, lts.device, perm, *(out or ()))
    return (perm, out) if permuted else perm


def check_mask(lts, lte, uts, ute, seqlen_q=None, out=None, stream=None, sync=True):
    """fm_check_mask: the number of row bounds outside [0, N_q] (seqlen_q, default N_k).  With
    sync=False the device int32 tensor `out` (allocated if None) is returned unread."""
    B, Hm, N = _mask_dims(lts)
    m = _mask(lts, lte, uts, ute)
    if out is not None:
        _expect(out, "out", (1,), torch.int32)
    _on_device(lts.device, [("lte", lte), ("uts", uts), ("ute", ute), ("out", out)])
    bad = torch.empty(1, dtype=torch.int32, device=lts.device) if out is None else out
    p = _problem(B, 1, 1, N if seqlen_q is None else int(seqlen_q), seqlen_kv=N, mask_heads=Hm)
    _check(library().fm_check_mask(ctypes.byref(p), ctypes.byref(m), _ptr(bad),
                                   _stream(lts.device, stream)), "fm_check_mask")
    _keep_alive(stream, lts.device, bad if out is None else None)
    return int(bad.item()) if sync else bad


def check_mask_multi(starts, ends, seqlen_q=None, out=None, stream=None, sync=True):
    """fm_check_mask_multi: as check_mask over the interval starts and ends."""
    m, B, Hm, M, N = _mask_multi(starts, ends)
    if out is not None:
        _expect(out, "out", (1,), torch.int32)
    _on_device(starts.device, [("ends", ends), ("out", out)])
    bad = torch.empty(1, dtype=torch.int32, device=starts.device) if out is None else out
    p = _problem(B, 1, 1, N if seqlen_q is None else int(seqlen_q), seqlen_kv=N, mask_heads=Hm)
    _check(library().fm_check_mask_multi(ctypes.byref(p), ctypes.byref(m), _ptr(bad),
                                         _stream(starts.device, stream)), "fm_check_mask_multi")
    _keep_alive(stream, starts.device, bad if out is None else None)
    return int(bad.item()) if sync else bad


def localize_mask_multi(starts, ends, offsets, chunk_len, out=None, stream=None):
    """fm_localize_mask_multi: every interval start and end renumbered into the rank's rows.
    Returns (starts, ends) of the input's shape."""
    m, B, Hm, M, N = _mask_multi(starts, ends)
    _offsets(offsets)
    fresh = out is None
    if not fresh:
        if len(out) != 2:
            raise ValueError("out must hold (starts, ends)")
        for i, t in enumerate(out):
            _expect(t, f"out[{i}]", starts.shape, torch.int32)
    _on_device(starts.device, [("ends", ends), ("offsets", offsets)] +
               ([] if fresh else [(f"out[{i}]", t) for i, t in enumerate(out)]))
    if fresh:
        out = (torch.empty_like(starts), torch.empty_like(ends))
    p = _problem(B, 1, 1, 0, seqlen_kv=N, mask_heads=Hm)
    _check(library().fm_localize_mask_multi(ctypes.byref(p), ctypes.byref(m), _ptr(offsets),
                                            int(offsets.numel()), int(chunk_len), _ptr(out[0]),
                                            _ptr(out[1]), _stream(starts.device, stream)),
           "fm_localize_mask_multi")
    _keep_alive(stream, starts.device, *(out if fresh else ()))
    return out


class _FlashMaskAttention(torch.autograd.Function):
    """Autograd glue over fm_attn_fwd / fm_attn_bwd: the forward keeps O and the LSE, the
    backward recomputes P from them in the library's backward kernels."""

    @staticmethod
    def forward(ctx, q, k, v, lts, lte, uts, ute, scale, key_order):
        o, lse = attn_fwd(q, k, v, lts, lte, uts, ute, scale=scale, key_order=key_order)
        ctx.save_for_backward(q, k, v, o, lse, lts, lte, uts, ute)
        ctx.scale, ctx.key_order = scale, key_order
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, o, lse, lts, lte, uts, ute = ctx.saved_tensors
        if dout.dtype != torch.bfloat16:
            raise TypeError(f"flashmask_attention: the output gradient must be bfloat16, "
                            f"got {dout.dtype}")
        dq, dk, dv = attn_bwd(q, k, v, o, lse, dout.contiguous(), lts, lte, uts, ute,
                              scale=ctx.scale, key_order=ctx.key_order)
        return dq, dk, dv, None, None, None, None, None, None


def flashmask_attention(q, k, v, lts, lte, uts, ute, scale=None, key_order=KEYS_NATURAL):
    """O = softmax(Q K^T * scale, masked) V with gradients for q, k and v: the drop-in for a
    dense-mask scaled-dot-product attention that the FlashMask Guide's integration section
    describes, taking the column-wise vectors instead of the N x N mask.  Shapes, dtypes and
    the mask convention are attn_fwd's (bf16 q [B][H_q][N_q][d], k and v [B][H_kv][N_k][d],
    int32 vectors [B][N_k] or [B][H_m][N_k]; key column j hides rows [LTS_j, LTE_j) and
    [UTS_j, UTE_j)).  A visible row range [FMS_j, FME_j] of the guide's two-vector form is
    UTS_j = 0, UTE_j = FMS_j, LTS_j = FME_j + 1, LTE_j = N_q.  The vectors take no gradient."""
    return _FlashMaskAttention.apply(q, k, v, lts, lte, uts, ute, scale, key_order)


# The C names, for callers that prefer them.
fm_tile_shape = tile_shape
fm_workspace_size = workspace_size
fm_classify_tiles = classify_tiles
fm_attn_fwd = attn_fwd
fm_attn_fwd_static = attn_fwd_static
fm_attn_bwd = attn_bwd
fm_debug_expand_mask = debug_expand_mask
fm_localize_mask = localize_mask
fm_key_order = key_order
fm_check_mask = check_mask
fm_check_mask_multi = check_mask_multi
fm_classify_tiles_multi = classify_tiles_multi
fm_attn_fwd_multi = attn_fwd_multi
fm_attn_bwd_multi = attn_bwd_multi
fm_debug_expand_mask_multi = debug_expand_mask_multi
fm_localize_mask_multi = localize_mask_multi
fm_classify_tiles_blocks = classify_tiles_blocks
fm_attn_fwd_blocks = attn_fwd_blocks
fm_attn_bwd_blocks = attn_bwd_blocks
fm_debug_expand_mask_blocks = debug_expand_mask_blocks
fm_status_string = status_string

fm_ipo_balance = ipo_balance
