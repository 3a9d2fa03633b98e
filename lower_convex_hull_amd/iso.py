"""Thin ctypes binding of libiso.so (include/iso.h), argument marshalling only.

Every step of the fit runs in the library's gfx950 kernels; this module only
passes pointers, sizes and the current torch stream.  It raises if the built
library is missing: there is no fallback.

Functions with the C names take raw device pointers (ints); ``fit`` is a
convenience wrapper over torch CUDA tensors that allocates the output and the
workspace with torch and calls ``iso_fit_ex``.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libiso.so")

ISO_OK = 0
ISO_WARN_NONFINITE = 1
ISO_ERR_ARG = -1
ISO_ERR_WEIGHT = -2
ISO_ERR_NOMEM = -3
ISO_ERR_HIP = -4
ISO_ERR_WORKSPACE = -5
ISO_ERR_DATA = -6
ISO_ERR_INVARIANT = -7

ISO_F_NOCHECK = 1
ISO_F_DECREASING = 2
ISO_F_COPY_CONTROL = 4
ISO_F_DEBUG_INVARIANTS = 8
ISO_F_WAVE_MERGES = 0x400
ISO_F_THREE_CASE = 0x800
ISO_F_TREE_MERGES = 0x1000
ISO_F_WEIGHTED_HINT = 0x100
ISO_F_PHASE_STAMPS = 0x200

ISO_PHASE_NAMES = ("short_rows", "chunk_hulls", "merge", "expand", "copy_bridge", "copy_move",
                   "merge_top", "chunk_redo")

ISO_NOALLOC_BYTES = 64 << 20

EXPORTS = ("iso_fit", "iso_fit_ex", "iso_fit_noalloc", "iso_workspace_bytes", "iso_status_str",
           "iso_release", "iso_chunk_size", "iso_short_row_max", "iso_timing_enable",
           "iso_timing_read", "iso_vjp", "iso_vjp_f64", "iso_vjp_workspace_bytes", "iso_fit_ex_f64",
           "iso_fit_f64", "iso_calib_fit", "iso_calib_apply", "iso_calib_workspace_bytes",
           "iso_copy_probe")

_lib = None


class IsoError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"libiso status {status}: {iso_status_str(status)}")
        self.status = status


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, u32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
        L.iso_fit.argtypes = [p, p, i64, i64, p]
        L.iso_fit.restype = ctypes.c_int
        L.iso_fit_ex.argtypes = [p, p, i64, i64, p, p, p, sz, p, u32]
        L.iso_fit_ex.restype = ctypes.c_int
        L.iso_fit_ex_f64.argtypes = [p, p, i64, i64, p, p, p, sz, p, u32]
        L.iso_fit_ex_f64.restype = ctypes.c_int
        L.iso_fit_f64.argtypes = [p, p, i64, i64, p]
        L.iso_fit_f64.restype = ctypes.c_int
        L.iso_copy_probe.argtypes = [p, p, sz, p]
        L.iso_copy_probe.restype = ctypes.c_int
        L.iso_calib_fit.argtypes = [p, p, p, i64, p, p, p, p, sz, p]
        L.iso_calib_fit.restype = ctypes.c_int
        L.iso_calib_apply.argtypes = [p, p, i64, p, p, i64, p, p]
        L.iso_calib_apply.restype = ctypes.c_int
        L.iso_calib_workspace_bytes.argtypes = [i64]
        L.iso_calib_workspace_bytes.restype = sz
        L.iso_fit_noalloc.argtypes = [p, p, i64, i64, p, p, p, u32]
        L.iso_fit_noalloc.restype = ctypes.c_int
        L.iso_vjp.argtypes = [p, p, p, p, i64, i64, p, p, p, sz, p]
        L.iso_vjp.restype = ctypes.c_int
        L.iso_vjp_f64.argtypes = [p, p, p, p, i64, i64, p, p, p, sz, p]
        L.iso_vjp_f64.restype = ctypes.c_int
        L.iso_vjp_workspace_bytes.argtypes = [i64, i64]
        L.iso_vjp_workspace_bytes.restype = sz
        L.iso_workspace_bytes.argtypes = [i64, i64, u32]
        L.iso_workspace_bytes.restype = sz
        L.iso_status_str.argtypes = [ctypes.c_int]
        L.iso_status_str.restype = ctypes.c_char_p
        L.iso_release.argtypes = []
        L.iso_release.restype = None
        L.iso_chunk_size.argtypes = [i64]
        L.iso_chunk_size.restype = i64
        L.iso_short_row_max.argtypes = []
        L.iso_short_row_max.restype = i64
        L.iso_timing_enable.argtypes = [ctypes.c_int]
        L.iso_timing_enable.restype = ctypes.c_int
        L.iso_timing_read.argtypes = [p, p, ctypes.c_int]
        L.iso_timing_read.restype = ctypes.c_int
        _lib = L
    return _lib


def iso_fit(y_ptr, w_ptr, rows, n, out_ptr) -> int:
    return lib().iso_fit(y_ptr, w_ptr, rows, n, out_ptr)


def iso_fit_ex(y_ptr, w_ptr, rows, n, out_ptr, block_id_ptr, ws_ptr, ws_bytes, stream, flags) -> int:
    return lib().iso_fit_ex(y_ptr, w_ptr, rows, n, out_ptr, block_id_ptr, ws_ptr, ws_bytes,
                            stream, flags)


def iso_fit_ex_f64(y_ptr, w_ptr, rows, n, out_ptr, block_id_ptr, ws_ptr, ws_bytes, stream,
                   flags) -> int:
    return lib().iso_fit_ex_f64(y_ptr, w_ptr, rows, n, out_ptr, block_id_ptr, ws_ptr, ws_bytes,
                                stream, flags)


def iso_fit_f64(y_ptr, w_ptr, rows, n, out_ptr) -> int:
    return lib().iso_fit_f64(y_ptr, w_ptr, rows, n, out_ptr)


def iso_copy_probe(src_ptr, dst_ptr, nbytes, stream) -> int:
    return lib().iso_copy_probe(src_ptr, dst_ptr, nbytes, stream)


def iso_calib_fit(scores_ptr, outcomes_ptr, segment_ptr, n, xp_ptr, fp_ptr, k_out, ws_ptr, ws_bytes,
                  stream) -> int:
    """k_out: a ctypes.c_int64 receiving the number of distinct keys."""
    return lib().iso_calib_fit(scores_ptr, outcomes_ptr, segment_ptr, n, xp_ptr, fp_ptr,
                               ctypes.byref(k_out), ws_ptr, ws_bytes, stream)


def iso_calib_apply(xp_ptr, fp_ptr, k, scores_ptr, segment_ptr, m, out_ptr, stream) -> int:
    return lib().iso_calib_apply(xp_ptr, fp_ptr, k, scores_ptr, segment_ptr, m, out_ptr, stream)


def iso_calib_workspace_bytes(n) -> int:
    return lib().iso_calib_workspace_bytes(n)


def iso_fit_noalloc(y_ptr, w_ptr, rows, n, out_ptr, block_id_ptr, stream, flags) -> int:
    return lib().iso_fit_noalloc(y_ptr, w_ptr, rows, n, out_ptr, block_id_ptr, stream, flags)


def iso_vjp(g_ptr, y_ptr, w_ptr, block_id_ptr, rows, n, grad_y_ptr, grad_w_ptr, ws_ptr, ws_bytes,
            stream) -> int:
    return lib().iso_vjp(g_ptr, y_ptr, w_ptr, block_id_ptr, rows, n, grad_y_ptr, grad_w_ptr, ws_ptr,
                         ws_bytes, stream)


def iso_vjp_f64(g_ptr, y_ptr, w_ptr, block_id_ptr, rows, n, grad_y_ptr, grad_w_ptr, ws_ptr,
                ws_bytes, stream) -> int:
    return lib().iso_vjp_f64(g_ptr, y_ptr, w_ptr, block_id_ptr, rows, n, grad_y_ptr, grad_w_ptr,
                             ws_ptr, ws_bytes, stream)


def iso_vjp_workspace_bytes(rows, n) -> int:
    return lib().iso_vjp_workspace_bytes(rows, n)


def iso_workspace_bytes(rows, n, flags=0) -> int:
    return lib().iso_workspace_bytes(rows, n, flags)


def iso_status_str(status: int) -> str:
    return lib().iso_status_str(status).decode()


def iso_release() -> None:
    lib().iso_release()


def iso_chunk_size(n: int) -> int:
    return lib().iso_chunk_size(n)


def iso_short_row_max() -> int:
    return lib().iso_short_row_max()


def iso_timing_enable(on: bool) -> int:
    return lib().iso_timing_enable(1 if on else 0)


def iso_timing_read():
    """Per-phase (total ms, launches) of the launches recorded since the last read."""
    n = len(ISO_PHASE_NAMES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    st = lib().iso_timing_read(ms, cnt, n)
    if st < 0:
        raise IsoError(st)
    return {ISO_PHASE_NAMES[i]: (ms[i], cnt[i]) for i in range(n)}


def _stream_handle(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def workspace(rows: int, n: int, weighted: bool, flags: int = 0, device=None):
    """A torch uint8 CUDA tensor large enough for iso_fit_ex (256-byte aligned by torch)."""
    import torch

    nbytes = iso_workspace_bytes(rows, n, flags | (ISO_F_WEIGHTED_HINT if weighted else 0))
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device or "cuda")


def fit(y, w=None, *, block_ids: bool = False, flags: int = 0, out=None, ws=None, stream=None,
        check: bool = True):
    """Weighted isotonic fit of each row of a 2-D (or 1-D) float32 or float64 CUDA tensor.

    Returns ``out`` (and ``block_id`` when ``block_ids``).  Raises IsoError on an
    error status; a NONFINITE warning is returned as NaN rows, not raised.
    """
    import torch

    if y.dtype not in (torch.float32, torch.float64) or not y.is_cuda:
        raise TypeError("y must be a float32 or float64 CUDA tensor")
    y2 = y.reshape(1, -1) if y.dim() == 1 else y
    if not y2.is_contiguous():
        raise ValueError("y must be contiguous")
    rows, n = y2.shape
    if w is not None:
        if w.dtype != y.dtype or not w.is_cuda or w.numel() != y2.numel() or not w.is_contiguous():
            raise ValueError("w must be a contiguous CUDA tensor of y's dtype, shaped like y")
    if out is None:
        out = torch.empty_like(y)
    bid = torch.empty(y.shape, dtype=torch.int32, device=y.device) if block_ids else None
    if ws is None:
        ws = workspace(rows, n, w is not None, flags, device=y.device)
    fn = iso_fit_ex if y.dtype == torch.float32 else iso_fit_ex_f64
    st = fn(y2.data_ptr(), None if w is None else w.data_ptr(), rows, n, out.data_ptr(),
                    None if bid is None else bid.data_ptr(), ws.data_ptr(),
                    ws.numel() * ws.element_size(), _stream_handle(stream),
                    flags | (0 if check else ISO_F_NOCHECK))
    if st < 0:
        raise IsoError(st)
    return (out, bid) if block_ids else out


def vjp(g, y, w, block_id, *, grad_w: bool = False, stream=None):
    """Backward pass over torch CUDA tensors (f32 or f64, like g): returns
    grad_y, or (grad_y, grad_w) when grad_w.  block_id is the forward call's."""
    import torch

    g2 = g.reshape(1, -1) if g.dim() == 1 else g
    rows, n = g2.shape
    gy = torch.empty_like(g)
    gw = torch.empty_like(g) if grad_w else None
    nb = iso_vjp_workspace_bytes(rows, n)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=g.device)
    fn = iso_vjp if g.dtype == torch.float32 else iso_vjp_f64
    ptr = lambda t: None if t is None else t.data_ptr()
    st = fn(g.data_ptr(), ptr(y), ptr(w), block_id.data_ptr(), rows, n, gy.data_ptr(), ptr(gw),
            ws.data_ptr(), nb, _stream_handle(stream))
    if st < 0:
        raise IsoError(st)
    return (gy, gw) if grad_w else gy


def calib_curve(scores, outcomes, segment=None, stream=None):
    """Calibration curve over torch CUDA f64 tensors: returns (xp, fp), each of
    the number of distinct keys."""
    import torch

    n = scores.numel()
    xp = torch.empty(n, dtype=torch.float64, device=scores.device)
    fp = torch.empty_like(xp)
    nb = iso_calib_workspace_bytes(n)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=scores.device)
    k = ctypes.c_int64(0)
    st = iso_calib_fit(scores.data_ptr(), outcomes.data_ptr(),
                       None if segment is None else segment.data_ptr(), n, xp.data_ptr(),
                       fp.data_ptr(), k, ws.data_ptr(), nb, _stream_handle(stream))
    if st < 0:
        raise IsoError(st)
    return xp[:k.value], fp[:k.value]
