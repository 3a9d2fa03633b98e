"""Test infrastructure: ctypes wrapper around the plain-C CPU oracle (iso_oracle.c).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The GPU library never imports, links or calls it.

The oracle computes the weighted isotonic fit of equation (1) of the paper
"Merge Hulls Without Copying Vertices: GPU Isotonic Regression" (section 2.1)
with pool adjacent violators in f64; see iso_oracle.c for the readings taken.
Parity is pinned for every routine here (tests/test_oracle.py): brute force over
contiguous partitions, KKT prefix conditions, worked examples printed on the
pages, closed forms and a library routine; the vector-Jacobian product (paper
section 6, "Gradient") by finite differences of the fit in y and in w, closed
forms and block sums.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "iso_oracle.c")
_BUILD = os.path.join(_HERE, "_build")

_libs: dict[int, ctypes.CDLL] = {}


def lib_path(mutant: int = 0) -> str:
    name = "liboracle.so" if mutant == 0 else f"liboracle_mutant{mutant}.so"
    return os.path.join(_BUILD, name)


def build(mutant: int = 0, force: bool = False) -> str:
    """Compile iso_oracle.c with gcc (mutant > 0 plants that planted mistake)."""
    out = lib_path(mutant)
    if (not force and os.path.exists(out)
            and os.path.getmtime(out) >= os.path.getmtime(_SRC)):
        return out
    os.makedirs(_BUILD, exist_ok=True)
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC",
           f"-DORACLE_MUTANT={mutant}", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _lib(mutant: int = 0) -> ctypes.CDLL:
    if mutant not in _libs:
        lib = ctypes.CDLL(build(mutant))
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_pava_f64.argtypes = [p, p, i64, p, p]
        lib.oracle_pava_f64.restype = i64
        lib.oracle_fit_rows_f32.argtypes = [p, p, i64, i64, p, p, p]
        lib.oracle_fit_rows_f32.restype = ctypes.c_int
        lib.oracle_brute_force.argtypes = [p, p, ctypes.c_int, p]
        lib.oracle_brute_force.restype = ctypes.c_double
        lib.oracle_hull_fit.argtypes = [p, p, i64, p]
        lib.oracle_hull_fit.restype = i64
        lib.oracle_vjp_f64.argtypes = [p, p, p, p, i64, p, p]
        lib.oracle_vjp_f64.restype = ctypes.c_int
        lib.oracle_vjp_rows_f32.argtypes = [p, p, p, p, i64, i64, p, p]
        lib.oracle_vjp_rows_f32.restype = ctypes.c_int
        _libs[mutant] = lib
    return _libs[mutant]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def pava(y, w=None, mutant: int = 0):
    """f64 weighted PAVA of one row. Returns (z f64, block_id int32, n_blocks)."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    w = None if w is None else np.ascontiguousarray(w, dtype=np.float64)
    n = y.shape[0]
    z = np.empty(n, np.float64)
    bid = np.empty(n, np.int32)
    nb = _lib(mutant).oracle_pava_f64(_ptr(y), _ptr(w), n, _ptr(z), _ptr(bid))
    if nb < 0:
        raise MemoryError("oracle: allocation failed")
    return z, bid, int(nb)


def fit_rows_f32(y, w=None, mutant: int = 0):
    """Rows of f32 data -> (f32 fit rounded once, f64 fit, block ids)."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    if y.ndim == 1:
        y = y[None, :]
    rows, n = y.shape
    if w is not None:
        w = np.ascontiguousarray(w, dtype=np.float32).reshape(rows, n)
    out = np.empty((rows, n), np.float32)
    out64 = np.empty((rows, n), np.float64)
    bid = np.empty((rows, n), np.int32)
    rc = _lib(mutant).oracle_fit_rows_f32(_ptr(y), _ptr(w), rows, n, _ptr(out),
                                          _ptr(out64), _ptr(bid))
    if rc != 0:
        raise MemoryError("oracle: allocation failed")
    return out, out64, bid


def brute_force(y, w=None):
    """Least-squares fit by enumerating contiguous partitions (n <= 24)."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    w = None if w is None else np.ascontiguousarray(w, dtype=np.float64)
    n = y.shape[0]
    z = np.empty(n, np.float64)
    err = _lib().oracle_brute_force(_ptr(y), _ptr(w), n, _ptr(z))
    if err < 0:
        raise ValueError("brute force supports 1 <= n <= 24")
    return z, float(err)


def hull_fit(y, w=None):
    """Slopes of the lower hull of the cumulative sum diagram. Returns (z, n_vertices)."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    w = None if w is None else np.ascontiguousarray(w, dtype=np.float64)
    n = y.shape[0]
    z = np.empty(n, np.float64)
    nv = _lib().oracle_hull_fit(_ptr(y), _ptr(w), n, _ptr(z))
    if nv < 0:
        raise MemoryError("oracle: allocation failed")
    return z, int(nv)


def vjp(y, w, g, block_id=None, mutant: int = 0):
    """Vector-Jacobian product of one row's fit in f64: (d/dy, d/dw) for the
    gradient g with respect to the fit, over block_id's blocks (None: the
    oracle's own).  d/dw is None for unit weights."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    g = np.ascontiguousarray(g, dtype=np.float64)
    w = None if w is None else np.ascontiguousarray(w, dtype=np.float64)
    bid = None if block_id is None else np.ascontiguousarray(block_id, dtype=np.int32)
    n = y.shape[0]
    gy = np.empty(n, np.float64)
    gw = np.empty(n, np.float64) if w is not None else None
    if _lib(mutant).oracle_vjp_f64(_ptr(y), _ptr(w), _ptr(g), _ptr(bid), n, _ptr(gy), _ptr(gw)) != 0:
        raise MemoryError("oracle: allocation failed")
    return gy, gw


def vjp_rows_f32(y, w, g, block_id=None, mutant: int = 0):
    """Rows of f32 data and gradient -> f64 (d/dy, d/dw) of each row's fit over
    block_id's blocks (None: the oracle's own); d/dw is None for unit weights."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    if y.ndim == 1:
        y = y[None, :]
    rows, n = y.shape
    g = np.ascontiguousarray(g, dtype=np.float32).reshape(rows, n)
    if w is not None:
        w = np.ascontiguousarray(w, dtype=np.float32).reshape(rows, n)
    bid = None if block_id is None else np.ascontiguousarray(block_id, dtype=np.int32).reshape(rows, n)
    gy = np.empty((rows, n), np.float64)
    gw = np.empty((rows, n), np.float64) if w is not None else None
    rc = _lib(mutant).oracle_vjp_rows_f32(_ptr(y), _ptr(w), _ptr(g), _ptr(bid), rows, n, _ptr(gy),
                                          _ptr(gw))
    if rc != 0:
        raise MemoryError("oracle: allocation failed")
    return gy, gw
