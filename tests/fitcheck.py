"""Checks shared by the tests: golden-file parsing, optimality conditions, the
weighted objective and the GPU-versus-oracle parity rule.

None of this computes the fit; it only judges one.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_cases(name: str):
    """Parse a golden file into dicts with keys case, source, y, w, z (Fractions)."""
    cases, cur = [], None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            val = val.strip()
            if key == "case":
                cur = {"case": val}
                cases.append(cur)
            elif key == "source":
                cur["source"] = val
            elif key in ("y", "z", "S"):
                cur[key] = [Fraction(t) for t in val.split()]
            elif key == "w":
                cur["w"] = None if val == "-" else [Fraction(t) for t in val.split()]
    return cases


def read_single(name: str):
    """Parse a golden file without case headers (key: values lines)."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            out[key] = [Fraction(t) for t in val.split()]
    return out


def objective(y, w, z) -> float:
    """sum_i w_i (z_i - y_i)^2 in f64 (paper section 2.1, equation (1))."""
    y = np.asarray(y, np.float64)
    z = np.asarray(z, np.float64)
    w = np.ones_like(y) if w is None else np.asarray(w, np.float64)
    return float(np.sum(w * (z - y) ** 2))


def objective_gap(y, w, out, z) -> float:
    """f(out) - f(z), formed term by term as w (o - z)(o + z - 2y) to avoid cancellation."""
    y = np.asarray(y, np.float64)
    z = np.asarray(z, np.float64)
    o = np.asarray(out, np.float64)
    w = np.ones_like(y) if w is None else np.asarray(w, np.float64)
    return float(np.sum(w * (o - z) * (o + z - 2.0 * y)))


def kkt_violation(y, w, z) -> dict:
    """Optimality conditions of the isotonic fit, in units of sum w|y| (at least 1).

    With lambda_k = sum_{i<=k} w_i (y_i - z_i):  lambda_k >= 0 for all k,
    lambda_n = 0, lambda_k = 0 wherever z_{k+1} > z_k, and z non-decreasing
    (Mova groupant card, entries "Invariant" and "kkt_prefix").
    """
    y = np.asarray(y, np.float64)
    z = np.asarray(z, np.float64)
    w = np.ones_like(y) if w is None else np.asarray(w, np.float64)
    scale = max(1.0, float(np.sum(w * np.abs(y))))
    lam = np.cumsum(w * (y - z))
    rise = np.zeros(len(y), bool)
    rise[:-1] = z[1:] > z[:-1]
    return {
        "neg_prefix": float(max(0.0, -lam.min())) / scale if len(lam) else 0.0,
        "total": abs(float(lam[-1])) / scale if len(lam) else 0.0,
        "at_rise": float(np.abs(lam[rise]).max()) / scale if rise.any() else 0.0,
        "step_down": float(max(0.0, -(np.diff(z).min() if len(z) > 1 else 0.0))),
    }


def kkt_ok(y, w, z, tau=1e-12) -> bool:
    v = kkt_violation(y, w, z)
    return v["neg_prefix"] <= tau and v["total"] <= tau and v["at_rise"] <= tau and v["step_down"] == 0.0


def parity(y, w, out, z64, rel_obj=1e-9, ref32=None):
    """The GPU-versus-oracle rule, per row:
      max |out - z| <= 1e-5 (1 + max|y|)   (z the oracle's f64 fit), and
      |f(out) - f(ref32)| <= 1e-9 max(f(z), 2^-24 sum w y^2),
    where ref32 is the oracle's fit rounded once to float32 (default: z rounded
    here).  Reading: both solvers round each slope once to the working type
    (paper section 6, "Output"), so the objectives compared are those of the two
    float32 outputs; on ill-conditioned rows (values near 1 +- 1e-7, or offset
    by 1e6) the rounding alone moves f(z) by more than 1e-9 relative.
    Returns (ok, worst_abs_ratio, worst_obj_ratio, row_of_worst)."""
    y = np.atleast_2d(np.asarray(y, np.float64))
    out = np.atleast_2d(np.asarray(out, np.float64))
    z64 = np.atleast_2d(np.asarray(z64, np.float64))
    r32 = (z64.astype(np.float32) if ref32 is None else np.atleast_2d(ref32)).astype(np.float64)
    wr = None if w is None else np.atleast_2d(np.asarray(w, np.float64))
    worst_a, worst_o, worst_row = 0.0, 0.0, -1
    for r in range(y.shape[0]):
        wrow = None if wr is None else wr[r]
        tol = 1e-5 * (1.0 + float(np.abs(y[r]).max()))
        a = float(np.abs(out[r] - z64[r]).max()) / tol if y.shape[1] else 0.0
        fz = objective(y[r], wrow, z64[r])
        wy2 = float(np.sum((np.ones_like(y[r]) if wrow is None else wrow) * y[r] ** 2))
        den = max(fz, 2.0 ** -24 * wy2, 1e-300)
        o = abs(objective_gap(y[r], wrow, out[r], r32[r])) / (rel_obj * den)
        if max(a, o) > max(worst_a, worst_o):
            worst_row = r
        worst_a, worst_o = max(worst_a, a), max(worst_o, o)
    return (worst_a <= 1.0 and worst_o <= 1.0), worst_a, worst_o, worst_row


def block_ids_consistent(oracle_bid, gpu_bid, z64, y, delta_scale=1e-6) -> bool:
    """Every oracle block start whose adjacent means differ by more than delta is a
    GPU block start, and every extra GPU block start separates means within delta."""
    ob = np.asarray(oracle_bid)
    gb = np.asarray(gpu_bid)
    z = np.asarray(z64, np.float64)
    delta = delta_scale * (1.0 + float(np.abs(np.asarray(y, np.float64)).max()))
    os_ = np.flatnonzero(np.diff(ob) != 0) + 1
    gs = np.flatnonzero(np.diff(gb) != 0) + 1
    if gb[0] != 0 or np.any(np.diff(gb) < 0) or np.any(np.diff(gb) > 1):
        return False
    gset = set(gs.tolist())
    oset = set(os_.tolist())
    for s in os_:
        if abs(z[s] - z[s - 1]) > delta and s not in gset:
            return False
    for s in gs:
        if s not in oset and abs(z[s] - z[s - 1]) > delta:
            return False
    return True


def _block_bounds(bid):
    """Start of each block of one row (block ids: a start wherever the id changes)."""
    bid = np.asarray(bid)
    return np.concatenate([[0], np.flatnonzero(np.diff(bid) != 0) + 1])


def vjp_tolerance(y, w, g, bid, out_eps=2.0 ** -24):
    """Per-element bound on |GPU - oracle| for the vector-Jacobian product of one
    row over the blocks bid: both sides form the block sums G = sum g,
    W = sum w and S = sum w y in f64 in different orders, each off the exact sum
    by at most m u sum|terms| (m terms, u = 2^-53), and round the result once to
    the output type (out_eps: 2^-24 for f32, 2^-53 for f64).  Returns
    (tol_gy, tol_gw); tol_gw is None for unit weights."""
    u = 2.0 ** -53
    y = np.asarray(y, np.float64)
    g = np.asarray(g, np.float64)
    wv = np.ones_like(y) if w is None else np.asarray(w, np.float64)
    st = _block_bounds(bid)
    m = np.diff(np.concatenate([st, [len(y)]])).astype(np.float64)
    G = np.add.reduceat(g, st)
    Ga = np.add.reduceat(np.abs(g), st)
    W = np.add.reduceat(wv, st)
    S = np.add.reduceat(wv * y, st)
    Sa = np.add.reduceat(np.abs(wv * y), st)
    eG = 2 * m * u * Ga  # sums on both sides
    eW = 2 * m * u * W
    eS = 2 * m * u * Sa
    r = G / W
    er = (eG + np.abs(r) * eW) / W * (1 + 1e-6)
    z = S / W
    ez = (eS + np.abs(z) * eW) / W * (1 + 1e-6)
    rep = np.repeat(np.arange(len(st)), m.astype(np.int64))
    gy = wv * r[rep]
    tol_gy = 2 * out_eps * np.abs(gy) + wv * er[rep] + 1e-300
    if w is None:
        return tol_gy, None
    d = y - z[rep]
    gw = d * r[rep]
    tol_gw = 2 * out_eps * np.abs(gw) + np.abs(d) * er[rep] + ez[rep] * (np.abs(r[rep]) + er[rep]) + 1e-300
    return tol_gy, tol_gw


def parity_f64(y, w, out, z64, rel=1e-9):
    """The f64 rule, per element: |out - z| <= rel (1 + |z|), z the oracle's f64 fit.
    rel = 1e-9 reads the paper's f64 accuracy class (its float64 errors stay
    within 1.3e-10 of 1 + |z*| on every family, section 7.6) with a margin for
    a different summation order.  Returns (ok, worst ratio, row of worst)."""
    out = np.atleast_2d(np.asarray(out, np.float64))
    z64 = np.atleast_2d(np.asarray(z64, np.float64))
    ratio = np.abs(out - z64) / (rel * (1.0 + np.abs(z64)))
    worst = float(ratio.max()) if ratio.size else 0.0
    row = int(np.unravel_index(np.argmax(ratio), ratio.shape)[0]) if ratio.size else -1
    return worst <= 1.0, worst, row
