"""Test infrastructure: CPU oracle of the calibration front end.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this module; the GPU library never uses it.

What it computes (paper "Merge Hulls Without Copying Vertices: GPU Isotonic
Regression", section 7.7 "Case study: calibrating a click model", and the blog
note "Isotonic Regression on GPU"'s lab notebook, its calibration cells): an
isotonic calibration curve from scores and outcomes, in this order:

  1. key every score (with segments: the segment index plus the score, the
     score capped just below 1, so that the keys sort segment by segment);
  2. sort the keys, carrying the outcomes;
  3. pool equal keys: each distinct key xp gets the count of its scores and
     the mean of their outcomes;
  4. with segments, lift each pooled mean by twice its segment index, so that
     no block of the fit can reach across a segment boundary;
  5. fit the means with the counts as weights (the oracle's f64 PAVA);
  6. drop the lift again: fp, the curve's value at each xp.

A curve is applied to new scores by linear interpolation between the two
distinct keys around each score, held at the end values outside them (the
lab notebook's apply step).  With segments the search stays inside the
query's own segment (reading: the pages fit per-segment curves but show no
per-segment apply; a query never takes a value from another segment).

`mutant` plants one deliberate mistake (1: counts ignored as weights, 2: the
lift not dropped again, 3: no hold outside the end keys) so that the tests
can show their pins catch it; the default has none.
"""
from __future__ import annotations

import numpy as np

import oracle

CAP = 1.0 - 1e-12  # scores are capped just below 1 when keyed by segment


def keys_of(scores, segment=None):
    """f64 keys: the score, or segment + min(score, CAP)."""
    s = np.asarray(scores, np.float64)
    if segment is None:
        return s
    return np.asarray(segment, np.float64) + np.minimum(s, CAP)


def curve(scores, outcomes, segment=None, mutant: int = 0):
    """Returns (xp, fp, counts): the distinct keys in increasing order, the
    fitted curve at each, and the number of scores pooled into each."""
    keys = keys_of(scores, segment)
    o = np.asarray(outcomes, np.float64)
    order = np.argsort(keys, kind="stable")
    ks = keys[order]
    os_ = o[order]
    xp, first, counts = np.unique(ks, return_index=True, return_counts=True)
    sums = np.add.reduceat(os_, first)  # each run of equal keys, left to right
    means = sums / counts
    lift = np.zeros_like(means) if segment is None else 2.0 * np.floor(xp)
    wts = counts.astype(np.float64) if mutant != 1 else None
    z, _, _ = oracle.pava(means + lift, wts)
    fp = z - lift if mutant != 2 else z
    return xp, fp, counts


def apply(xp, fp, scores, segment=None, mutant: int = 0):
    """The curve (xp, fp) at new scores (keyed like the curve's)."""
    xp = np.asarray(xp, np.float64)
    fp = np.asarray(fp, np.float64)
    q = keys_of(scores, segment)
    out = np.empty(len(q), np.float64)
    if segment is None:
        lo_all = np.zeros(len(q), np.int64)
        hi_all = np.full(len(q), len(xp), np.int64)
    else:
        seg = np.asarray(segment, np.float64)
        lo_all = np.searchsorted(xp, seg, side="left")          # first key of the segment
        hi_all = np.searchsorted(xp, seg + 1.0, side="left")    # one past its last
    for j in range(len(q)):
        lo, hi = int(lo_all[j]), int(hi_all[j])
        if hi <= lo:
            out[j] = np.nan  # the segment has no curve
            continue
        if hi - lo == 1:
            out[j] = fp[lo]
            continue
        i = int(np.searchsorted(xp[lo:hi], q[j], side="left")) + lo
        i = min(max(i, lo + 1), hi - 1)
        t = (q[j] - xp[i - 1]) / max(xp[i] - xp[i - 1], 1e-300)
        if mutant != 3:
            t = min(max(t, 0.0), 1.0)
        out[j] = fp[i - 1] + t * (fp[i] - fp[i - 1])
    return out
