"""Pins of the calibration oracle (oracle/calib.py) against what the pages and
the mathematics fix, none of them the oracle itself:
  * scikit-learn's IsotonicRegression with clipping, the reference the paper's
    calibration is checked against (section 7.7), on scores with ties;
  * brute force over the contiguous partitions of the sorted scores that keep
    equal scores together (the least-squares fit with ties sharing a value);
  * per-segment curves equal curves fitted on each segment alone;
  * the blog note's worked clicks example (tests/golden/worked_examples.txt);
  * closed forms of the interpolation.
Each planted mistake of the oracle must fail at least one pin."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import calib
from tests import fitcheck


def _tied_scores(rng, n, grid):
    return np.round(rng.random(n) * grid) / grid


def pin_sklearn(mutant=0):
    skl = pytest.importorskip("sklearn.isotonic")
    fails = []
    rng = np.random.default_rng(1)
    for k, (n, grid) in enumerate(((3000, 100), (20000, 1000), (500, 7), (4000, 1e9))):
        s = _tied_scores(rng, n, grid)
        y = (rng.random(n) < 0.2 + 0.5 * s).astype(np.float64) if k % 2 == 0 else rng.normal(s, 0.3)
        xp, fp, counts = calib.curve(s, y, mutant=mutant)
        ir = skl.IsotonicRegression(out_of_bounds="clip").fit(s, y)
        if np.abs(ir.predict(xp) - fp).max() > 1e-12 or counts.sum() != n:
            fails.append(f"sklearn curve n={n} grid={grid}")
        q = rng.random(500) * 1.4 - 0.2
        if np.abs(ir.predict(q) - calib.apply(xp, fp, q, mutant=mutant)).max() > 1e-12:
            fails.append(f"sklearn apply n={n} grid={grid}")
    return fails


def pin_tied_brute_force(mutant=0):
    """n <= 10 scores with ties: the least-squares non-decreasing fit in which
    equal scores share one value, over every admissible partition."""
    fails = []
    rng = np.random.default_rng(2)
    for _ in range(150):
        n = int(rng.integers(1, 11))
        s = rng.integers(0, 5, n).astype(np.float64)
        y = rng.integers(0, 2, n).astype(np.float64) if rng.random() < 0.5 else rng.normal(0, 1, n)
        order = np.argsort(s, kind="stable")
        ss, ys = s[order], y[order]
        best = None
        for cuts in range(1 << (n - 1)):
            ok = all(not ((cuts >> i) & 1) or ss[i] != ss[i + 1] for i in range(n - 1))
            if not ok:
                continue
            bounds = [0] + [i + 1 for i in range(n - 1) if (cuts >> i) & 1] + [n]
            means = [ys[a:b].mean() for a, b in zip(bounds[:-1], bounds[1:])]
            if any(m2 < m1 for m1, m2 in zip(means[:-1], means[1:])):
                continue
            f = np.concatenate([np.full(b - a, m) for (a, b), m in zip(zip(bounds[:-1], bounds[1:]), means)])
            err = float(((f - ys) ** 2).sum())
            if best is None or err < best[0] - 1e-12:
                best = (err, f)
        xp, fp, _ = calib.curve(s, y, mutant=mutant)
        got = fp[np.searchsorted(xp, ss)]
        if np.abs(got - best[1]).max() > 1e-12:
            fails.append(f"tied brute force s={s.tolist()} y={y.tolist()}")
            if len(fails) > 3:
                break
    return fails


def pin_segments_independent(mutant=0):
    fails = []
    rng = np.random.default_rng(3)
    nseg = 12
    n = 6000
    seg = rng.integers(0, nseg, n)
    seg[seg == 5] = 6  # one segment without scores
    s = _tied_scores(rng, n, 200)
    s[rng.random(n) < 0.01] = 1.0  # scores at the top, capped below 1
    y = (rng.random(n) < np.clip(0.1 + 0.3 * s + 0.05 * seg, 0, 1)).astype(np.float64)
    xp, fp, counts = calib.curve(s, y, seg, mutant=mutant)
    for j in range(nseg):
        m = seg == j
        got = (np.floor(xp) == j)
        if not m.any():
            if got.any():
                fails.append(f"segment {j} should be empty")
            continue
        xj, fj, cj = calib.curve(np.minimum(s[m], calib.CAP), y[m], mutant=mutant)
        if not (np.array_equal(xp[got] - j, xj) or np.allclose(xp[got] - j, xj, rtol=0, atol=1e-12)):
            fails.append(f"segment {j} keys")
        elif np.abs(fp[got] - fj).max() > 1e-12 or not np.array_equal(counts[got], cj):
            fails.append(f"segment {j} curve")
    q = rng.random(400)
    qs = rng.integers(0, nseg, 400)
    a = calib.apply(xp, fp, q, qs, mutant=mutant)
    for j in range(nseg):
        m = qs == j
        got = np.floor(xp) == j
        if not got.any():
            if not np.all(np.isnan(a[m])):
                fails.append(f"apply to empty segment {j}")
            continue
        xj, fj, _ = calib.curve(np.minimum(s[seg == j], calib.CAP), y[seg == j])
        if np.abs(a[m] - calib.apply(xj, fj, np.minimum(q[m], calib.CAP))).max() > 1e-12:
            fails.append(f"apply segment {j}")
    return fails


def pin_golden_clicks(mutant=0):
    fails = []
    for c in fitcheck.read_cases("worked_examples.txt"):
        if c["case"] != "clicks_zero_one":
            continue
        y = np.array([float(v) for v in c["y"]])
        want = np.array([float(v) for v in c["z"]])
        s = np.arange(1, len(y) + 1, dtype=np.float64) / 16.0  # sorted, distinct scores
        xp, fp, _ = calib.curve(s[::-1].copy(), y[::-1].copy(), mutant=mutant)
        if not np.allclose(fp, want, rtol=0, atol=1e-15):
            fails.append("golden clicks")
        # the same scores repeated twice pool into counts of 2 with the same fit
        xp2, fp2, c2 = calib.curve(np.concatenate([s, s]), np.concatenate([y, y]), mutant=mutant)
        if not (np.allclose(fp2, want, rtol=0, atol=1e-15) and np.all(c2 == 2)):
            fails.append("golden clicks pooled")
    return fails


def pin_apply_closed_forms(mutant=0):
    fails = []
    xp = np.array([0.1, 0.4, 0.5, 0.9])
    fp = np.array([0.0, 0.2, 0.2, 1.0])
    q = np.array([0.1, 0.4, 0.5, 0.9, -3.0, 7.0, 0.25, 0.7])
    want = np.array([0.0, 0.2, 0.2, 1.0, 0.0, 1.0, 0.1, 0.6])
    if np.abs(calib.apply(xp, fp, q, mutant=mutant) - want).max() > 1e-15:
        fails.append("apply closed forms")
    if np.abs(calib.apply(xp[:1], fp[:1], q, mutant=mutant) - 0.0).max() > 0:
        fails.append("apply one key")
    return fails


PINS = (pin_sklearn, pin_tied_brute_force, pin_segments_independent, pin_golden_clicks,
        pin_apply_closed_forms)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_calib_oracle_pin(pin):
    fails = pin()
    assert not fails, "\n".join(fails)


@pytest.mark.parametrize("mutant", [1, 2, 3])
def test_planted_calib_mistakes_are_caught(mutant):
    caught = [p.__name__ for p in PINS if p(mutant=mutant)]
    assert caught, f"calibration mutant {mutant} passed every pin"
