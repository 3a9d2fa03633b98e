"""Pins of the CPU oracle against what the pages and the mathematics fix.

The oracle (oracle/iso_oracle.c) is weighted pool adjacent violators in f64.
It is checked here against things other than itself:
  * the worked examples printed on the pages (tests/golden/),
  * brute force over all contiguous partitions for n <= 12,
  * the KKT prefix conditions of the problem,
  * idempotence on non-decreasing inputs, ties included,
  * closed forms (constant, strictly decreasing, two elements, strictly increasing),
  * the slopes of the lower hull of the cumulative sum diagram (a second route),
  * exact rational arithmetic on integer data,
  * scipy's isotonic_regression, a library routine for the same problem.
Each planted mistake in the oracle (compile switch ORACLE_MUTANT) must fail at
least one of these pins (test_planted_mistakes_are_caught).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle
from lower_convex_hull_amd import inputs
from tests import fitcheck

MUTANTS = range(1, 7)


# ----------------------------------------------------------------------------- pins

def pin_golden(mutant=0):
    fails = []
    for c in fitcheck.read_cases("worked_examples.txt"):
        y = np.array([float(v) for v in c["y"]])
        w = None if c["w"] is None else np.array([float(v) for v in c["w"]])
        z, _, _ = oracle.pava(y, w, mutant=mutant)
        want = np.array([float(v) for v in c["z"]])
        if not np.allclose(z, want, rtol=0, atol=1e-14):
            fails.append(f"golden {c['case']}: {z} != {want}")
    return fails


def _small_cases(seed0, count):
    rng = np.random.default_rng(seed0)
    for k in range(count):
        n = int(rng.integers(1, 13))
        kind = k % 3
        if kind == 0:  # integers with ties
            y = rng.integers(-3, 4, n).astype(np.float64)
        elif kind == 1:
            y = rng.normal(0, 1, n)
        else:
            y = np.cumsum(rng.normal(0, 1, n))
        wk = (k // 3) % 3
        w = None if wk == 0 else (0.1 + rng.random(n) if wk == 1 else np.exp(8 * rng.random(n)))
        yield y, w


def pin_brute_force(mutant=0, count=600):
    fails = []
    for y, w in _small_cases(11, count):
        zb, eb = oracle.brute_force(y, w)
        z, _, _ = oracle.pava(y, w, mutant=mutant)
        e = fitcheck.objective(y, w, z)
        scale = 1.0 + np.abs(y).max()
        if not (np.abs(z - zb).max() <= 1e-12 * scale and abs(e - eb) <= 1e-12 * max(1.0, eb)):
            fails.append(f"brute force n={len(y)} y={y.tolist()} w={None if w is None else w.tolist()}")
            if len(fails) > 3:
                break
    return fails


def pin_kkt(mutant=0):
    fails = []
    for fi, fam in enumerate(inputs.FAMILIES):
        for wk in inputs.WEIGHTINGS:
            n = 5000
            y = inputs.family(fam, n, 100 + fi).astype(np.float64)
            w = inputs.weights(wk, n, 100 + fi)
            z, _, _ = oracle.pava(y, w, mutant=mutant)
            # rounding of f64 sums over large offsets sets the floor of tau
            tau = 1e-12 if fam != "offset" else 1e-9
            if not fitcheck.kkt_ok(y, w, z, tau=tau):
                fails.append(f"kkt {fam}/{wk}: {fitcheck.kkt_violation(y, w, z)}")
    return fails


def pin_idempotent(mutant=0):
    fails = []
    rng = np.random.default_rng(5)
    for k in range(40):
        n = int(rng.integers(1, 300))
        y = np.sort(rng.integers(0, 20, n).astype(np.float64))  # ties included
        # f32-representable weights, as the library takes: w*y is exact in f64
        w = None if k % 2 == 0 else (0.1 + rng.random(n)).astype(np.float32).astype(np.float64)
        z, _, _ = oracle.pava(y, w, mutant=mutant)
        # ties are pooled (reading: a point on a chord is not a vertex), so with
        # non-unit weights a tied block's mean may differ from y by rounding only
        ok = np.array_equal(z, y) if w is None else np.allclose(z, y, rtol=1e-14, atol=0)
        if not ok:
            fails.append(f"idempotence n={n}")
    return fails


def pin_closed_forms(mutant=0):
    fails = []
    rng = np.random.default_rng(9)
    # constant row: identity
    z, _, nb = oracle.pava(np.full(50, 2.5), None, mutant=mutant)
    if not np.all(z == 2.5):
        fails.append("constant")
    # strictly decreasing row: one block at the weighted mean
    y = -np.sort(rng.random(64))
    w = 0.1 + rng.random(64)
    z, _, nb = oracle.pava(y, w, mutant=mutant)
    if not (np.allclose(z, np.sum(w * y) / np.sum(w), rtol=0, atol=1e-14) and nb == 1):
        fails.append("decreasing")
    # two elements a > b: the weighted mean
    for a, b, wa, wb in ((3.0, 1.0, 1.0, 3.0), (2.0, -2.0, 0.5, 1.5), (1.0, 0.0, 7.0, 1.0)):
        z, _, _ = oracle.pava(np.array([a, b]), np.array([wa, wb]), mutant=mutant)
        m = (wa * a + wb * b) / (wa + wb)
        if not np.allclose(z, [m, m], rtol=0, atol=1e-15):
            fails.append(f"pair {a},{b}")
    # strictly increasing row: identity with n blocks
    # f32-representable data and weights (as the library takes): w*y/w == y exactly
    y = np.unique(rng.random(400).astype(np.float32))[:200].astype(np.float64)
    wi = (0.5 + rng.random(200)).astype(np.float32).astype(np.float64)
    z, _, nb = oracle.pava(y, wi, mutant=mutant)
    if not (np.array_equal(z, y) and nb == 200):
        fails.append("increasing")
    return fails


def pin_exact_rational(mutant=0):
    """Integer data (as in the calibration workload): every sum is exact in f64, so
    the f64 fit equals the rational fit of brute force in exact arithmetic."""
    fails = []
    rng = np.random.default_rng(21)
    for k in range(120):
        n = int(rng.integers(1, 10))
        y = rng.integers(0, 2, n)
        w = rng.integers(1, 9, n)
        best = None
        for cuts in range(1 << (n - 1)):
            bounds = [0] + [i + 1 for i in range(n - 1) if (cuts >> i) & 1] + [n]
            means = [Fraction(int(np.dot(w[a:b], y[a:b])), int(w[a:b].sum()))
                     for a, b in zip(bounds[:-1], bounds[1:])]
            if any(m2 < m1 for m1, m2 in zip(means[:-1], means[1:])):
                continue
            zz = []
            for (a, b), m in zip(zip(bounds[:-1], bounds[1:]), means):
                zz += [m] * (b - a)
            err = sum(int(w[i]) * (zz[i] - int(y[i])) ** 2 for i in range(n))
            if best is None or err < best[0]:
                best = (err, zz)
        z, _, _ = oracle.pava(y.astype(np.float64), w.astype(np.float64), mutant=mutant)
        want = np.array([float(v) for v in best[1]])
        if not np.array_equal(z, want):
            fails.append(f"rational y={y.tolist()} w={w.tolist()}")
            if len(fails) > 3:
                break
    return fails


def pin_hull_route(mutant=0):
    fails = []
    for fi, fam in enumerate(("gaussian", "random_walk", "sawtooth", "piecewise", "cliff")):
        for wk in inputs.WEIGHTINGS:
            y = inputs.family(fam, 20000, 300 + fi).astype(np.float64)
            w = inputs.weights(wk, 20000, 300 + fi)
            z, _, _ = oracle.pava(y, w, mutant=mutant)
            zh, _ = oracle.hull_fit(y, w)
            scale = 1.0 + np.abs(y).max()
            if np.abs(z - zh).max() > 1e-9 * scale:
                fails.append(f"hull route {fam}/{wk}: {np.abs(z - zh).max()}")
    return fails


ALL_PINS = (pin_golden, pin_brute_force, pin_kkt, pin_idempotent, pin_closed_forms,
            pin_exact_rational, pin_hull_route)


# ----------------------------------------------------------------------------- tests

@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    fails = pin()
    assert not fails, "\n".join(fails)


def test_golden_running_totals_match_hull_route():
    """The printed running totals of [1,3,2,4] (P_0 = 0) give, through their lower
    hull, the same fit as the first worked example."""
    g = fitcheck.read_single("csd_running_totals.txt")
    y = np.array([float(v) for v in g["y"]])
    S = g["S"]
    assert S[0] == 0 and all(S[k + 1] - S[k] == g["y"][k] for k in range(len(y)))
    zh, nv = oracle.hull_fit(y)
    assert nv == 4  # P_2 = (2, 4) lies above the chord from (1, 1) to (3, 6)
    assert np.allclose(zh, [1, 2.5, 2.5, 4], rtol=0, atol=1e-15)


def test_hull_route_is_exact_on_small_cases():
    for y, w in _small_cases(77, 300):
        zb, _ = oracle.brute_force(y, w)
        zh, _ = oracle.hull_fit(y, w)
        assert np.abs(zh - zb).max() <= 1e-12 * (1 + np.abs(y).max())


def test_block_ids_are_canonical():
    """Blocks have strictly increasing means and partition the row (Mova card,
    entry "Invariant"); block ids are 0-based and rise by one at each start."""
    y = inputs.family("gaussian", 3000, 3).astype(np.float64)
    w = inputs.weights("uniform", 3000, 3).astype(np.float64)
    z, bid, nb = oracle.pava(y, w)
    assert bid[0] == 0 and bid[-1] == nb - 1
    assert set(np.diff(bid).tolist()) <= {0, 1}
    starts = np.flatnonzero(np.diff(bid)) + 1
    assert np.all(z[starts] > z[starts - 1])
    for b in range(nb):
        idx = bid == b
        assert np.isclose(z[idx][0], np.sum(w[idx] * y[idx]) / np.sum(w[idx]), rtol=1e-13)


def test_f32_rows_round_once():
    y, w = inputs.calibration(3, 4096, 5)
    out, out64, bid = oracle.fit_rows_f32(y, w)
    assert np.array_equal(out, out64.astype(np.float32))
    for r in range(3):
        z, b, _ = oracle.pava(y[r].astype(np.float64), w[r].astype(np.float64))
        assert np.array_equal(out64[r], z) and np.array_equal(bid[r], b)


def test_dense_row_is_identity():
    """A strictly increasing row is its own fit, each point a block (closed form
    for the dense-hull workload)."""
    y, _ = inputs.dense(200_000, 4)
    assert np.all(np.diff(y[0].astype(np.float64)) > 0)
    out, out64, bid = oracle.fit_rows_f32(y)
    assert np.array_equal(out[0], y[0]) and bid[0, -1] == 200_000 - 1


def test_library_routine_agrees():
    """scipy's isotonic_regression solves the same problem (the paper checks its
    f64 reference against SciPy, section 7.6)."""
    opt = pytest.importorskip("scipy.optimize")
    if not hasattr(opt, "isotonic_regression"):
        pytest.skip("scipy too old")
    for fam in ("gaussian", "random_walk", "sawtooth"):
        y = inputs.family(fam, 10000, 8).astype(np.float64)
        w = inputs.weights("uniform", 10000, 8).astype(np.float64)
        ref = opt.isotonic_regression(y, weights=w, increasing=True).x
        z, _, _ = oracle.pava(y, w)
        assert np.abs(z - ref).max() <= 1e-10 * (1 + np.abs(y).max())


@pytest.mark.parametrize("mutant", MUTANTS)
def test_planted_mistakes_are_caught(mutant):
    caught = []
    for pin in (pin_golden, pin_closed_forms, pin_idempotent, pin_exact_rational):
        if pin(mutant=mutant):
            caught.append(pin.__name__)
    if not caught:
        if pin_brute_force(mutant=mutant, count=200):
            caught.append("pin_brute_force")
    assert caught, f"mutant {mutant} passed every pin"


# ----------------------------------------------------------------------------- VJP pins
# The vector-Jacobian product of the fit (paper section 6, "Gradient"; the
# paper's appendix C checks it against finite differences in y and in w in
# float64 and against block sums).

VJP_MUTANTS = range(7, 11)


def _generic_cases(seed0, count, nmax=24):
    """Continuous data (no ties, blocks stable under tiny perturbations)."""
    rng = np.random.default_rng(seed0)
    for k in range(count):
        n = int(rng.integers(1, nmax + 1))
        y = rng.normal(0, 1, n) + (np.linspace(0, 2, n) if k % 2 else 0.0)
        wk = k % 3
        w = None if wk == 0 else (0.1 + rng.random(n) if wk == 1 else np.exp(4 * rng.random(n)))
        g = rng.normal(0, 1, n)
        yield y, w, g


def _fd(fit, y, w, g, h):
    """Central differences of L = g . fit(y, w) in every y_i and w_i."""
    n = len(y)
    dy = np.empty(n)
    dw = None if w is None else np.empty(n)
    for i in range(n):
        e = np.zeros(n)
        e[i] = h
        dy[i] = (g @ fit(y + e, w) - g @ fit(y - e, w)) / (2 * h)
        if w is not None:
            dw[i] = (g @ fit(y, w + e) - g @ fit(y, w - e)) / (2 * h)
    return dy, dw


def pin_vjp_finite_differences(mutant=0, count=90):
    fails = []
    fit = lambda y, w: oracle.pava(y, w)[0]
    for y, w, g in _generic_cases(71, count):
        gy, gw = oracle.vjp(y, w, g, mutant=mutant)
        dy, dw = _fd(fit, y, w, g, 1e-6)
        tol = 1e-6 * (1.0 + np.abs(g).sum())
        bad = np.abs(gy - dy).max() > tol or (w is not None and np.abs(gw - dw).max() > tol)
        if bad:
            fails.append(f"vjp finite differences n={len(y)} weighted={w is not None}")
            if len(fails) > 3:
                break
    return fails


def pin_vjp_brute_force_route(mutant=0, count=60):
    """The same finite differences taken on the brute-force fit (n <= 10), so
    the blocks the product averages over are pinned independently of PAVA."""
    fails = []
    fit = lambda y, w: oracle.brute_force(y, w)[0]
    for y, w, g in _generic_cases(73, count, nmax=10):
        gy, gw = oracle.vjp(y, w, g, mutant=mutant)
        dy, dw = _fd(fit, y, w, g, 1e-6)
        tol = 1e-6 * (1.0 + np.abs(g).sum())
        if np.abs(gy - dy).max() > tol or (w is not None and np.abs(gw - dw).max() > tol):
            fails.append(f"vjp brute-force route n={len(y)}")
    return fails


def pin_vjp_closed_forms(mutant=0):
    fails = []
    rng = np.random.default_rng(17)
    n = 300
    g = rng.normal(0, 1, n)
    w = 0.2 + rng.random(n)
    # strictly increasing: every element its own block, d/dy = g, d/dw = 0
    y = np.sort(rng.random(n))
    gy, gw = oracle.vjp(y, w, g, mutant=mutant)
    if not (np.allclose(gy, g, rtol=1e-14, atol=1e-15) and np.allclose(gw, 0.0, atol=1e-15)):
        fails.append("vjp increasing")
    # strictly decreasing: one block; d/dy_i = w_i sum(g)/sum(w), d/dw_i = (y_i - mean) sum(g)/sum(w)
    y = -np.sort(rng.random(n))
    gy, gw = oracle.vjp(y, w, g, mutant=mutant)
    r = g.sum() / w.sum()
    m = (w * y).sum() / w.sum()
    if not (np.allclose(gy, w * r, rtol=1e-12, atol=1e-14) and np.allclose(gw, (y - m) * r, rtol=1e-10, atol=1e-14)):
        fails.append("vjp decreasing")
    # unit weights, constant row: the mean of g everywhere
    gy, gw = oracle.vjp(np.full(n, 0.5), None, g, mutant=mutant)
    if not np.allclose(gy, g.mean(), rtol=1e-12, atol=1e-14) or gw is not None:
        fails.append("vjp constant")
    return fails


def pin_vjp_block_sums(mutant=0):
    """Over any given partition, d/dy summed over a block is G, and w-weighted
    d/dw summed over a block is zero (z is the block's weighted mean)."""
    fails = []
    rng = np.random.default_rng(19)
    for k in range(30):
        n = int(rng.integers(2, 400))
        y = rng.normal(0, 1, n)
        w = 0.1 + rng.random(n)
        g = rng.normal(0, 1, n)
        starts = np.sort(rng.choice(np.arange(1, n), size=int(rng.integers(0, n // 3 + 1)), replace=False))
        bid = np.zeros(n, np.int32)
        bid[starts] = 1
        bid = np.cumsum(bid).astype(np.int32)
        gy, gw = oracle.vjp(y, w, g, block_id=bid, mutant=mutant)
        for b in range(bid[-1] + 1):
            idx = bid == b
            if abs(gy[idx].sum() - g[idx].sum()) > 1e-12 * (1 + np.abs(g[idx]).sum()):
                fails.append(f"vjp block sum d/dy block {b}")
                break
            if abs((w[idx] * gw[idx]).sum()) > 1e-12 * (1 + np.abs(w[idx] * gw[idx]).sum() + abs(g[idx].sum())):
                fails.append(f"vjp block sum d/dw block {b}")
                break
    return fails


VJP_PINS = (pin_vjp_finite_differences, pin_vjp_brute_force_route, pin_vjp_closed_forms,
            pin_vjp_block_sums)


@pytest.mark.parametrize("pin", VJP_PINS, ids=lambda p: p.__name__)
def test_oracle_vjp_pin(pin):
    fails = pin()
    assert not fails, "\n".join(fails)


def test_oracle_vjp_rows_match_single_rows():
    y, w = inputs.calibration(3, 5000, 12)
    g = np.random.default_rng(3).normal(0, 1, y.shape).astype(np.float32)
    _, _, bid = oracle.fit_rows_f32(y, w)
    gy, gw = oracle.vjp_rows_f32(y, w, g, bid)
    for r in range(3):
        a, b = oracle.vjp(y[r], w[r], g[r])
        assert np.array_equal(gy[r], a) and np.array_equal(gw[r], b)
    bid[1, :] = -1  # a non-finite row of the fit
    gy, gw = oracle.vjp_rows_f32(y, w, g, bid)
    assert np.all(np.isnan(gy[1])) and np.all(np.isnan(gw[1])) and not np.isnan(gy[[0, 2]]).any()


@pytest.mark.parametrize("mutant", VJP_MUTANTS)
def test_planted_vjp_mistakes_are_caught(mutant):
    caught = [p.__name__ for p in (pin_vjp_closed_forms, pin_vjp_block_sums) if p(mutant=mutant)]
    if not caught and pin_vjp_finite_differences(mutant=mutant, count=30):
        caught.append("pin_vjp_finite_differences")
    assert caught, f"mutant {mutant} passed every VJP pin"
