"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws numbers: it holds none of the fit's arithmetic, and both
the GPU path and the CPU oracle receive the arrays it returns.

Workloads (the shapes of the measurements in the paper "Merge Hulls Without
Copying Vertices: GPU Isotonic Regression", section 7, and of the note's lab
notebook):

* ``noisy(rows, n, seed)`` - a rising ramp 0..3 plus standard normal noise, in
  float32, the lab notebook's data of its first table.
* ``dense(n, seed)`` - a strictly increasing row: distinct points of the 2^-24
  grid in [0, 1), sorted.  Every point of its cumulative sum diagram is a hull
  vertex (the paper's "increasing" family).
* ``calibration(rows, n, seed)`` - per row, scores sorted ascending from
  N(-3.2, 1), clicks y ~ Bernoulli(sigmoid(score)) as 0/1 float32 and integer
  counts w ~ U{1..8} as float32 (the shape of the paper's click-model
  calibration, section 7.7; no records of any dataset are used).
* ``family(name, n, seed)`` and ``weights(kind, n, seed)`` - the paper's
  accuracy families and weightings (section 7.6), synthetic.
* ``click_scores(n, seed, segments)`` - unsorted f64 click-model scores with
  recurring values, 0/1 clicks and optional segment ids, for the calibration
  front end (section 7.7's shapes; no dataset records).
"""
from __future__ import annotations

import numpy as np

CONFIGS = {
    # name: (rows, n, kind, seed)
    "c1_row4096_noisy": (1, 4096, "noisy", 1),
    "c2_batch1024x1024_noisy": (1024, 1024, "noisy", 2),
    "c3_row1e7_noisy": (1, 10_000_000, "noisy", 3),
    "c4_row1e7_dense": (1, 10_000_000, "dense", 4),
    "c5_calib256x2p20": (256, 1 << 20, "calibration", 5),
}


def noisy(rows: int, n: int, seed: int):
    rng = np.random.default_rng(seed)
    y = np.linspace(0, 3, n, dtype=np.float32) + rng.standard_normal((rows, n), dtype=np.float32)
    return y.astype(np.float32, copy=False), None


def dense(n: int, seed: int, rows: int = 1):
    """Distinct multiples of 2^-24 in [0, 1), sorted: exact float32, strictly increasing."""
    rng = np.random.default_rng(seed)
    out = np.empty((rows, n), np.float32)
    for r in range(rows):
        k = np.sort(rng.choice(1 << 24, size=n, replace=False))
        out[r] = (k.astype(np.float64) * 2.0 ** -24).astype(np.float32)
    return out, None


def _sorted_normal(rng, rows: int, n: int, mean: float):
    """Sorted N(mean, 1) samples per row in O(n): sorted uniforms from normalised
    cumulative sums of exponentials (Renyi's representation), then the normal
    quantile function."""
    from scipy.special import ndtri

    e = rng.standard_exponential((rows, n + 1))
    c = np.cumsum(e, axis=1)
    u = c[:, :n] / c[:, n:n + 1]
    return mean + ndtri(u)


def calibration(rows: int, n: int, seed: int):
    rng = np.random.default_rng(seed)
    y = np.empty((rows, n), np.float32)
    w = np.empty((rows, n), np.float32)
    for r in range(rows):
        s = _sorted_normal(rng, 1, n, -3.2)[0]
        p = 1.0 / (1.0 + np.exp(-s))
        y[r] = (rng.random(n) < p).astype(np.float32)
        w[r] = rng.integers(1, 9, size=n).astype(np.float32)
    return y, w


def config(name: str, rows: int | None = None, n: int | None = None):
    """Inputs of a named workload, optionally with fewer rows or elements (same recipe)."""
    r0, n0, kind, seed = CONFIGS[name]
    rows = r0 if rows is None else rows
    n = n0 if n is None else n
    if kind == "noisy":
        return noisy(rows, n, seed)
    if kind == "dense":
        return dense(n, seed, rows)
    if kind == "calibration":
        return calibration(rows, n, seed)
    raise KeyError(kind)


FAMILIES = ("increasing", "decreasing", "constant", "piecewise", "gaussian", "random_walk",
            "sawtooth", "cliff", "collinear", "offset")


def family(name: str, n: int, seed: int) -> np.ndarray:
    """One float32 row of an accuracy family (paper section 7.6, synthetic)."""
    rng = np.random.default_rng(seed)
    t = np.arange(n, dtype=np.float64)
    if name == "increasing":
        y = np.sort(rng.random(n))
    elif name == "decreasing":
        y = -np.sort(rng.random(n))
    elif name == "constant":
        y = np.full(n, 0.75)
    elif name == "piecewise":
        k = max(1, n // 50)
        levels = rng.normal(0, 1, k)
        y = np.repeat(levels, -(-n // k))[:n] + 0.1 * rng.normal(0, 1, n)
    elif name == "gaussian":
        y = rng.normal(0, 1, n)
    elif name == "random_walk":
        y = np.cumsum(rng.normal(0, 1, n))
    elif name == "sawtooth":
        period = max(2, n // 37)
        y = (t % period) / period + 0.01 * t / max(n, 1)
    elif name == "cliff":
        y = np.linspace(0, 1, n) + 0.01 * rng.normal(0, 1, n)
        y[-1] = -1e3
    elif name == "collinear":
        y = 1.0 + 1e-7 * rng.normal(0, 1, n)
    elif name == "offset":
        y = 1e6 + np.linspace(0, 3, n) + rng.normal(0, 1, n)
    else:
        raise KeyError(name)
    return y.astype(np.float32)


WEIGHTINGS = ("none", "uniform", "exp")


def weights(kind: str, n: int, seed: int):
    """None, U[0.1, 1.1] or e^U[0, 8] weights (paper section 7.6)."""
    if kind == "none":
        return None
    rng = np.random.default_rng(seed + 7919)
    if kind == "uniform":
        return (0.1 + rng.random(n)).astype(np.float32)
    if kind == "exp":
        return np.exp(8.0 * rng.random(n)).astype(np.float32)
    raise KeyError(kind)


def cancellation(n: int, big: float, seed: int) -> np.ndarray:
    """Per 64 elements: 32 values of +B, one of -32B and 31 small nearly collinear
    values (the paper's cancellation family, section 7.6)."""
    rng = np.random.default_rng(seed)
    y = np.empty(n, np.float64)
    for s in range(0, n, 64):
        blk = np.concatenate([np.full(32, big), [-32.0 * big],
                              1.0 + 1e-3 * np.arange(31) + 1e-9 * rng.normal(0, 1, 31)])
        y[s:s + 64] = blk[:min(64, n - s)]
    return y.astype(np.float32)


def consecutive_floats(n: int, start: float = 1.0) -> np.ndarray:
    """n consecutive float32 values upward from ``start``: every point its own block."""
    base = np.array([start], np.float32).view(np.int32)[0]
    return (base + np.arange(n, dtype=np.int64)).astype(np.int32).view(np.float32)


def click_scores(n: int, seed: int, segments: int = 0, keep: float = 0.1):
    """Synthetic stand-in for the paper's click-model calibration (section 7.7;
    no records of its dataset are used): a model's predicted click
    probabilities and the observed clicks, f64.

    Scores are sigmoid(logit) of logits ~ N(-1.5, 1.2^2), rounded to float32
    precision so that equal scores recur (as repeated feature vectors give
    repeated scores).  The model is taken to have been trained with only a
    fraction `keep` of the non-clicks, so its probabilities are too high; a
    click is drawn with the probability keep*s / (keep*s + 1 - s).  With
    `segments`, each score also gets a segment index in [0, segments) drawn
    with probabilities proportional to 1/(j+1)^1.1 (a few large segments and a
    long tail).  Returns (scores, clicks, segment or None)."""
    rng = np.random.default_rng(seed)
    logit = rng.normal(-1.5, 1.2, n)
    s = (1.0 / (1.0 + np.exp(-logit))).astype(np.float32).astype(np.float64)
    p = keep * s / (keep * s + 1.0 - s)
    y = (rng.random(n) < p).astype(np.float64)
    seg = None
    if segments:
        pr = 1.0 / np.arange(1, segments + 1) ** 1.1
        seg = rng.choice(segments, size=n, p=pr / pr.sum()).astype(np.int32)
    return s, y, seg
