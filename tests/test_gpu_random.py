"""Seeded random fits against the oracle: shapes from one element to rows of
a dozen groups of chunks, every accuracy family, with and without weights,
increasing and decreasing fits, block ids checked (paper section 7.6's
families; the tolerance of tests/fitcheck.py)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from lower_convex_hull_amd import inputs, iso
from tests import fitcheck

pytestmark = pytest.mark.gpu

G = 64 * 4096
FAMILIES = ["gaussian", "random_walk", "piecewise", "sawtooth", "cliff", "collinear", "offset", "increasing",
            "decreasing"]


@pytest.fixture(scope="module")
def torch():
    import torch as t

    assert t.cuda.is_available()
    iso.lib()
    return t


@pytest.mark.parametrize("seed", [5, 6])
def test_random_shapes_families_weights_and_directions(torch, seed):
    from tests.test_gpu_parity import gpu_fit

    rng = np.random.default_rng(seed)
    for case in range(120):
        size = rng.integers(0, 4)
        n = int([rng.integers(1, 4097), rng.integers(4097, 300_000), rng.integers(300_000, 2 * G),
                 rng.integers(2 * G, 12 * G)][size])
        rows = int(rng.integers(1, 9 if n < 300_000 else 3))
        fam = FAMILIES[rng.integers(0, len(FAMILIES))]
        y = np.stack([inputs.family(fam, n, int(rng.integers(0, 1 << 30))) for _ in range(rows)])
        if rng.random() < 0.3:
            y = (y + float(rng.uniform(-2, 2)) * np.linspace(0, 1, n)[None, :]).astype(np.float32)
        wk = ["none", "uniform", "exp"][rng.integers(0, 3)]
        w = None if wk == "none" else np.stack([inputs.weights(wk, n, int(rng.integers(0, 1 << 30)))
                                                for _ in range(rows)])
        dec = bool(rng.random() < 0.2)
        name = f"seed {seed} case {case}: rows={rows} n={n} {fam} weights={wk} decreasing={dec}"
        st, out, bid = gpu_fit(torch, y, w, iso.ISO_F_DECREASING if dec else 0, True)
        assert st == iso.ISO_OK, (name, iso.iso_status_str(st))
        _, z64, obid = oracle.fit_rows_f32(-y if dec else y, w)
        if dec:
            z64 = -z64
        ok, wa, wo, r = fitcheck.parity(y, w, out, z64)
        assert ok, (name, wa, wo, r)
        for i in range(rows):
            assert fitcheck.block_ids_consistent(obid[i], bid[i], z64[i], y[i]), (name, i)
