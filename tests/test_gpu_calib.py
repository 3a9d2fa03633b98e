"""GPU parity of the calibration front end (iso_calib_fit, iso_calib_apply)
against the CPU calibration oracle (oracle/calib.py): the distinct keys bit for
bit, the fitted curve under the f64 fit rule (tests/fitcheck.parity_f64), and
the interpolated values within what the curve's own difference allows."""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest

from lower_convex_hull_amd import inputs, iso
from oracle import calib
from tests import fitcheck

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as t

    assert t.cuda.is_available()
    iso.lib()
    return t


def gpu_curve(torch, s, y, seg=None):
    st_ = torch.from_numpy(np.ascontiguousarray(s, np.float64)).cuda()
    yt = torch.from_numpy(np.ascontiguousarray(y, np.float64)).cuda()
    gt = None if seg is None else torch.from_numpy(np.ascontiguousarray(seg, np.int32)).cuda()
    n = len(s)
    xp = torch.empty(max(n, 1), dtype=torch.float64, device="cuda")
    fp = torch.empty_like(xp)
    nb = iso.iso_calib_workspace_bytes(max(n, 1))
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")
    k = ctypes.c_int64(-1)
    rc = iso.iso_calib_fit(st_.data_ptr(), yt.data_ptr(), None if gt is None else gt.data_ptr(), n,
                           xp.data_ptr(), fp.data_ptr(), k, ws.data_ptr(), nb, iso._stream_handle(None))
    torch.cuda.synchronize()
    return rc, xp[:k.value].cpu().numpy(), fp[:k.value].cpu().numpy(), (xp, fp, k.value)


def gpu_apply(torch, xp_t, fp_t, k, q, qseg=None):
    qt = torch.from_numpy(np.ascontiguousarray(q, np.float64)).cuda()
    gt = None if qseg is None else torch.from_numpy(np.ascontiguousarray(qseg, np.int32)).cuda()
    out = torch.empty_like(qt)
    rc = iso.iso_calib_apply(xp_t.data_ptr(), fp_t.data_ptr(), k, qt.data_ptr(),
                             None if gt is None else gt.data_ptr(), len(q), out.data_ptr(),
                             iso._stream_handle(None))
    torch.cuda.synchronize()
    return rc, out.cpu().numpy()


def check(torch, s, y, seg=None, name="", nq=100_000):
    say(f"[calib] {name} n={len(s)} segments={'-' if seg is None else int(seg.max()) + 1}")
    rc, xp, fp, dev = gpu_curve(torch, s, y, seg)
    assert rc == iso.ISO_OK, iso.iso_status_str(rc)
    oxp, ofp, _ = calib.curve(s, y, seg)
    assert np.array_equal(xp, oxp), f"{name}: distinct keys differ"
    ok, worst, _ = fitcheck.parity_f64(None, None, fp[None, :], ofp[None, :])
    say(f"[calib]   {len(xp)} distinct keys; max |fp - oracle| / (1 + |fp|) = {worst * 1e-9:.3g}")
    assert ok, f"{name}: curve ratio {worst:.3g}"
    rng = np.random.default_rng(len(s))
    q = np.concatenate([rng.random(nq) * 1.2 - 0.1, oxp[: min(len(oxp), 1000)] - (0 if seg is None else np.floor(oxp[:1000]))])
    qseg = None if seg is None else rng.integers(-1, int(seg.max()) + 2, len(q)).astype(np.int32)
    if qseg is not None:
        q = np.abs(q)
    rc, out = gpu_apply(torch, dev[0], dev[1], dev[2], q, qseg)
    assert rc == iso.ISO_OK
    want = calib.apply(oxp, ofp, q, qseg)
    # interpolation is a convex combination of two curve values: its error is
    # at most the curve's, plus rounding of the combination
    tol = 1e-9 * (1.0 + np.abs(ofp).max()) + 4 * 2.0 ** -53 * np.abs(want)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(out), nan), f"{name}: NaN pattern of apply"
    assert np.all(np.abs(out[~nan] - want[~nan]) <= tol[~nan]), f"{name}: apply"


def test_calib_one_curve_day(torch):
    """One curve over 6.5 million scores (the size of the paper's one-day curve)."""
    s, y, _ = inputs.click_scores(6_500_000, 71)
    check(torch, s, y, name="one curve 6.5e6")


def test_calib_segment_curves(torch):
    """280 curves laid end to end in one problem (the paper's per-segment curves)."""
    s, y, seg = inputs.click_scores(2_000_000, 72, segments=280)
    check(torch, s, y, seg, name="280 segments")


@pytest.mark.parametrize("n", [1, 2, 3, 1000, 4096, 4097, 100_000])
def test_calib_sizes_and_ties(torch, n):
    rng = np.random.default_rng(n)
    s = np.round(rng.random(n) * 50) / 50  # heavy ties
    y = rng.normal(s, 0.2)                   # real-valued outcomes
    check(torch, s, y, name=f"ties n={n}", nq=2000)
    s2 = rng.random(n)                        # all distinct
    check(torch, s2, (rng.random(n) < s2).astype(np.float64), name=f"distinct n={n}", nq=2000)
    seg = rng.integers(0, 7, n).astype(np.int32)
    check(torch, s2, y, seg, name=f"segments n={n}", nq=2000)


def test_calib_constant_scores_and_errors(torch):
    s = np.full(5000, 0.25)
    y = (np.arange(5000) % 3 == 0).astype(np.float64)
    rc, xp, fp, _ = gpu_curve(torch, s, y)
    assert rc == 0 and np.array_equal(xp, [0.25]) and abs(fp[0] - y.mean()) <= 1e-15
    bad = s.copy()
    bad[17] = np.nan
    assert gpu_curve(torch, bad, y)[0] == iso.ISO_ERR_DATA
    seg = np.zeros(5000, np.int32)
    seg[3] = -1
    assert gpu_curve(torch, s, y, seg)[0] == iso.ISO_ERR_DATA
    yb = y.copy()
    yb[9] = np.inf
    assert gpu_curve(torch, s, yb)[0] == iso.ISO_ERR_DATA
