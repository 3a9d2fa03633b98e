"""GPU parity of the f64 fit (iso_fit_ex_f64, iso_fit_f64: f64 y, w and out
through the same kernels) against the CPU oracle's f64 PAVA, element by element
(tests/fitcheck.parity_f64), with block ids checked as for f32."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from lower_convex_hull_amd import inputs, iso
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


def gpu_fit64(torch, y, w=None, flags=0):
    yt = torch.from_numpy(np.ascontiguousarray(y, np.float64)).cuda()
    wt = None if w is None else torch.from_numpy(np.ascontiguousarray(w, np.float64)).cuda()
    rows, n = yt.shape
    out = torch.empty_like(yt)
    bid = torch.empty((rows, n), dtype=torch.int32, device="cuda")
    ws = iso.workspace(rows, n, wt is not None, flags)
    st = iso.iso_fit_ex_f64(yt.data_ptr(), None if wt is None else wt.data_ptr(), rows, n, out.data_ptr(),
                            bid.data_ptr(), ws.data_ptr(), ws.numel(), iso._stream_handle(None), flags)
    torch.cuda.synchronize()
    return st, out.cpu().numpy(), bid.cpu().numpy()


def oracle64(y, w=None, sign=1.0):
    z = np.empty_like(y, dtype=np.float64)
    b = np.empty(y.shape, np.int32)
    for r in range(y.shape[0]):
        zr, br, _ = oracle.pava(sign * y[r], None if w is None else w[r])
        z[r] = sign * zr
        b[r] = br
    return z, b


def check64(torch, y, w=None, flags=0, name="", block_ids=True):
    y = np.atleast_2d(np.asarray(y, np.float64))
    if w is not None:
        w = np.asarray(w, np.float64).reshape(y.shape)
    say(f"[f64] {name} rows={y.shape[0]} n={y.shape[1]} weighted={w is not None} flags={flags}")
    st, out, bid = gpu_fit64(torch, y, w, flags)
    assert st == iso.ISO_OK, iso.iso_status_str(st)
    z, obid = oracle64(y, w, -1.0 if flags & iso.ISO_F_DECREASING else 1.0)
    ok, worst, row = fitcheck.parity_f64(y, w, out, z)
    say(f"[f64]   max |out - z| / (1 + |z|) = {worst * 1e-9:.3g}")
    assert ok, f"{name}: worst ratio {worst:.3g} in row {row}"
    if block_ids:
        for r in range(y.shape[0]):
            assert fitcheck.block_ids_consistent(obid[r], bid[r], z[r], y[r], delta_scale=1e-9), (name, r)
    return out, bid, z


def f64_noisy(rows, n, seed):
    rng = np.random.default_rng(seed)
    return np.linspace(0, 3, n) + rng.standard_normal((rows, n))


def test_f64_short_and_batched_rows(torch):
    check64(torch, f64_noisy(1, 4096, 1), name="c1-like")
    check64(torch, f64_noisy(1024, 1024, 2), name="c2-like")
    for n in (1, 2, 3, 63, 64, 65, 1023, 1025, 4095, 4096):
        y = f64_noisy(3, n, 10 + n)
        w = np.exp(8 * np.random.default_rng(n).random((3, n)))
        check64(torch, y, None, name=f"ragged {n}")
        check64(torch, y, w, name=f"ragged-w {n}")


def test_f64_long_rows(torch):
    check64(torch, f64_noisy(1, 10_000_000, 3), name="c3-like 1e7", block_ids=False)
    for n in (4097, 8193, 100_003, 1_000_000):
        y = f64_noisy(2, n, 20 + n)
        w = 0.1 + np.random.default_rng(n).random((2, n))
        check64(torch, y, None, name=f"long {n}")
        check64(torch, y, w, name=f"long-w {n}")


def test_f64_dense_row_is_identity(torch):
    y, _ = inputs.dense(10_000_000, 4)
    y = y.astype(np.float64)
    st, out, bid = gpu_fit64(torch, y)
    assert st == 0 and np.array_equal(out, y)
    assert np.array_equal(bid[0], np.arange(y.shape[1], dtype=np.int32))


def test_f64_calibration_rows(torch):
    y, w = inputs.config("c5_calib256x2p20", rows=16)
    check64(torch, y.astype(np.float64), w.astype(np.float64), name="c5x16")


@pytest.mark.parametrize("n", [1000, 4097, 12289, 100_003])
@pytest.mark.parametrize("fam", inputs.FAMILIES)
def test_f64_families(torch, fam, n):
    for k, wk in enumerate(inputs.WEIGHTINGS):
        rng = np.random.default_rng(2000 + k)
        y = inputs.family(fam, n, 1000 + k).astype(np.float64)
        if fam not in ("increasing", "decreasing", "constant", "sawtooth"):
            y = y + 1e-9 * rng.standard_normal(n) * (1.0 + np.abs(y))  # bits beyond f32
        w = inputs.weights(wk, n, 1000 + k)
        check64(torch, y[None, :], None if w is None else w.astype(np.float64), name=f"{fam}/{wk}/{n}")


def test_f64_cliffs_and_decreasing(torch):
    y, _ = inputs.dense(300_000, 22)
    y = y.astype(np.float64)
    for c in (8191, 40_000, 299_999):
        y[0, c] = -200.0
    check64(torch, y, None, name="cliffs")
    yd = f64_noisy(2, 30_000, 9)[:, ::-1].copy()
    check64(torch, yd, None, flags=iso.ISO_F_DECREASING, name="decreasing")


def test_f64_nonfinite_and_blocking_entry(torch):
    y = f64_noisy(3, 9000, 7)
    y[1, 5] = np.inf
    st, out, bid = gpu_fit64(torch, y)
    assert st == iso.ISO_WARN_NONFINITE and np.all(np.isnan(out[1])) and np.all(bid[1] == -1)
    y = f64_noisy(2, 20_000, 8)
    w = 0.5 + np.random.default_rng(8).random((2, 20_000))
    yt, wt = torch.from_numpy(y).cuda(), torch.from_numpy(w).cuda()
    out = torch.empty_like(yt)
    assert iso.iso_fit_f64(yt.data_ptr(), wt.data_ptr(), 2, 20_000, out.data_ptr()) == iso.ISO_OK
    z, _ = oracle64(y, w)
    assert fitcheck.parity_f64(y, w, out.cpu().numpy(), z)[0]
    iso.iso_release()


def test_f64_copy_control_matches(torch):
    y = f64_noisy(1, 500_000, 31)
    out_c, _, z = check64(torch, y, None, flags=iso.ISO_F_COPY_CONTROL, name="copy control f64")
    st, out_s, _ = gpu_fit64(torch, y)
    assert st == 0 and np.array_equal(out_c, out_s)
