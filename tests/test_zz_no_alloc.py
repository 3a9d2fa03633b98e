"""iso_fit_noalloc (the entry point that allocates nothing, its workspace a fixed
device array of the library) against iso_fit_ex with a caller workspace, through
the C ABI: two calls in a row, the second on a smaller input, each compared with
the other entry point's output bit for bit and with the oracle."""
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


def _both(torch, y, w, flags):
    yt = torch.from_numpy(y).cuda()
    wt = None if w is None else torch.from_numpy(w).cuda()
    rows, n = y.shape
    wp = None if wt is None else wt.data_ptr()
    out_a = torch.empty_like(yt)
    bid_a = torch.empty(yt.shape, dtype=torch.int32, device="cuda")
    st_a = iso.iso_fit_noalloc(yt.data_ptr(), wp, rows, n, out_a.data_ptr(), bid_a.data_ptr(),
                               iso._stream_handle(None), flags)
    out_b = torch.empty_like(yt)
    bid_b = torch.empty(yt.shape, dtype=torch.int32, device="cuda")
    ws = iso.workspace(rows, n, wt is not None, flags)
    st_b = iso.iso_fit_ex(yt.data_ptr(), wp, rows, n, out_b.data_ptr(), bid_b.data_ptr(),
                          ws.data_ptr(), ws.numel(), iso._stream_handle(None), flags)
    torch.cuda.synchronize()
    return (st_a, out_a.cpu().numpy(), bid_a.cpu().numpy()), (st_b, out_b.cpu().numpy(),
                                                              bid_b.cpu().numpy())


@pytest.mark.parametrize("kind", ["long", "long-weighted", "short"])
def test_noalloc_matches_fit_ex_twice(torch, kind):
    if kind == "long":
        shapes = [(2, 2_000_000), (1, 300_001)]
    elif kind == "long-weighted":
        shapes = [(4, 600_000), (3, 20_000)]
    else:
        shapes = [(512, 4096), (7, 1000)]
    for k, (rows, n) in enumerate(shapes):
        if kind == "long-weighted":
            y, w = inputs.calibration(rows, n, 90 + k)
        else:
            y, w = inputs.noisy(rows, n, 90 + k)
        say(f"[noalloc] {kind} call {k + 1}: rows={rows} n={n}")
        assert iso.iso_workspace_bytes(rows, n, iso.ISO_F_WEIGHTED_HINT if w is not None else 0) \
            <= iso.ISO_NOALLOC_BYTES
        (st_a, out_a, bid_a), (st_b, out_b, bid_b) = _both(torch, y, w, 0)
        assert st_a == iso.ISO_OK and st_b == iso.ISO_OK
        assert np.array_equal(out_a, out_b) and np.array_equal(bid_a, bid_b)
        _, z64, obid = oracle.fit_rows_f32(y, w)
        ok, wa, wo, r = fitcheck.parity(y, w, out_a, z64)
        assert ok, (kind, rows, n, wa, wo, r)
        for r in range(rows):
            assert fitcheck.block_ids_consistent(obid[r], bid_a[r], z64[r], y[r]), (kind, r)


def test_noalloc_rejects_shapes_beyond_its_array(torch):
    n = 20_000_000
    assert iso.iso_workspace_bytes(1, n, 0) > iso.ISO_NOALLOC_BYTES
    y = torch.zeros(16, dtype=torch.float32, device="cuda")  # never read: nothing is launched
    out = torch.zeros(16, dtype=torch.float32, device="cuda")
    st = iso.iso_fit_noalloc(y.data_ptr(), None, 1, n, out.data_ptr(), None,
                             iso._stream_handle(None), 0)
    assert st == iso.ISO_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert float(out.abs().sum()) == 0.0


def test_noalloc_reports_data_flags(torch):
    y, _ = inputs.noisy(3, 9000, 95)
    y[1, 123] = np.nan
    yt = torch.from_numpy(y).cuda()
    out = torch.empty_like(yt)
    st = iso.iso_fit_noalloc(yt.data_ptr(), None, 3, 9000, out.data_ptr(), None,
                             iso._stream_handle(None), 0)
    assert st == iso.ISO_WARN_NONFINITE
    o = out.cpu().numpy()
    assert np.all(np.isnan(o[1])) and not np.isnan(o[[0, 2]]).any()
