"""GPU parity: libiso.so (through its C ABI) against the CPU oracle, element by
element, on seeded inputs.

Rule (per row): max |out - z| <= 1e-5 (1 + max|y|) and the weighted objective
within 1e-9 relative of the oracle's (tests/fitcheck.parity).  Block ids: every
oracle block start between means that differ by more than 1e-6 (1 + max|y|) is
a GPU block start, and every extra GPU start separates means within that.
"""
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


def gpu_fit(torch, y, w=None, flags=0, block_ids=True):
    yt = torch.from_numpy(np.ascontiguousarray(y, np.float32)).cuda()
    wt = None if w is None else torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    rows, n = yt.shape
    out = torch.empty_like(yt)
    bid = torch.empty((rows, n), dtype=torch.int32, device="cuda") if block_ids else None
    ws = iso.workspace(rows, n, wt is not None, flags)
    st = iso.iso_fit_ex(yt.data_ptr(), None if wt is None else wt.data_ptr(), rows, n,
                        out.data_ptr(), None if bid is None else bid.data_ptr(), ws.data_ptr(),
                        ws.numel(), iso._stream_handle(None), flags)
    torch.cuda.synchronize()
    return st, out.cpu().numpy(), (None if bid is None else bid.cpu().numpy())


def check(torch, y, w=None, flags=0, name="", block_ids=True):
    y = np.atleast_2d(np.asarray(y, np.float32))
    if w is not None:
        w = np.asarray(w, np.float32).reshape(y.shape)
    say(f"[parity] {name} rows={y.shape[0]} n={y.shape[1]} weighted={w is not None} flags={flags}")
    st, out, bid = gpu_fit(torch, y, w, flags, block_ids)
    assert st == iso.ISO_OK, iso.iso_status_str(st)
    ysign = -y if flags & iso.ISO_F_DECREASING else y
    _, z64, obid = oracle.fit_rows_f32(ysign, w)
    if flags & iso.ISO_F_DECREASING:
        z64 = -z64
    ok, wa, wo, row = fitcheck.parity(y, w, out, z64)
    assert ok, f"{name}: abs ratio {wa:.3g}, objective ratio {wo:.3g}, row {row}"
    if block_ids:
        for r in range(y.shape[0]):
            assert fitcheck.block_ids_consistent(obid[r], bid[r], z64[r], y[r]), f"{name}: block ids row {r}"
    return out, bid, z64


# --------------------------------------------------------------------------- pages' examples

def test_worked_examples(torch):
    for c in fitcheck.read_cases("worked_examples.txt"):
        y = np.array([[float(v) for v in c["y"]]], np.float32)
        want = np.array([float(v) for v in c["z"]])
        st, out, bid = gpu_fit(torch, y)
        assert st == 0
        assert np.allclose(out[0], want, rtol=0, atol=1e-6), c["case"]


def test_tiny_rows_against_brute_force(torch):
    rng = np.random.default_rng(31)
    for n in range(1, 13):
        for wk in ("none", "uniform", "exp"):
            rows = 64
            y = rng.integers(-3, 4, (rows, n)).astype(np.float32)
            y[rows // 2:] = rng.normal(0, 1, (rows - rows // 2, n)).astype(np.float32)
            w = None if wk == "none" else (
                (0.1 + rng.random((rows, n))) if wk == "uniform" else np.exp(8 * rng.random((rows, n)))
            ).astype(np.float32)
            st, out, _ = gpu_fit(torch, y, w)
            assert st == 0
            for r in range(rows):
                zb, _ = oracle.brute_force(y[r].astype(np.float64),
                                           None if w is None else w[r].astype(np.float64))
                tol = 1e-5 * (1 + np.abs(y[r]).max())
                assert np.abs(out[r] - zb).max() <= tol, (n, wk, r)


# --------------------------------------------------------------------------- the five workloads

def test_c1_row4096(torch):
    y, w = inputs.config("c1_row4096_noisy")
    check(torch, y, w, name="c1")


def test_c2_batch1024x1024(torch):
    y, w = inputs.config("c2_batch1024x1024_noisy")
    check(torch, y, w, name="c2")


def test_c3_row1e7_noisy(torch):
    y, w = inputs.config("c3_row1e7_noisy")
    check(torch, y, w, name="c3", block_ids=True)


def test_c4_row1e7_dense(torch):
    y, w = inputs.config("c4_row1e7_dense")
    out, bid, _ = check(torch, y, w, name="c4")
    # closed form: a strictly increasing row is its own fit, every element a block
    assert np.array_equal(out[0], y[0])
    assert np.array_equal(bid[0], np.arange(y.shape[1], dtype=np.int32))


def test_c5_calibration_rows(torch):
    # 16 of the 256 rows at full length (2^20), same recipe; every row of the
    # full batch is compared in test_c5_full_batch_every_row.
    y, w = inputs.config("c5_calib256x2p20", rows=16)
    check(torch, y, w, name="c5x16")


def test_c5_full_batch_every_row(torch):
    """The whole 256 x 2^20 calibration batch in one call, every row compared
    with the oracle element by element (values and block ids)."""
    y, w = inputs.config("c5_calib256x2p20")
    say("[parity] c5 full batch 256 x 2^20, every row against the oracle")
    st, out, bid = gpu_fit(torch, y, w, block_ids=True)
    assert st == 0
    for r0 in range(0, y.shape[0], 32):
        sl = slice(r0, r0 + 32)
        _, z64, obid = oracle.fit_rows_f32(y[sl], w[sl])
        ok, wa, wo, r = fitcheck.parity(y[sl], w[sl], out[sl], z64)
        assert ok, (wa, wo, r0 + r)
        for r in range(z64.shape[0]):
            assert fitcheck.block_ids_consistent(obid[r], bid[r0 + r], z64[r], y[r0 + r]), \
                f"c5 block ids row {r0 + r}"


# --------------------------------------------------------------------------- families, sizes, edges

@pytest.mark.parametrize("n", [1000, 4096, 4097, 5000, 12289, 100_003])
@pytest.mark.parametrize("fam", inputs.FAMILIES)
def test_families(torch, fam, n):
    for k, wk in enumerate(inputs.WEIGHTINGS):
        y = inputs.family(fam, n, 1000 + k)
        w = inputs.weights(wk, n, 1000 + k)
        check(torch, y[None, :], w, name=f"{fam}/{wk}/{n}")


@pytest.mark.parametrize("n", [1, 2, 3, 63, 64, 65, 1023, 1024, 1025, 4095, 4096, 4097, 8192, 8193])
def test_ragged_sizes(torch, n):
    rows = 3
    y, _ = inputs.noisy(rows, n, 40 + n)
    w = inputs.weights("uniform", rows * n, 40 + n).reshape(rows, n)
    check(torch, y, None, name=f"ragged/{n}")
    check(torch, y, w, name=f"ragged-w/{n}")


def test_short_row_shapes_by_batch_size(torch):
    """Short rows take wider workgroups when the batch is too small to fill the
    GPU and the narrower ones otherwise: both shapes on each side of the
    switch (rows*4 or rows*8 waves against 8192), unit and integer weights."""
    cases = [(2048, 700, "noisy"), (2049, 700, "noisy"), (1024, 2000, "noisy"), (1025, 2000, "noisy"),
             (2049, 1024, "calibration"), (1025, 4096, "calibration")]
    for rows, n, kind in cases:
        if kind == "noisy":
            y, w = inputs.noisy(rows, n, rows + n)
        else:
            y, w = inputs.calibration(rows, n, rows + n)
        check(torch, y, w, name=f"short shapes {kind} {rows}x{n}", block_ids=rows * n <= 3_000_000)


def test_batch_of_long_rows(torch):
    y, w = inputs.calibration(6, 20_000, 77)
    check(torch, y, w, name="long-batch")
    y2, _ = inputs.noisy(5, 50_000, 78)
    check(torch, y2, None, name="long-batch-noisy")


def test_long_walks_and_bisection(torch):
    """Dense (strictly increasing) rows with cliffs: a merge then removes thousands
    of vertices, so walks exceed their caps and the wave walk and the nested
    bisection run (at low and at high levels of the merge tree)."""
    rng = np.random.default_rng(21)
    for n, cliffs in ((300_000, (8191, 40_000, 123_457, 299_999)), (70_000, (4095, 69_999)),
                      (1_000_000, (524_287, 999_999))):
        y, _ = inputs.dense(n, 22)
        y = y.copy()
        for c in cliffs:
            y[0, c] = -float(rng.uniform(50, 500))
        check(torch, y, None, name=f"cliffs/{n}")
        w = inputs.weights("exp", n, 23)[None, :]
        check(torch, y, w, name=f"cliffs-w/{n}")


def test_mixed_dense_and_noisy_stretches(torch):
    """One row whose groups of chunk hulls are partly short (noise) and partly
    long (strictly increasing stretches), so the short-hull and the
    segment-list merge paths meet in one row and in its top stage."""
    rng = np.random.default_rng(31)
    parts = []
    for k in range(8):
        seg = 300_000
        if k % 2 == 0:
            d, _ = inputs.dense(seg, 32 + k)
            parts.append(d[0] * 2.0 + k * 0.25)
        else:
            parts.append((np.linspace(0, 3, seg) + rng.standard_normal(seg)).astype(np.float32) * 0.5 + k * 0.25)
    y = np.concatenate(parts).astype(np.float32)[None, :]
    check(torch, y, None, name="mixed/2.4e6", block_ids=False)
    w = inputs.weights("exp", y.shape[1], 33)[None, :]
    check(torch, y, w, name="mixed-w/2.4e6", block_ids=False)


def test_rows_with_many_groups(torch):
    """Rows of 60 groups of 64 chunks: the second merge stage holds only part
    of its group windows in registers and reads the rest where it uses them
    (unit weights and weighted, compact-array and segment-list paths)."""
    n = 60 * 64 * 4096 - 777
    y, _ = inputs.noisy(1, n, 35)
    check(torch, y, None, name="noisy/60 groups", block_ids=False)
    w = inputs.weights("exp", n, 36)[None, :]
    check(torch, y, w, name="noisy-w/60 groups", block_ids=False)
    d, _ = inputs.dense(n, 37)
    d = d.copy()
    d[0, n // 3] = -50.0  # one cliff: group hulls too long for their windows
    check(torch, d, None, name="dense-cliff/60 groups", block_ids=False)


def test_row_beyond_two_stage_merge(torch):
    """A row with more groups than the two-stage merge keeps in LDS: one
    workgroup merges every level with its lists in the workspace."""
    n = 96 * 64 * 4096 + 12345
    y, _ = inputs.noisy(1, n, 34)
    check(torch, y, None, name="noisy/2.5e7", block_ids=False)


def test_batch_of_rows_beyond_two_stage_merge(torch):
    """Three rows beyond the two-stage merge in one call (weighted, block ids
    checked): the row merge's tree levels spread over workgroups of every row
    at once (grid rows x workgroups), and the records formed by the expansion
    from each row's root list."""
    n = 80 * 64 * 4096 + 7
    y, _ = inputs.noisy(3, n, 35)
    w = inputs.weights("uniform", 3 * n, 35).reshape(3, n)
    y[1] = np.sort(y[1])  # a strictly increasing stretch ...
    y[1, n // 3] = -5.0   # ... with a cliff: bridges reach across groups
    check(torch, y, w, name="3 rows beyond two stages", block_ids=True)


def test_rows_of_1e8(torch):
    """Rows of 10^8 elements (the paper's longest rows, Tables 1-3): beyond the
    two-stage merge, the groups' lists are merged through the remaining levels
    by one workgroup.  Noisy (against the oracle), consecutive floats (closed
    form: the fit is the row, every element its own block), and consecutive
    floats with cliffs so that bridges reach across groups at high levels."""
    n = 100_000_000
    y, _ = inputs.noisy(1, n, 81)
    check(torch, y, None, name="noisy/1e8", block_ids=False)
    del y
    y = inputs.consecutive_floats(n)[None, :]
    say("[parity] consecutive floats n=1e8")
    st, out, bid = gpu_fit(torch, y)
    assert st == 0 and np.array_equal(out, y)
    assert np.array_equal(bid[0], np.arange(n, dtype=np.int32))
    del out, bid
    y = y.copy()
    for c in (4096 * 64 * 3 + 5, 31_000_017, 77_777_777, n - 1):
        y[0, c] = 0.5
    check(torch, y, None, name="consecutive+cliffs/1e8", block_ids=False)


def test_sawtooth_and_walk_families_at_1e6(torch):
    for fam in ("sawtooth", "random_walk", "cliff", "piecewise"):
        y = inputs.family(fam, 1_000_000, 24)[None, :]
        check(torch, y, None, name=f"{fam}/1e6", block_ids=False)


@pytest.mark.parametrize("case", ["c3", "c4", "c5x8", "families", "cliffs"])
def test_copy_control_matches(torch, case):
    """The vertex-copying merge control (ISO_F_COPY_CONTROL) gives the oracle's fit,
    and the same output as the segment-list merge."""
    if case == "c3":
        ys = [inputs.config("c3_row1e7_noisy")]
    elif case == "c4":
        ys = [inputs.config("c4_row1e7_dense")]
    elif case == "c5x8":
        ys = [inputs.config("c5_calib256x2p20", rows=8)]
    elif case == "families":
        ys = [(inputs.family(f, 123_457, 5)[None, :], inputs.weights(wk, 123_457, 5))
              for f in ("gaussian", "random_walk", "sawtooth", "cliff") for wk in ("none", "exp")]
    else:
        y, _ = inputs.dense(300_000, 22)
        y = y.copy()
        for c in (8191, 40_000, 299_999):
            y[0, c] = -100.0
        ys = [(y, None)]
    for y, w in ys:
        if w is not None:
            w = np.asarray(w).reshape(y.shape)
        out_c, bid_c, _ = check(torch, y, w, flags=iso.ISO_F_COPY_CONTROL, name=f"copy/{case}")
        st, out_s, bid_s = gpu_fit(torch, y, w)
        assert st == 0
        assert np.array_equal(out_c, out_s), f"copy/{case}: outputs differ from the segment-list merge"


def test_decreasing_flag(torch):
    y, _ = inputs.noisy(4, 3000, 9)
    check(torch, y[:, ::-1].copy(), None, flags=iso.ISO_F_DECREASING, name="dec-short")
    y, _ = inputs.noisy(2, 30000, 10)
    check(torch, y[:, ::-1].copy(), None, flags=iso.ISO_F_DECREASING, name="dec-long")


def test_consecutive_floats_are_fixed_points(torch):
    for n in (3000, 200_000):
        y = inputs.consecutive_floats(n)[None, :]
        say(f"[parity] consecutive floats n={n}")
        st, out, bid = gpu_fit(torch, y)
        assert st == 0
        assert np.array_equal(out, y)
        assert np.array_equal(bid[0], np.arange(n, dtype=np.int32))


def test_cancellation_family_stress(torch):
    # a stress test, not a gate: B up to 1e6 (paper section 7.6 goes further)
    for big in (1e3, 1e6):
        y = inputs.cancellation(20_000, big, 5)[None, :]
        check(torch, y, None, name=f"cancellation/{big:g}", block_ids=False)


def test_constant_and_decreasing_rows(torch):
    n = 9000
    y = np.full((2, n), 0.25, np.float32)
    st, out, bid = gpu_fit(torch, y)
    assert st == 0 and np.all(out == 0.25)
    y = -np.sort(np.random.default_rng(3).random((2, n)), axis=1).astype(np.float32)
    check(torch, y, None, name="strictly-decreasing")


def test_nonfinite_rows_and_bad_weights(torch):
    y, _ = inputs.noisy(4, 5000, 12)
    y[1, 17] = np.nan
    y[3, 4999] = np.inf
    st, out, bid = gpu_fit(torch, y)
    assert st == iso.ISO_WARN_NONFINITE
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(out[3]))
    assert np.all(bid[1] == -1) and np.all(bid[3] == -1)
    _, z64, _ = oracle.fit_rows_f32(y[[0, 2]])
    assert fitcheck.parity(y[[0, 2]], None, out[[0, 2]], z64)[0]
    ys, _ = inputs.noisy(3, 500, 13)
    ys[2, 0] = -np.inf
    st, out, bid = gpu_fit(torch, ys)
    assert st == iso.ISO_WARN_NONFINITE and np.all(np.isnan(out[2])) and not np.isnan(out[:2]).any()
    for n in (500, 5000):
        y, _ = inputs.noisy(2, n, 14)
        w = np.ones_like(y)
        w[1, 3] = 0.0
        st, _, _ = gpu_fit(torch, y, w)
        assert st == iso.ISO_ERR_WEIGHT
        w[1, 3] = -1.0
        st, _, _ = gpu_fit(torch, y, w)
        assert st == iso.ISO_ERR_WEIGHT
        w[1, 3] = np.nan
        st, _, _ = gpu_fit(torch, y, w)
        assert st == iso.ISO_ERR_WEIGHT


def test_nonfinite_and_bad_weight_in_a_later_group(torch):
    """Rows long enough for two merge stages: a data flag raised in a chunk of a
    later group reaches the row's status through the group records."""
    n = 300_000  # 74 chunks, two groups
    y, _ = inputs.noisy(2, n, 15)
    y[1, 280_000] = np.nan
    st, out, bid = gpu_fit(torch, y)
    assert st == iso.ISO_WARN_NONFINITE
    assert np.all(np.isnan(out[1])) and np.all(bid[1] == -1) and not np.isnan(out[0]).any()
    _, z64, _ = oracle.fit_rows_f32(y[[0]])
    assert fitcheck.parity(y[[0]], None, out[[0]], z64)[0]
    y2, _ = inputs.noisy(2, n, 16)
    w = np.ones_like(y2)
    w[1, 290_000] = 0.0
    st, _, _ = gpu_fit(torch, y2, w)
    assert st == iso.ISO_ERR_WEIGHT


def _one_fallback_chunk_rows(rows, n, chunk, seed):
    """Noisy rows in which one chunk of row 0 is strictly increasing but for one
    repeated value: that chunk's hull keeps about 4096 vertices, so the chunk
    kernel gives up on it and it is rebuilt (by the first merge stage, or by
    the fallback kernel for rows beyond the two-stage merge)."""
    y, _ = inputs.noisy(rows, n, seed)
    c = iso.iso_chunk_size(n)
    a, b = chunk * c, min(n, (chunk + 1) * c)
    d, _ = inputs.dense(b - a, seed + 1)
    seg = 1.0 + d[0]
    seg[(b - a) // 2] = seg[(b - a) // 2 - 1]  # one tie: not strictly increasing
    y[0, a:b] = seg
    return y


def test_workspace_contents_need_no_initialisation(torch):
    """A workspace full of 0xFF bytes, then reused across shapes with its
    previous call's contents left in it: rows where exactly one chunk is
    rebuilt still match the oracle (the rebuild depends only on what the chunk
    kernel wrote in the same call)."""
    cases = [(1, 300_000, 17), (3, 150_000, 5), (2, 2 * 4096 + 77, 1), (1, 96 * 64 * 4096 + 5, 3000)]
    nbytes = max(iso.iso_workspace_bytes(r, n, 0) for r, n, _ in cases)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    for rows, n, chunk in cases + cases[:2]:
        y = _one_fallback_chunk_rows(rows, n, chunk, 40 + rows)
        say(f"[parity] stale workspace rows={rows} n={n} fallback chunk {chunk}")
        yt = torch.from_numpy(y).cuda()
        out = torch.empty_like(yt)
        bid = torch.empty(yt.shape, dtype=torch.int32, device="cuda")
        st = iso.iso_fit_ex(yt.data_ptr(), None, rows, n, out.data_ptr(), bid.data_ptr(),
                            ws.data_ptr(), nbytes, iso._stream_handle(None), 0)
        torch.cuda.synchronize()
        assert st == iso.ISO_OK, iso.iso_status_str(st)
        o = out.cpu().numpy()
        _, z64, obid = oracle.fit_rows_f32(y)
        ok, wa, wo, r = fitcheck.parity(y, None, o, z64)
        assert ok, (rows, n, wa, wo, r)
        b = bid.cpu().numpy()
        for r in range(rows):
            assert fitcheck.block_ids_consistent(obid[r], b[r], z64[r], y[r]), (rows, n, r)
        del yt, out, bid
    # the blocking entry point's cached workspace, reused across two shapes
    for rows, n, chunk in ((1, 300_000, 40), (4, 100_000, 3)):
        y = _one_fallback_chunk_rows(rows, n, chunk, 60 + rows)
        yt = torch.from_numpy(y).cuda()
        out = torch.empty_like(yt)
        assert iso.iso_fit(yt.data_ptr(), None, rows, n, out.data_ptr()) == iso.ISO_OK
        _, z64, _ = oracle.fit_rows_f32(y)
        assert fitcheck.parity(y, None, out.cpu().numpy(), z64)[0], (rows, n)
    iso.iso_release()


def test_deterministic(torch):
    y, _ = inputs.noisy(1, 300_000, 15)
    _, a, ba = gpu_fit(torch, y)
    _, b, bb = gpu_fit(torch, y)
    assert np.array_equal(a, b) and np.array_equal(ba, bb)


def test_iso_fit_blocking_entry(torch):
    y, w = inputs.calibration(2, 9000, 16)
    yt = torch.from_numpy(y).cuda()
    wt = torch.from_numpy(w).cuda()
    out = torch.empty_like(yt)
    torch.cuda.synchronize()
    st = iso.iso_fit(yt.data_ptr(), wt.data_ptr(), 2, 9000, out.data_ptr())
    assert st == 0
    _, z64, _ = oracle.fit_rows_f32(y, w)
    assert fitcheck.parity(y, w, out.cpu().numpy(), z64)[0]
    iso.iso_release()


def test_iso_fit_reports_allocation_failure(torch):
    """A shape whose workspace (about 1e13 bytes) is more than the device holds:
    iso_fit's allocation fails, it returns ISO_ERR_NOMEM with nothing launched
    (the tiny buffers passed are never read), and the library keeps working."""
    n = 1 << 40
    assert iso.iso_workspace_bytes(1, n, 0) > 10 ** 12
    y = torch.zeros(16, dtype=torch.float32, device="cuda")
    out = torch.full((16,), 7.0, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    assert iso.iso_fit(y.data_ptr(), None, 1, n, out.data_ptr()) == iso.ISO_ERR_NOMEM
    torch.cuda.synchronize()
    assert float(out.sum()) == 16 * 7.0
    y2, _ = inputs.noisy(2, 20_000, 19)
    yt = torch.from_numpy(y2).cuda()
    o2 = torch.empty_like(yt)
    assert iso.iso_fit(yt.data_ptr(), None, 2, 20_000, o2.data_ptr()) == iso.ISO_OK
    _, z64, _ = oracle.fit_rows_f32(y2)
    assert fitcheck.parity(y2, None, o2.cpu().numpy(), z64)[0]
    iso.iso_release()


def test_fit_wrapper_on_torch_stream(torch):
    y, _ = inputs.noisy(8, 7000, 17)
    yt = torch.from_numpy(y).cuda()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, bid = iso.fit(yt, block_ids=True, stream=s)
    s.synchronize()
    _, z64, _ = oracle.fit_rows_f32(y)
    assert fitcheck.parity(y, None, out.cpu().numpy(), z64)[0]


def test_constant_runs_are_single_blocks(torch):
    """Increasing runs of one f32 value each (values in [0.5, 1), not dyadic
    fractions with few bits): the points of a run are exactly collinear in the
    cumulative sum diagram (every S is an exact f64 sum here), so each run is
    one block, as the oracle pools equal means.  The hull predicates must
    round both products of a cross product on their own: a fused
    multiply-add leaves the rounding error of one product instead of zero,
    which shows on runs long enough for the products to need more than 53
    bits."""
    rng = np.random.default_rng(81)
    for rows, n, most in ((4, 3000, 8), (1, 300_000, 750), (1, 3_000_000, 7500), (1, 3_000_000, 1_000_000)):
        y = np.empty((rows, n), np.float32)
        for r in range(rows):
            lens = rng.integers(1, most, size=n)
            starts = np.concatenate([[0], np.cumsum(lens)])
            nr = int(np.searchsorted(starts, n)) + 1
            vals = (0.5 + 0.49 * np.arange(nr) / nr).astype(np.float32)
            run = np.searchsorted(starts, np.arange(n), side="right") - 1
            y[r] = vals[run]
        st, out, bid = gpu_fit(torch, y)
        assert st == iso.ISO_OK, iso.iso_status_str(st)
        _, z64, obid = oracle.fit_rows_f32(y)
        assert fitcheck.parity(y, None, out, z64)[0], n
        for r in range(rows):
            assert np.array_equal(bid[r], obid[r]), (n, r, int(bid[r].max()), int(obid[r].max()))


def test_random_long_rows_against_oracle(torch):
    """Seeded random long rows of 2 to 30 groups of 64 chunks: trends up and
    down (so that the second stage's bridges between neighbouring groups drop
    groups in some rows), V shapes, steps and sawtooths, with and without
    weights, each against the oracle."""
    G = 64 * 4096
    rng = np.random.default_rng(97)
    for case in range(16):
        n = int(rng.integers(2 * G, 30 * G)) + int(rng.integers(0, 4096))
        kind = ("trend", "vee", "steps", "saw")[case % 4]
        t = np.linspace(0.0, 1.0, n)
        sd = float(rng.uniform(0.1, 3.0))
        if kind == "trend":
            y = float(rng.uniform(-3, 3)) * t + sd * rng.standard_normal(n)
        elif kind == "vee":
            y = 3.0 * np.abs(t - float(rng.uniform(0.2, 0.8))) + sd * rng.standard_normal(n)
        elif kind == "steps":
            k = int(rng.integers(2, 40))
            y = np.repeat(rng.normal(0, 1, k), -(-n // k))[:n] + 0.1 * sd * rng.standard_normal(n)
        else:
            period = int(rng.integers(1000, n // 3))
            y = (np.arange(n) % period) / period + 0.1 * sd * rng.standard_normal(n)
        y = y.astype(np.float32)[None, :]
        w = inputs.weights(("none", "uniform", "exp")[case % 3], n, case)
        check(torch, y, None if w is None else w[None, :], name=f"random {case} {kind} n={n}",
              block_ids=True)
