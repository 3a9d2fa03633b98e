"""The merge's device-side invariant checks (ISO_F_DEBUG_INVARIANTS: paper
section 4, Definition 4.3 and Theorem 4.4, checked after every segment-list
merge level and on every root list) and its path counters, and the
merge-schedule variants (ISO_F_WAVE_MERGES, ISO_F_THREE_CASE: paper section
7.4 and appendix A; ISO_F_TREE_MERGES) against the oracle.  The counters
show which merge paths a workload takes, so the tests below also prove that
the stress data reaches the wave walks, the nested bisection, the three-case
search, the chunk rebuild, and the second stage's group drops and its tree
fallback."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from lower_convex_hull_amd import inputs, iso
from tests import fitcheck

pytestmark = pytest.mark.gpu

NAMES = ("violations", "rebuilt", "to_wave", "bisect", "three_case", "levels", "root_vertices", "local_rounds")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as t

    assert t.cuda.is_available()
    iso.lib()
    return t


def fit_dbg(torch, y, w=None, flags=0):
    """Fit with the debug checks; returns (status, out, counters)."""
    y = np.atleast_2d(np.asarray(y, np.float32))
    yt = torch.from_numpy(y).cuda()
    wt = None if w is None else torch.from_numpy(np.asarray(w, np.float32).reshape(y.shape)).cuda()
    rows, n = yt.shape
    hint = iso.ISO_F_WEIGHTED_HINT if wt is not None else 0
    f = flags | iso.ISO_F_DEBUG_INVARIANTS
    nb0 = iso.iso_workspace_bytes(rows, n, hint | (f & ~iso.ISO_F_DEBUG_INVARIANTS))
    nb = iso.iso_workspace_bytes(rows, n, hint | f)
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(yt)
    st = iso.iso_fit_ex(yt.data_ptr(), None if wt is None else wt.data_ptr(), rows, n, out.data_ptr(), None,
                        ws.data_ptr(), nb, iso._stream_handle(None), f)
    torch.cuda.synchronize()
    cnt = ws[nb0:nb0 + 64].view(torch.int64).cpu().numpy()
    return st, out.cpu().numpy(), dict(zip(NAMES, cnt.tolist()))


def check(torch, y, w=None, flags=0, name="", interior=True):
    """interior: the root lists have vertices besides the row ends to check."""
    y = np.atleast_2d(np.asarray(y, np.float32))
    st, out, c = fit_dbg(torch, y, w, flags)
    say(f"[debug] {name} rows={y.shape[0]} n={y.shape[1]} flags={flags}: {c}")
    assert st == iso.ISO_OK, iso.iso_status_str(st)
    assert c["violations"] == 0 and (c["root_vertices"] > 0 or not interior)
    _, z64, _ = oracle.fit_rows_f32(y, w)
    ok, wa, wo, r = fitcheck.parity(y, w, out, z64)
    assert ok, (name, wa, wo, r)
    return out, c


def cliffs(n, at, seed):
    y, _ = inputs.dense(n, seed)
    y = y.copy()
    rng = np.random.default_rng(seed)
    for c in at:
        y[0, c] = -float(rng.uniform(50, 500))
    return y


def test_invariants_hold_on_every_workload_shape(torch):
    for name, (y, w) in (("c3", inputs.config("c3_row1e7_noisy")), ("c4", inputs.config("c4_row1e7_dense")),
                         ("c5x8", inputs.config("c5_calib256x2p20", rows=8))):
        _, c = check(torch, y, w, name=name)
        assert c["levels"] == 0 or c["levels"] > 0
    for fam in ("sawtooth", "random_walk", "piecewise", "cliff"):
        check(torch, inputs.family(fam, 1_000_003, 3)[None, :], None, name=fam)
    n = 60 * 64 * 4096 - 777
    y, _ = inputs.noisy(1, n, 35)
    check(torch, y, None, name="60 groups")
    d, _ = inputs.dense(n, 37)
    d = d.copy()
    d[0, n // 3] = -50.0
    _, c = check(torch, d, None, name="dense cliff, 60 groups")
    assert c["levels"] > 0  # the segment-list levels ran and were checked
    y, _ = inputs.noisy(1, 96 * 64 * 4096 + 12345, 34)
    _, c = check(torch, y, None, name="beyond the two-stage merge")
    assert c["levels"] > 0


def test_stress_data_reaches_the_long_walk_paths(torch):
    """The cliff rows of the parity suite (test_long_walks_and_bisection): walks
    reach their caps, go to waves, and beyond those caps to the nested bisection."""
    tot = dict.fromkeys(NAMES, 0)
    for n, at in ((300_000, (8191, 40_000, 123_457, 299_999)), (1_000_000, (524_287, 999_999))):
        _, c = check(torch, cliffs(n, at, 22), None, name=f"cliffs/{n}")
        for k in NAMES:
            tot[k] += c[k]
    assert tot["to_wave"] > 0 and tot["bisect"] > 0, tot


def test_rebuilt_chunks_are_counted(torch):
    """Rows in which exactly one chunk's hull has about 4096 vertices without
    being strictly increasing: the chunk kernel gives up on it and the first
    merge stage (or the fallback kernel, beyond the two-stage merge) rebuilds it."""
    from tests.test_gpu_parity import _one_fallback_chunk_rows

    for rows, n, chunk in ((1, 300_000, 17), (3, 150_000, 5), (1, 96 * 64 * 4096 + 5, 3000)):
        y = _one_fallback_chunk_rows(rows, n, chunk, 40 + rows)
        _, c = check(torch, y, None, name=f"one rebuilt chunk rows={rows} n={n}")
        assert c["rebuilt"] == 1, c


@pytest.mark.parametrize("variant", ["wave_merges", "three_case"])
def test_schedule_variants(torch, variant):
    flag = iso.ISO_F_WAVE_MERGES if variant == "wave_merges" else iso.ISO_F_THREE_CASE
    tot = dict.fromkeys(NAMES, 0)
    cases = [("cliffs/300k", cliffs(300_000, (8191, 40_000, 123_457, 299_999), 22), None),
             ("cliffs/1e6", cliffs(1_000_000, (524_287, 999_999), 22), None),
             ("cliffs-w/300k", cliffs(300_000, (4095, 150_000, 299_999), 23),
              inputs.weights("exp", 300_000, 23)[None, :]),
             ("sawtooth", inputs.family("sawtooth", 1_000_003, 5)[None, :], None),
             ("dense", inputs.dense(2_000_000, 6)[0], None)]
    n = 96 * 64 * 4096 + 12345
    d = inputs.consecutive_floats(n)[None, :].copy()
    for c in (4096 * 64 * 3 + 5, 10_000_019, n - 1):
        d[0, c] = 0.5
    cases.append(("beyond two-stage, cliffs", d, None))
    for name, y, w in cases:
        out_v, c = check(torch, y, w, flags=flag, name=f"{variant} {name}")
        for k in NAMES:
            tot[k] += c[k]
    if variant == "three_case":
        assert tot["three_case"] > 0, tot
        assert tot["to_wave"] == 0, tot  # thread-per-merge levels never hand over
    else:
        assert tot["to_wave"] == 0, tot


def _cascade_row(ng):
    """One row of ng groups of 64 chunks, each group strictly decreasing (its
    hull the two end points), with group sums that put the first group
    boundary low and the others on a convex parabola: every boundary but the
    ends lies above the chord from the row's start to the next boundary, so
    the bridges between neighbouring groups drop one group per round."""
    L = kGroupLen
    a, H = 1.0, 2.0 * ng * (ng + 1)
    k = np.arange(L, dtype=np.float64)
    y = np.empty(ng * L, np.float32)
    for g in range(ng):
        mean = H + a if g == 0 else a * (2 * g + 1)
        y[g * L:(g + 1) * L] = mean + 50.0 * (0.5 - k / L)
    return y[None, :]


kGroupLen = 64 * 4096


@pytest.mark.parametrize("case", ["decreasing", "cascade6", "cascade12", "noisy"])
def test_top_merge_drops_groups_and_falls_back_to_the_tree(torch, case):
    """The second stage's bridges between neighbouring groups: groups that keep
    no vertex are dropped round by round (a decreasing trend drops them all at
    once; the cascades one a round, the longer one beyond the round limit,
    where the merge tree takes over); every result matches the oracle and,
    bit for bit, the merge tree's (ISO_F_TREE_MERGES)."""
    if case == "decreasing":
        # a decreasing trend over the first groups, then an increasing one
        rng = np.random.default_rng(71)
        n = 9 * kGroupLen + 1234
        y = (3.0 * np.abs(np.linspace(-0.5, 1.0, n)) + 2.0 * rng.standard_normal(n)).astype(np.float32)[None, :]
    elif case == "noisy":
        y, _ = inputs.noisy(1, 39 * kGroupLen - 4321, 72)
    else:
        y = _cascade_row(int(case[len("cascade"):]))
    inner = not case.startswith("cascade")  # a cascade's hull is its two end points
    out, c = check(torch, y, None, name=f"top merge {case}", interior=inner)
    out_t, c_t = check(torch, y, None, flags=iso.ISO_F_TREE_MERGES, name=f"top merge {case}, tree", interior=inner)
    assert np.array_equal(out, out_t)
    assert c_t["local_rounds"] == 0
    want = {"decreasing": lambda r: r >= 1, "cascade6": lambda r: r == 4, "cascade12": lambda r: r == 8,
            "noisy": lambda r: r == 0}[case]
    assert want(c["local_rounds"]), c


def test_weighted_noisy_chunks_fit_the_compact_arrays(torch):
    """Weighted chunks keep fewer live points in LDS (room for 512 a wave, so
    that four workgroups fit a CU); the extra test of each candidate against
    the chord two points away keeps noisy weighted rows inside that room: no
    chunk is rebuilt.  A steep trend inside every chunk may overflow it; the
    rebuilt chunks then still give the oracle's fit."""
    n = 2_000_000 + 77
    y, _ = inputs.noisy(1, n, 81)
    for kind in ("uniform", "exp"):
        w = inputs.weights(kind, n, 82)[None, :]
        _, c = check(torch, y, w, name=f"noisy weighted {kind}")
        assert c["rebuilt"] == 0, c
    steep = (np.linspace(0, 5000, n) + np.random.default_rng(83).standard_normal(n)).astype(np.float32)[None, :]
    check(torch, steep, inputs.weights("uniform", n, 84)[None, :], name="steep weighted")
