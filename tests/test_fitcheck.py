"""The parity rule itself: it accepts the oracle's own float32 output on every
accuracy family and weighting, and rejects outputs with a planted error."""
import numpy as np
import pytest

import oracle
from lower_convex_hull_amd import inputs
from tests import fitcheck


@pytest.mark.parametrize("fam", inputs.FAMILIES)
def test_rule_accepts_oracle_and_rejects_planted_error(fam):
    for k, wk in enumerate(inputs.WEIGHTINGS):
        y = inputs.family(fam, 3000, 50 + k)[None]
        w = inputs.weights(wk, 3000, 50 + k)
        w2 = None if w is None else w[None]
        o32, z64, bid = oracle.fit_rows_f32(y, w2)
        assert fitcheck.parity(y, w2, o32, z64)[0]
        assert fitcheck.block_ids_consistent(bid[0], bid[0], z64[0], y[0])
        bad = o32.copy()
        bad[0, 1500] += np.float32(2e-5 * (1 + np.abs(y).max()))
        assert not fitcheck.parity(y, w2, bad, z64)[0]
        # a merged block (a dropped block start between different means) is caught
        starts = np.flatnonzero(np.diff(bid[0])) + 1
        far = [s for s in starts if abs(z64[0, s] - z64[0, s - 1]) > 1e-3 * (1 + np.abs(y).max())]
        if far:
            gb = bid[0].copy()
            gb[far[0]:] -= 1
            assert not fitcheck.block_ids_consistent(bid[0], gb, z64[0], y[0])
