"""Pins of the O_cache oracle (no GPU).

Pinned by: T = D is the identity projection (so a corrected decision-scale
sparse output is exactly its full output); a 2x upsampling replicates each
decision token over a 2x2 block (closed form); the projection of every
schedule pair equals a brute-force search over the cell overlap of the unit
square (the target token's centre falls in its source cell); zero residual
leaves the output alone; the correction is linear."""
import numpy as np
import pytest

from oracle import ocache as OC
from varsparse_inputs import SCHEDULE_13


def test_identity_when_target_is_decision_scale():
    rng = np.random.default_rng(1)
    full, sparse = rng.normal(size=(2, 3, 64, 8)), rng.normal(size=(2, 3, 64, 8))
    out = OC.correct(sparse, full, sparse, 8, 8)
    np.testing.assert_allclose(out, full, rtol=0, atol=1e-12)   # s + (f - s) up to one rounding
    assert np.array_equal(OC.nearest_source(8, 8), np.arange(64))


def test_double_resolution_is_2x2_replication():
    rng = np.random.default_rng(2)
    r = rng.normal(size=(1, 1, 16, 5))
    up = OC.upsample(r, 4, 8).reshape(1, 1, 8, 8, 5)
    base = r.reshape(1, 1, 4, 4, 5)
    for dy in (0, 1):
        for dx in (0, 1):
            assert np.array_equal(up[:, :, dy::2, dx::2], base)


@pytest.mark.parametrize("i", range(len(SCHEDULE_13) - 1))
def test_projection_is_the_cell_containing_the_centre(i):
    # every later scale of the schedule against every earlier one
    for j in range(i, len(SCHEDULE_13)):
        hd, ht = SCHEDULE_13[i], SCHEDULE_13[j]
        src = OC.nearest_source(hd, ht).reshape(ht, ht)
        for y in range(ht):
            centre = (y + 0.5) / ht
            # brute force: the decision-scale row whose cell [a/hd, (a+1)/hd) holds ...
            cand = [a for a in range(hd) if a / hd <= y / ht < (a + 1) / hd]
            assert len(cand) == 1
            # ... the target row's top edge, which is floor(y hd / ht)
            assert src[y, 0] // hd == cand[0]
            assert abs(centre - (src[y, 0] // hd + 0.5) / hd) <= 0.5 / hd + 0.5 / ht


def test_zero_residual_and_linearity():
    rng = np.random.default_rng(3)
    o_t = rng.normal(size=(1, 2, 36, 4))
    f = rng.normal(size=(1, 2, 16, 4))
    s = rng.normal(size=(1, 2, 16, 4))
    assert np.array_equal(OC.correct(o_t, f, f, 4, 6), o_t)
    a = OC.correct(o_t, f, s, 4, 6) - o_t
    b = OC.correct(o_t, 2 * f, 2 * s, 4, 6) - o_t
    np.testing.assert_allclose(b, 2 * a, rtol=0, atol=1e-12)
