"""GPU parity: CSLA block mask and lists, bit-exact against the oracle."""
import numpy as np
import pytest
import torch

from tests._common import oracle_mask
from varsparse_inputs import SCHEDULE_13, SCHEDULE_16, TINY_SIDES

pytestmark = pytest.mark.gpu

CASES = [
    # (sides, q_scale, tile, n_sink, radius per scale, budget)
    (TINY_SIDES, 4, 4, 3, (4,) * 5, -1),
    (TINY_SIDES, 4, 4, 0, (0,) * 5, -1),
    (SCHEDULE_13, 12, 8, 5, (2,) * 13, -1),                # 2B-shaped last scale
    (SCHEDULE_13, 11, 8, 5, (2,) * 12, -1),
    (SCHEDULE_13, 10, 8, 5, (3,) * 11, -1),
    (SCHEDULE_13, 12, 8, 2, (-1, -1, 0, 1, 2, -1, 3, 0, 1, 4, 2, -1, 1), -1),
    (SCHEDULE_13, 12, 8, 0, (-1,) * 12 + (0,), -1),
    (SCHEDULE_13, 12, 8, 5, (64,) * 13, -1),               # dense
    (SCHEDULE_16, 15, 8, 5, (2,) * 16, -1),                # high-resolution stress
    ((1, 3, 5, 7, 10), 4, 5, 1, (1,) * 5, -1),              # tile 5: partial key tiles everywhere
] + [(SCHEDULE_13, 12, 8, 5, None, k) for k in (43, 26, 17, 9)] \
  + [(SCHEDULE_13, 11, 8, 5, None, k) for k in (27, 16, 11, 5, 1, 200)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"q{c[1]}_t{c[2]}_s{c[3]}_b{c[5]}")
def test_mask_bit_exact(case):
    import block_sparse_cross_csla_amd as vs
    sides, q, t, n_sink, radius, budget = case
    if sides[q] % t:
        pytest.skip("query side not a multiple of the tile")
    print(f"mask case q={q} t={t} n_sink={n_sink} budget={budget}", flush=True)
    cnt, idx, mask = vs.build_mask(sides, t, q, n_sink, radius=radius, budget=budget, want_mask=True)
    torch.cuda.synchronize()
    want = oracle_mask(tuple(sides), q, t, n_sink, radius if radius is None else tuple(radius), budget)
    got = mask.cpu().numpy().astype(bool)
    assert (got == want).all(), f"{(got != want).sum()} mask entries differ"
    cnt = cnt.cpu().numpy()
    idx = idx.cpu().numpy()
    assert (cnt == want.sum(axis=1)).all()
    for r in range(want.shape[0]):
        assert (idx[r, : cnt[r]] == np.flatnonzero(want[r])).all()
        assert (idx[r, cnt[r]:] == -1).all()


def test_mask_is_deterministic_and_list_only():
    import block_sparse_cross_csla_amd as vs
    a = vs.build_mask(SCHEDULE_13, 8, 12, 5, radius=(2,) * 13)
    b = vs.build_mask(SCHEDULE_13, 8, 12, 5, radius=(2,) * 13, want_mask=True)
    torch.cuda.synchronize()
    assert a[2] is None
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
