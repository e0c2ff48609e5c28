"""bench.py's host-side accounting, on the CPU: the FLOP count that the
line's `value` and `roofline.achieved` divide by, the key tiles' token counts,
the reported block sparsities (the derived pins of the 2B workload: 82.50%
count, 84.31% token-weighted), and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
from oracle import csla, geometry as G
from varsparse_inputs import TINY_SIDES, workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_tile_sizes_match_the_oracle_geometry():
    for sides, q, t in ((W.LAST_SCALE_2B.sides, 12, 8), (TINY_SIDES, 4, 4), ((1, 3, 5, 7, 10), 4, 5)):
        tiles = G.key_tiles(sides, q, t)
        assert list(bench.tile_sizes(sides, q, t)) == [tile.tokens().size for tile in tiles]


def _brute_force_flops(mask, sides, q, t, d):
    """4 d FLOP (QK^T and PV) per kept (query token, key token) pair."""
    qts, kts = G.query_tiles(sides, q, t), G.key_tiles(sides, q, t)
    pairs = sum(qts[i].tokens().size * kts[j].tokens().size for i, j in zip(*np.nonzero(mask)))
    return 4.0 * d * pairs


def test_kept_flops_of_the_2b_workload():
    w = W.LAST_SCALE_2B
    mask = csla.block_mask(w.sides, w.q_scale, w.tile, w.n_sink, list(w.radii))
    cnt, idx = csla.lists_from_mask(mask)
    sizes = bench.tile_sizes(w.sides, w.q_scale, w.tile)
    heads = w.B * w.H
    flops = bench.kept_flops(cnt, idx, sizes, w.tile * w.tile, w.d, heads)
    assert flops == _brute_force_flops(mask, w.sides, w.q_scale, w.tile, w.d) * heads
    assert flops == 1.10746402816e11
    nqb, nkb, nq, nk = G.counts(w.sides, w.q_scale, w.tile)
    assert round(1 - cnt.sum() / (nqb * nkb), 4) == 0.8250
    assert round(1 - flops / (4.0 * w.d * nq * nk * heads), 4) == 0.8431


def test_kept_flops_per_head_lists():
    """Per-(b, h) lists are summed head by head; shared lists count once per head."""
    sides, q, t, d = TINY_SIDES, 4, 4, 64
    rng = np.random.default_rng(5)
    nqb, nkb, _, _ = G.counts(sides, q, t)
    masks = rng.random((2, 3, nqb, nkb)) < 0.4
    sizes = bench.tile_sizes(sides, q, t)
    cnt = np.zeros((2, 3, nqb), np.int32)
    idx = np.full((2, 3, nqb, nkb), -1, np.int32)
    want = 0.0
    for b in range(2):
        for h in range(3):
            cnt[b, h], idx[b, h] = csla.lists_from_mask(masks[b, h])
            want += _brute_force_flops(masks[b, h], sides, q, t, d)
    assert bench.kept_flops(cnt, idx, sizes, t * t, d, 6) == want
    shared_cnt, shared_idx = csla.lists_from_mask(masks[0, 0])
    assert bench.kept_flops(shared_cnt, shared_idx, sizes, t * t, d, 6) == \
        6 * _brute_force_flops(masks[0, 0], sides, q, t, d)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]
