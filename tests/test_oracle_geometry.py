"""Pins for oracle.geometry: closed forms and partition invariants."""
import numpy as np

from oracle import geometry as G
from varsparse_inputs import SCHEDULE_13, SCHEDULE_16, TINY_SIDES


def test_cache_lengths_closed_form():
    # sum of side^2 over the schedule, written out
    assert G.scale_offsets(TINY_SIDES)[-1] == 1 + 4 + 16 + 64 + 256 == 341
    assert G.scale_offsets(SCHEDULE_13)[-1] == 10521
    assert G.scale_offsets(SCHEDULE_13)[12] == 6425       # cache of the side-48 query scale
    assert G.scale_offsets(SCHEDULE_13)[10] == 2521       # cache of the side-32 decision scale
    assert G.scale_offsets(SCHEDULE_16)[-1] == 42521


def test_tile_counts():
    # ceil(side / 8)^2 summed: 1,1,1,1,1,4,4,9,9,16,25,36,64
    assert G.counts(SCHEDULE_13, 12, 8) == (64, 172, 4096, 10521)
    assert G.counts(SCHEDULE_13, 11, 8) == (36, 108, 2304, 6425)
    assert G.counts(SCHEDULE_13, 9, 8) == (16, 47, 1024, 2521)
    assert G.counts(TINY_SIDES, 4, 4) == (16, 23, 256, 341)
    assert G.counts(SCHEDULE_16, 15, 8) == (256, 672, 16384, 42521)


def test_tiles_partition_tokens():
    for sides, q, t in [(TINY_SIDES, 4, 4), (SCHEDULE_13, 12, 8), ((1, 3, 5, 7), 3, 2)]:
        nk = G.scale_offsets(sides)[q + 1]
        seen = np.zeros(nk, int)
        for tl in G.key_tiles(sides, q, t):
            seen[tl.tokens()] += 1
            assert 1 <= tl.rows <= t and 1 <= tl.cols <= t
        assert (seen == 1).all()


def test_partial_tile_tokens_by_hand():
    # side 3, t = 2: tile (0,1) is rows {0,1} x col {2}; tile (1,1) is the single token (2,2)
    tiles = G.key_tiles((1, 3), 1, 2)
    assert [tl.scale for tl in tiles] == [0, 1, 1, 1, 1]
    assert list(tiles[2].tokens()) == [1 + 2, 1 + 3 + 2]
    assert list(tiles[4].tokens()) == [1 + 8]
    assert list(tiles[3].tokens()) == [1 + 6, 1 + 7]
