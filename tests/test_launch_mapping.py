"""Host-side model of AdamW's block -> chunk mapping (the one written in
adamw_stream: tiles renumbered over the 8 XCDs, a capped grid looping over
rounds of tiles), checked for tiny caps and sizes: every 8-element chunk of
the body is updated exactly once, whatever the cap.  The same for the
gather's and the statistics passes' renumbering of tiles (or groups of
tiles) over a grid rounded up to a multiple of 8.  ZeRO-DP Stage 1 ("ZeRO:
Memory Optimizations Toward Training Trillion Parameter Models", paper
summary page): a rank updates all of its part, once."""
import math

import numpy as np
import pytest

BLOCK = 256  # threads per block, one chunk per lane and round


def adam_grid(nchunks, cap):
    g = max(1, min(math.ceil(nchunks / BLOCK), cap))
    return (g + 7) // 8 * 8  # whole rounds of the 8 XCDs


def chunks_updated(nchunks, cap):
    grid = adam_grid(nchunks, cap)
    per_xcd = (grid + 7) // 8
    count = np.zeros(nchunks, np.int64)
    lanes = np.arange(BLOCK)
    for b in range(grid):
        tile = (b % 8) * per_xcd + b // 8
        base = tile * BLOCK + lanes
        while True:
            live = base[base < nchunks]
            if live.size == 0:
                break
            np.add.at(count, live, 1)
            base = base + grid * BLOCK
    return count, grid


@pytest.mark.parametrize("cap", [8, 16, 64])
@pytest.mark.parametrize("nchunks", [0, 1, 255, 256, 257, 8 * 256, 8 * 256 + 1, 64 * 256 * 3 + 7,
                                     70_001])
def test_every_chunk_once(cap, nchunks):
    count, grid = chunks_updated(nchunks, cap)
    assert grid <= max(cap, 8) and grid % 8 == 0
    assert (count == 1).all()


def test_uncapped_grid_is_one_round():
    """Below the cap each block takes at most one tile."""
    nchunks = 123_457
    grid = adam_grid(nchunks, 1 << 30)
    assert grid * BLOCK >= nchunks and (grid - 8) * BLOCK < nchunks
    count, _ = chunks_updated(nchunks, 1 << 30)
    assert (count == 1).all()


def xcd_tile(b, grid):
    """The gather's and the statistics passes' block -> tile (or tile group)
    renumbering: each XCD (block b runs on XCD b mod 8) takes a contiguous
    eighth of a grid rounded up to a multiple of 8."""
    return (b % 8) * (grid // 8) + b // 8


@pytest.mark.parametrize("units", [1, 7, 8, 9, 63, 64, 65, 1000, 8_388_600])
def test_xcd_renumbering_covers_each_unit_once(units):
    """Blocks whose renumbered index is at or past the unit count exit; the
    others cover [0, units) exactly once, and the eight XCDs' shares are
    contiguous runs."""
    grid = (units + 7) // 8 * 8
    b = np.arange(grid)
    t = (b % 8) * (grid // 8) + b // 8
    assert sorted(t.tolist()) == list(range(grid))  # a permutation of the grid
    live = t[t < units]
    assert np.array_equal(np.sort(live), np.arange(units))
    for x in range(8):
        mine = np.sort(t[b % 8 == x])
        assert (np.diff(mine) == 1).all()


@pytest.mark.parametrize("T", [1, 2, 4])
@pytest.mark.parametrize("n_tiles", [1, 3, 4, 5, 31, 32, 33, 64, 4097])
def test_stats_groups_cover_each_tile_once(T, n_tiles):
    """The in-place statistics pass: block b takes the T tiles from
    xcd_tile(b) * T on, skipping tiles past the table; every tile once."""
    groups = (n_tiles + T - 1) // T
    grid = (groups + 7) // 8 * 8
    count = np.zeros(n_tiles, np.int64)
    for b in range(grid):
        tile0 = xcd_tile(b, grid) * T
        if tile0 >= n_tiles:
            continue
        for q in range(T):
            if tile0 + q < n_tiles:
                count[tile0 + q] += 1
    assert (count == 1).all()
