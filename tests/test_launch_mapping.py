"""Host-side model of AdamW's block -> chunk mapping (the one written in
adamw_stream: tiles renumbered over the 8 XCDs, a capped grid looping over
rounds of tiles), checked for tiny caps and sizes: every 8-element chunk of
the body is updated exactly once, whatever the cap.  ZeRO-DP Stage 1 ("ZeRO:
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
