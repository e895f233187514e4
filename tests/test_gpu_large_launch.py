"""Gathers and gradient statistics too large for one kernel launch.

The library keeps a dispatch below 2^31 work-items, so with 256-thread
blocks one launch has at most 8,388,600 blocks.  The gather takes one
2,048-element tile of 16-bit values per block, and the statistics one
4,096-gradient tile.  So a single 16-bit tensor of more than 8,388,600 x 2,048
elements (34 GB) has to be split across gather launches, and more than
8,388,600 x 4,096 gradients (69 GB) across statistics launches.  These sizes
fit one MI355X.

Both cases are checked against properties that hold at any size, with no
oracle pass over 10^10 elements:
- the gathered buffer equals its source byte for byte;
- the values repeat a short pattern of small dyadic fp16 numbers, so every
  partial sum of squares is an integer multiple of 2^-6 below 2^53 * 2^-6 and
  is exact in fp64, whatever the summation order.  The squared norm must
  therefore equal the closed form exactly, and the overflow flag must be 0.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import zero_sharded_mixed_grads_amd as z
from util import dev, progress

MAX_LAUNCH_BLOCKS = 0x7FFFFFFF // 256 // 8 * 8
PATTERN = [0.5, -1.0, 1.5, 2.0, -0.25, 3.0, 0.125]  # exact in fp16; squares are k / 64


def _need(nbytes):
    free, _ = torch.cuda.mem_get_info(dev())
    if free < nbytes + (4 << 30):
        pytest.skip(f"needs {nbytes / 1e9:.0f} GB of free device memory, {free / 1e9:.0f} GB free")


def _fill_pattern(buf):
    """buf[i] = PATTERN[i mod len(PATTERN)] for a 1-D fp16 tensor."""
    p = len(PATTERN)
    pat = torch.tensor(PATTERN, dtype=torch.float16, device=buf.device)
    rows = buf.numel() // p
    buf[:rows * p].view(rows, p).copy_(pat.expand(rows, p))
    rest = buf.numel() - rows * p
    if rest:
        buf[rows * p:].copy_(pat[:rest])


def _sq_norm_closed_form(first, n):
    """Sum of squares of PATTERN[i mod p] for i in [first, first + n), exactly."""
    p = len(PATTERN)
    per = [Fraction(v) ** 2 for v in PATTERN]
    full, rest = divmod(n, p)
    total = full * sum(per)
    for i in range(first, first + rest):
        total += per[i % p]
    return total


def _equal_chunked(a, b, chunk=1 << 30):
    for lo in range(0, a.numel(), chunk):
        if not torch.equal(a[lo:lo + chunk], b[lo:lo + chunk]):
            return False
    return True


@pytest.mark.gpu
def test_gather_stats_split_across_launches():
    """One tensor of more than a launch's worth of tiles, at source phase 1:
    the gather splits it between two launches; the copy is exact and the
    fused squared norm equals the closed form."""
    n = MAX_LAUNCH_BLOCKS * 2048 + 10_001
    _need(4 * n + 16 + (256 << 20))
    raw = torch.empty(n + 8, dtype=torch.float16, device=dev())
    _fill_pattern(raw)
    src = raw[1:1 + n]                    # 16-bit phase 1 within its line
    dst = torch.empty(n, dtype=torch.float16, device=dev())
    ws_n = z.zero_bucket_flatten_stats_workspace([n], 0, n)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev())
    stats = z.new_grad_stats(dev())
    progress(f"  gather of {n} fp16 elements")
    z.zero_bucket_flatten_stats([src], [n], "f16", 0, n, dst, 1.0, ws, ws_n, stats)
    torch.cuda.synchronize()
    st = z.read_grad_stats(stats)
    assert st.overflow == 0
    assert Fraction(st.sq_norm) == _sq_norm_closed_form(1, n)
    assert _equal_chunked(dst, src)
    # a range that starts inside the tensor and ends one element short of it
    del ws
    lo, cnt = 3, n - 4
    ws_n = z.zero_bucket_flatten_stats_workspace([n], lo, cnt)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev())
    dst2 = dst[:cnt]
    dst2.zero_()
    z.zero_bucket_flatten_stats([src], [n], "f16", lo, cnt, dst2, 1.0, ws, ws_n, stats)
    torch.cuda.synchronize()
    st = z.read_grad_stats(stats)
    assert st.overflow == 0
    assert Fraction(st.sq_norm) == _sq_norm_closed_form(1 + lo, cnt)
    assert _equal_chunked(dst2, src[lo:lo + cnt])
    del raw, src, dst, dst2, ws
    torch.cuda.empty_cache()


@pytest.mark.gpu
def test_grad_stats_split_across_launches():
    """More gradients than one launch's worth of statistics tiles."""
    n = MAX_LAUNCH_BLOCKS * 4096 + 777
    _need(2 * n + 16 + (256 << 20))
    raw = torch.empty(n + 8, dtype=torch.float16, device=dev())
    _fill_pattern(raw)
    g = raw[3:3 + n]                      # 16-bit phase 3 within its line
    ws = z.new_workspace(n, dev())
    stats = z.new_grad_stats(dev())
    progress(f"  statistics of {n} fp16 gradients")
    z.zero_grad_stats(g, "f16", n, 1.0, ws, ws.numel(), stats)
    torch.cuda.synchronize()
    st = z.read_grad_stats(stats)
    assert st.overflow == 0
    assert Fraction(st.sq_norm) == _sq_norm_closed_form(3, n)
    # one non-finite value anywhere still raises the flag
    raw[3 + n - 1] = float("inf")
    z.zero_grad_stats(g, "f16", n, 1.0, ws, ws.numel(), stats)
    torch.cuda.synchronize()
    assert z.read_grad_stats(stats).overflow == 1
    del raw, g, ws
    torch.cuda.empty_cache()


def test_closed_form_is_exact():
    """The pattern's squares are multiples of 2^-6 and the sums stay far below
    2^53 of those units, so fp64 holds every partial sum exactly."""
    assert all(np.float16(v) == v for v in PATTERN)
    n = MAX_LAUNCH_BLOCKS * 4096 + 777
    assert _sq_norm_closed_form(0, n) * 64 < 2 ** 53
    assert all((Fraction(v) ** 2 * 64).denominator == 1 for v in PATTERN)
