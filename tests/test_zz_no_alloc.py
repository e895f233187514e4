"""zero_grad_stats_noalloc (statistics with the library's own device scratch,
for callers that cannot allocate) against zero_grad_stats with a caller
workspace: the overflow flag bit-exact and the squared norm within the
1e-5 relative bar for the norm (it differs only in the order of the fp64 sums), over two
calls in a row whose second input is smaller, so that partials left in the
shared scratch by the first call cannot leak into the second."""
import numpy as np
import pytest
import torch

import zero_sharded_mixed_grads_amd as z
from synth import gen
from util import dev, progress


def _grads(n, dtype, seed, phase):
    raw = torch.empty(n + 8, dtype=torch.bfloat16 if dtype == "bf16" else torch.float16,
                      device=dev())
    g = raw[phase:phase + n]
    if n:
        gen.device_fill_normal_(g, seed, 1e-3, 1024.0)
    return raw, g


def _both(g, dtype, n, inv):
    st_ref, st_na = z.new_grad_stats(dev()), z.new_grad_stats(dev())
    ws = z.new_workspace(n, dev())
    z.zero_grad_stats(g, dtype, n, inv, ws, ws.numel(), st_ref)
    z.zero_grad_stats_noalloc(g, dtype, n, inv, st_na)
    torch.cuda.synchronize()
    return z.read_grad_stats(st_ref), z.read_grad_stats(st_na)


def _check(ref, na, label):
    assert na.overflow == ref.overflow, label
    if not ref.overflow:
        assert abs(na.sq_norm - ref.sq_norm) <= 1e-5 * ref.sq_norm, (label, na.sq_norm,
                                                                     ref.sq_norm)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("sizes", [(40_000_003, 1_000_001), (5_000_000, 77), (8_192 * 4096 + 9, 0)])
def test_noalloc_matches_workspace_stats_twice(dtype, sizes):
    inv = 1.0 / 1024.0
    for k, n in enumerate(sizes):
        phase = (3 + k) % 8
        raw, g = _grads(n, dtype, 11 + k, phase)
        ref, na = _both(g, dtype, n, inv)
        _check(ref, na, f"call {k} n={n}")
        if n == 0:
            assert na.sq_norm == 0.0 and na.overflow == 0
        progress(f"noalloc {dtype} call {k}: n={n} phase={phase} sq {na.sq_norm:.12e} vs "
                 f"{ref.sq_norm:.12e}")
        del raw, g


@pytest.mark.gpu
def test_noalloc_overflow_then_clean_and_device_scale():
    """An overflowing call, then a smaller clean one (the flag must clear),
    with the inverse scale read from a device loss-scale state."""
    scale = z.new_loss_scale(dev())
    z.zero_loss_scale_init(z.loss_scaler(init_scale=2.0 ** 10), scale)
    n1, n2 = 3_000_017, 2_999
    raw1, g1 = _grads(n1, "f16", 21, 1)
    g1[n1 // 2] = float("inf")
    raw2, g2 = _grads(n2, "f16", 22, 6)
    for g, n, ov in ((g1, n1, 1), (g2, n2, 0)):
        st_ref, st_na = z.new_grad_stats(dev()), z.new_grad_stats(dev())
        ws = z.new_workspace(n, dev())
        z.zero_grad_stats(g, "f16", n, 1.0, ws, ws.numel(), st_ref, d_scale=scale)
        z.zero_grad_stats_noalloc(g, "f16", n, 1.0, st_na, d_scale=scale)
        torch.cuda.synchronize()
        ref, na = z.read_grad_stats(st_ref), z.read_grad_stats(st_na)
        assert ref.overflow == na.overflow == ov
        _check(ref, na, f"n={n}")
    progress("noalloc: overflow flag set, then cleared on the next, smaller call")
