"""Paths that a launch takes only beyond the per-launch block cap, run on
small inputs through a second build of the same sources whose cap is 64
blocks instead of 8,388,600 (ZeRO-DP Stage 1 on the paper summary page of
"ZeRO: Memory Optimizations Toward Training Trillion Parameter Models": a
rank updates its whole 1/Nd part, whatever its size):
- AdamW's capped grid loops over several rounds of tiles, with the tiles of
  each round renumbered over the 8 XCDs, and the neighbour-lane exchange of
  unaligned 16-bit streams in every round (above about 17e9 parameters with
  the real cap);
- the statistics pass goes out in several launches (above 34e9 gradients);
- the gather splits its segment table and a single tensor across launches
  (above 17e9 16-bit elements).
Each result must equal the default build's bit for bit (the kernels and the
fixed reduction order are the same; only the grid differs), and AdamW's the
oracle's within the one-step bar."""
import contextlib
import os

import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_grads_amd as z
from synth import AdamW, gen
from util import Guarded, check_adam_one_step, check_params16, dev, progress

CAPPED = os.path.join(os.path.dirname(z.LIB_PATH), "libzero_mi355x_capped.so")
CAP = 64
_capped_lib = None


@contextlib.contextmanager
def capped():
    global _capped_lib
    if _capped_lib is None:
        _capped_lib = z.load(CAPPED)
    saved = z._lib
    z._lib = _capped_lib
    try:
        yield
    finally:
        z._lib = saved


def _state(n, g_phase, p_phase, f_phase, seed):
    rng = np.random.default_rng(seed)
    th0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = (rng.random(n) * 1e-8).astype(np.float32)
    gb = gen.f32_to_bits16((rng.standard_normal(n) * 1e-3 * 1024).astype(np.float32), "f16")
    bufs = dict(g=Guarded(n, np.uint16, g_phase, gb), th=Guarded(n, np.float32, f_phase, th0),
                m=Guarded(n, np.float32, f_phase, m0), v=Guarded(n, np.float32, f_phase, v0),
                p=Guarded(n, np.uint16, p_phase))
    return dict(gb=gb, th0=th0, m0=m0, v0=v0, **bufs)


def _adam(c, hp, n):
    stats, state = z.new_grad_stats(dev()), z.new_adam_state(dev())
    ws = z.new_workspace(n, dev())
    z.zero_grad_stats(c["g"].ptr(), "f16", n, hp.inv_loss_scale, ws, ws.numel(), stats)
    z.zero_adam_step(z.adamw(**hp.__dict__), c["g"].ptr(), "f16", c["th"].ptr(), c["m"].ptr(),
                     c["v"].ptr(), c["p"].ptr(), "f16", n, stats, state)
    torch.cuda.synchronize()
    return z.read_grad_stats(stats), z.read_adam_state(state)


def _raw(c):
    return {k: c[k].raw.cpu().numpy().copy() for k in ("th", "m", "v", "p")}


@pytest.mark.gpu
def test_capped_build_is_loaded():
    with capped():
        assert z.lib()._name == CAPPED
    assert z.lib()._name == z.LIB_PATH


@pytest.mark.gpu
@pytest.mark.parametrize("g_phase", range(8))
@pytest.mark.parametrize("p_phase", range(8))
def test_adamw_rounds_equal_default_build(g_phase, p_phase):
    """8 * 70,000 + 13 elements: 274 tiles of 2,048 on a 64-block grid, five
    rounds, the last one partial; a 1-element fp32 head."""
    n = 8 * 70_000 + 13
    hp = AdamW(max_grad_norm=0.5, inv_loss_scale=1.0 / 1024)
    seed = 8 * g_phase + p_phase
    ref = _state(n, g_phase, p_phase, 3, seed)
    st_ref, ad_ref = _adam(ref, hp, n)
    cap = _state(n, g_phase, p_phase, 3, seed)
    with capped():
        st_cap, ad_cap = _adam(cap, hp, n)
    assert st_cap.sq_norm == st_ref.sq_norm and st_cap.overflow == st_ref.overflow == 0
    assert ad_cap.step == ad_ref.step == 1 and ad_cap.coef == ad_ref.coef
    a, b = _raw(ref), _raw(cap)
    for k in a:  # guard bands included: the canaries are intact on both
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
    for k in ("g", "th", "m", "v", "p"):
        assert cap[k].canaries_intact(), k
    if (g_phase, p_phase) in ((0, 0), (1, 1), (7, 2)):
        s = oracle.step_scalars(hp, True, st_cap.sq_norm, 0, 0)
        th, m, v = cap["th0"].copy(), cap["m0"].copy(), cap["v0"].copy()
        p = np.zeros(n, np.uint16)
        oracle.adamw_(s, cap["gb"], "f16", th, m, v, p, "f16")
        e = check_adam_one_step(hp, s, oracle.value16(cap["gb"], "f16"), cap["th0"], cap["m0"],
                                cap["v0"], cap["th"].host(), cap["m"].host(), cap["v"].host(),
                                th, m, v, label="capped")
        check_params16(cap["p"].host(), cap["th"].host(), th, "f16", "capped")
        progress(f"capped AdamW phases ({g_phase}, {p_phase}) vs oracle: {e}")


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_stats_launch_pieces_equal_default_build(dtype):
    """2,000,003 gradients at phase 3: 489 tiles of 4,096, eight launches."""
    n = 2_000_003
    raw = torch.empty(n + 8, dtype=torch.float16 if dtype == "f16" else torch.bfloat16,
                      device=dev())
    g = raw[3:3 + n]
    gen.device_fill_normal_(g, 5, 1e-3, 1024.0)
    out = []
    for ctx in (contextlib.nullcontext(), capped()):
        with ctx:
            st = z.new_grad_stats(dev())
            ws = z.new_workspace(n, dev())
            z.zero_grad_stats(g, dtype, n, 1.0 / 1024, ws, ws.numel(), st)
            torch.cuda.synchronize()
            out.append(z.read_grad_stats(st))
    assert out[0].sq_norm == out[1].sq_norm and out[0].overflow == out[1].overflow == 0
    sq, ov = oracle.grad_stats(g.view(torch.int16).cpu().numpy().view(np.uint16), dtype,
                               1.0 / 1024)
    assert ov == 0 and abs(out[1].sq_norm - sq) <= 1e-12 * sq


@pytest.mark.gpu
@pytest.mark.parametrize("stats", [False, True])
def test_gather_launch_pieces_equal_default_build(stats):
    """Five fp16 tensors (one of 1,000,000 elements, 489 tiles) gathered into
    a destination at phase 5: a dozen launches, the large tensor split across
    launches at line boundaries."""
    numels = [300_001, 7, 1_000_000, 33, 200_000]
    host = [gen.f32_to_bits16((np.random.default_rng(i).standard_normal(k) * 0.5)
                              .astype(np.float32), "f16") for i, k in enumerate(numels)]
    ts = [torch.from_numpy(h.view(np.int16)).to(dev()) for h in host]
    lo, hi = 5, sum(numels) - 3
    outs = []
    for ctx in (contextlib.nullcontext(), capped()):
        with ctx:
            dst = Guarded(hi - lo, np.uint16, 5)
            st = z.new_grad_stats(dev())
            if stats:
                nb = z.zero_bucket_flatten_stats_workspace(numels, lo, hi - lo)
                ws = torch.empty(nb, dtype=torch.uint8, device=dev())
                z.zero_bucket_flatten_stats(ts, numels, "f16", lo, hi - lo, dst.ptr(), 1.0, ws,
                                            nb, st)
            else:
                z.zero_bucket_flatten(ts, numels, "f16", lo, hi - lo, dst.ptr())
            torch.cuda.synchronize()
            assert dst.canaries_intact()
            outs.append((dst.host().copy(), z.read_grad_stats(st)))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[1][0], oracle.flatten(host, lo, hi))
    if stats:
        assert outs[0][1].sq_norm == outs[1][1].sq_norm and outs[1][1].overflow == 0
        sq, _ = oracle.grad_stats(outs[1][0], "f16", 1.0)
        assert abs(outs[1][1].sq_norm - sq) <= 1e-12 * sq


@pytest.mark.gpu
@pytest.mark.parametrize("p_phase", [0, 3])
@pytest.mark.parametrize("f_phase", [0, 1])
def test_tensor_step_launch_pieces_equal_default_build(p_phase, f_phase):
    """The step read in place from five tensors (one of 1,000,000 elements, 489
    tiles) over a dozen launches of at most 64 tiles, the large tensor split
    between launches: statistics and every output equal the default build's bit
    for bit."""
    numels = [300_001, 7, 1_000_000, 33, 200_000]
    lo, hi = 5, sum(numels) - 3
    n = hi - lo
    host = [gen.f32_to_bits16((np.random.default_rng(10 + i).standard_normal(k) * 1e-3 * 1024)
                              .astype(np.float32), "f16") for i, k in enumerate(numels)]
    ts = [torch.from_numpy(h.view(np.int16)).to(dev()) for h in host]
    hp = AdamW(max_grad_norm=0.5, inv_loss_scale=1.0 / 1024)
    outs = []
    for ctx in (contextlib.nullcontext(), capped()):
        with ctx:
            c = _state(n, 0, p_phase, f_phase, 99)
            gs, st = z.new_grad_stats(dev()), z.new_adam_state(dev())
            nb = z.zero_bucket_flatten_stats_workspace(numels, lo, n)
            ws = torch.empty(nb, dtype=torch.uint8, device=dev())
            for _ in range(2):
                z.zero_grad_stats_tensors(ts, numels, "f16", lo, n, hp.inv_loss_scale, ws, nb, gs)
                z.zero_adam_step_tensors(z.adamw(**hp.__dict__), ts, numels, "f16", lo, n,
                                         c["th"].ptr(), c["m"].ptr(), c["v"].ptr(), c["p"].ptr(),
                                         "f16", gs, st)
            torch.cuda.synchronize()
            for k in ("th", "m", "v", "p"):
                assert c[k].canaries_intact(), k
            outs.append((z.read_grad_stats(gs), _raw(c), bytes(st.cpu().numpy())))
    (sa, ra, ta), (sb, rb, tb) = outs
    assert sa.sq_norm == sb.sq_norm and sa.overflow == sb.overflow == 0 and ta == tb
    for k in ra:
        assert np.array_equal(ra[k].view(np.uint8), rb[k].view(np.uint8)), k
