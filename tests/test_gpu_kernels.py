"""Kernel-level parity of the HIP path against the oracle, through the C ABI.

Sizes span several tiles and ragged tails; 16-bit and fp32 buffers are placed
at every phase within a 16-byte line; guard bands around every buffer must
stay untouched.  Bars: flatten, overflow flags, skip and step counter
bit-exact; squared norm within 1e-5 relative; master/m/v within 1e-6 of the
size of each update's terms; 16-bit params within 1 ulp.
"""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_grads_amd as z
from synth import AdamW, gen
from util import Guarded, check_adam_one_step, check_params16, dev

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ flatten
def _rand_bits(rng, n, es):
    if es == 2:
        return rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
    return rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32).view(np.int32)


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("dst_phase", [0, 1, 3, 7])
def test_flatten_ragged_phases(dt, dst_phase):
    es = 4 if dt == "f32" else 2
    dst_phase = dst_phase % (16 // es)
    rng = np.random.default_rng(100 + dst_phase)
    numels = [1, 7, 8, 9, 3, 1000, 4099, 70_001, 2, 16, 33, 262_145, 5]
    host = [_rand_bits(rng, k, es) for k in numels]
    npdt = np.uint16 if es == 2 else np.float32
    srcs = [Guarded(k, npdt, phase=(i * 3) % (16 // es), init=h) for i, (k, h) in
            enumerate(zip(numels, host))]
    psi = sum(numels)
    for lo, hi in [(0, psi), (3, psi - 2), (17, 17 + 5000), (psi - 1, psi), (1009, 1009 + 262_145)]:
        dst = Guarded(hi - lo, npdt, phase=dst_phase)
        z.zero_bucket_flatten([s.ptr() for s in srcs], numels, dt, lo, hi - lo, dst.ptr())
        torch.cuda.synchronize()
        ref = oracle.flatten(host, lo, hi)
        got = dst.host()
        assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), (lo, hi)
        assert dst.canaries_intact()
    assert all(s.canaries_intact() for s in srcs)


def test_flatten_many_segments_and_buckets():
    """More tensors than one launch's segment table; every bucket window."""
    rng = np.random.default_rng(7)
    numels = [int(k) for k in rng.integers(1, 300, 500)]
    host = [_rand_bits(rng, k, 2) for k in numels]
    srcs = [Guarded(k, np.uint16, phase=i % 8, init=h) for i, (k, h) in enumerate(zip(numels, host))]
    psi = sum(numels)
    B = 10_007
    whole = oracle.flatten(host, 0, psi)
    buf = Guarded(B, np.uint16, phase=5)
    for b in range(-(-psi // B)):
        lo, hi = b * B, min((b + 1) * B, psi)
        z.zero_bucket_flatten([s.ptr() for s in srcs], numels, "bf16", lo, hi - lo, buf.ptr())
        torch.cuda.synchronize()
        assert np.array_equal(buf.host()[:hi - lo], whole[lo:hi]), b
        assert buf.canaries_intact()


def test_flatten_empty_and_zero_size_tensors():
    numels = [0, 5, 0, 11, 0]
    host = [np.arange(k, dtype=np.uint16) + 100 * i for i, k in enumerate(numels)]
    srcs = [Guarded(k, np.uint16, init=h) if k else None for k, h in zip(numels, host)]
    ptrs = [s.ptr() if s else None for s in srcs]
    dst = Guarded(16, np.uint16, phase=2)
    z.zero_bucket_flatten(ptrs, numels, "f16", 0, 0, dst.ptr())
    z.zero_bucket_flatten(ptrs, numels, "f16", 2, 14, dst.ptr())
    torch.cuda.synchronize()
    assert np.array_equal(dst.host()[:14], oracle.flatten(host, 2, 16))
    assert dst.canaries_intact()


# ---------------------------------------------------------------- grad stats
def _stats(g: Guarded, dtype, n, inv):
    stats = z.new_grad_stats(dev())
    ws = z.new_workspace(n, dev())
    z.zero_grad_stats(g.ptr(), dtype, n, inv, ws, ws.numel(), stats)
    return z.read_grad_stats(stats)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 1000, 65_537, 1_000_003])
def test_grad_stats_parity(dtype, n):
    rng = np.random.default_rng(n)
    bits = gen.f32_to_bits16((rng.standard_normal(n) * 3.0).astype(np.float32), dtype)
    inv = 2.0 ** -5
    sq_ref, ov_ref = oracle.grad_stats(bits, dtype, inv)
    for phase in range(8):
        g = Guarded(n, np.uint16, phase=phase, init=bits)
        st = _stats(g, dtype, n, inv)
        assert st.overflow == ov_ref == 0
        assert abs(st.sq_norm - sq_ref) <= 1e-12 * sq_ref, (phase, st.sq_norm, sq_ref)
        assert g.canaries_intact()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_grad_stats_overflow_positions(dtype):
    n = 100_003
    rng = np.random.default_rng(1)
    bits = gen.f32_to_bits16(rng.standard_normal(n).astype(np.float32), dtype)
    pinf, ninf, nan = gen.specials(dtype)
    assert _stats(Guarded(n, np.uint16, phase=3, init=bits), dtype, n, 1.0).overflow == 0
    for pos in (0, 1, 5, n // 2, n - 8, n - 1):
        for special in (pinf, ninf, nan, nan | 0x8000):
            b = bits.copy()
            b[pos] = special
            for phase in (0, 5):
                st = _stats(Guarded(n, np.uint16, phase=phase, init=b), dtype, n, 1.0)
                assert st.overflow == 1 == oracle.grad_stats(b, dtype, 1.0)[1], (pos, phase)


def test_grad_stats_extremes_and_determinism():
    n = 300_001
    rng = np.random.default_rng(2)
    # bf16 values spanning the whole exponent range: squares leave fp32 range
    mag = rng.integers(1, 254, n).astype(np.uint32) << 7
    bits = (mag | rng.integers(0, 128, n).astype(np.uint32) |
            (rng.integers(0, 2, n).astype(np.uint32) << 15)).astype(np.uint16)
    sq_ref, _ = oracle.grad_stats(bits, "bf16", 1.0)
    g = Guarded(n, np.uint16, phase=1, init=bits)
    a = _stats(g, "bf16", n, 1.0)
    b = _stats(g, "bf16", n, 1.0)
    assert abs(a.sq_norm - sq_ref) <= 1e-12 * sq_ref
    assert a.sq_norm == b.sq_norm  # bit-reproducible
    # fp16 subnormals only
    sub = rng.integers(1, 1024, n).astype(np.uint16)
    sq_ref, _ = oracle.grad_stats(sub, "f16", 2.0 ** -16)
    st = _stats(Guarded(n, np.uint16, init=sub), "f16", n, 2.0 ** -16)
    assert abs(st.sq_norm - sq_ref) <= 1e-12 * sq_ref


# ----------------------------------------------------------------- AdamW
def _adam_case(n, gdt, pdt, g_phase, p_phase, f_phases, hp, seed, stats_mode="clip",
               inject=None):
    """Runs one zero_adam_step from a random state; returns everything needed
    for the comparison."""
    rng = np.random.default_rng(seed)
    th0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = (rng.random(n) * 1e-8).astype(np.float32)
    gb = gen.f32_to_bits16((rng.standard_normal(n) * 1e-3 / hp.inv_loss_scale).astype(np.float32),
                           gdt)
    if inject is not None:
        for i, b in inject:
            gb[i] = b
    g = Guarded(n, np.uint16, phase=g_phase, init=gb)
    th = Guarded(n, np.float32, phase=f_phases[0], init=th0)
    m = Guarded(n, np.float32, phase=f_phases[1], init=m0)
    v = Guarded(n, np.float32, phase=f_phases[2], init=v0)
    p = Guarded(n, np.uint16, phase=p_phase)
    state = z.new_adam_state(dev())
    stats = None
    if stats_mode != "none":
        stats = z.new_grad_stats(dev())
        ws = z.new_workspace(n, dev())
        z.zero_grad_stats(g.ptr(), gdt, n, hp.inv_loss_scale, ws, ws.numel(), stats)
    z.zero_adam_step(z.adamw(**hp.__dict__), g.ptr(), gdt, th.ptr(), m.ptr(), v.ptr(), p.ptr(),
                     pdt, n, stats, state)
    torch.cuda.synchronize()
    return dict(gb=gb, th0=th0, m0=m0, v0=v0, g=g, th=th, m=m, v=v, p=p, state=state,
                stats=stats)


def _oracle_step(c, hp, gdt, pdt, have_stats, sq=None, ov=None):
    n = c["gb"].size
    if have_stats and sq is None:
        sq, ov = oracle.grad_stats(c["gb"], gdt, hp.inv_loss_scale)
    s = oracle.step_scalars(hp, have_stats, sq or 0.0, ov or 0, 0)
    th, m, v = c["th0"].copy(), c["m0"].copy(), c["v0"].copy()
    p = np.full(n, 0x5A5A, np.uint16)
    oracle.adamw_(s, c["gb"], gdt, th, m, v, p, pdt)
    return s, th, m, v, p


@pytest.mark.parametrize("gdt,pdt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "bf16"),
                                     ("bf16", "f16")])
@pytest.mark.parametrize("n", [1, 5, 8, 9, 1000, 100_003])
def test_adam_one_step_dtypes_sizes(gdt, pdt, n):
    hp = AdamW(max_grad_norm=0.01, inv_loss_scale=2.0 ** -10)
    c = _adam_case(n, gdt, pdt, 0, 0, (0, 0, 0), hp, seed=n)
    st = z.read_grad_stats(c["stats"])
    s, th, m, v, p = _oracle_step(c, hp, gdt, pdt, True, st.sq_norm, st.overflow)
    e = check_adam_one_step(hp, s, oracle.value16(c["gb"], gdt), c["th0"], c["m0"],
                            c["v0"], c["th"].host(), c["m"].host(), c["v"].host(), th, m, v)
    check_params16(c["p"].host(), c["th"].host(), th, pdt)
    sa = z.read_adam_state(c["state"])
    assert sa.step == 1 and sa.skip == 0 and abs(sa.coef - s.coef) <= 1e-12
    for b in ("g", "th", "m", "v", "p"):
        assert c[b].canaries_intact(), b


@pytest.mark.parametrize("g_phase", range(8))
@pytest.mark.parametrize("p_phase", range(8))
def test_adam_16bit_phases(g_phase, p_phase):
    hp = AdamW(max_grad_norm=0.0, inv_loss_scale=2.0 ** -16)
    n = 8 * 1000 + 13
    c = _adam_case(n, "f16", "f16", g_phase, p_phase, (1, 1, 1), hp, seed=g_phase * 8 + p_phase)
    st = z.read_grad_stats(c["stats"])
    s, th, m, v, p = _oracle_step(c, hp, "f16", "f16", True, st.sq_norm, st.overflow)
    e = check_adam_one_step(hp, s, oracle.value16(c["gb"], "f16"), c["th0"], c["m0"],
                            c["v0"], c["th"].host(), c["m"].host(), c["v"].host(), th, m, v)
    check_params16(c["p"].host(), c["th"].host(), th, "f16")
    for b in ("g", "th", "m", "v", "p"):
        assert c[b].canaries_intact(), b


@pytest.mark.parametrize("f_phases", [(0, 0, 0), (1, 1, 1), (2, 2, 2), (3, 3, 3), (0, 1, 2),
                                      (3, 0, 0), (0, 0, 1)])
def test_adam_fp32_phases_and_fallback(f_phases):
    hp = AdamW(max_grad_norm=0.02, inv_loss_scale=1.0)
    for n in (3, 4099, 50_001):
        c = _adam_case(n, "bf16", "bf16", 3, 6, f_phases, hp, seed=n + sum(f_phases))
        st = z.read_grad_stats(c["stats"])
        s, th, m, v, p = _oracle_step(c, hp, "bf16", "bf16", True, st.sq_norm, st.overflow)
        e = check_adam_one_step(hp, s, oracle.value16(c["gb"], "bf16"), c["th0"], c["m0"],
                                c["v0"], c["th"].host(), c["m"].host(), c["v"].host(), th, m, v)
        check_params16(c["p"].host(), c["th"].host(), th, "bf16")
        for b in ("g", "th", "m", "v", "p"):
            assert c[b].canaries_intact(), b


def test_adam_without_stats_never_clips_or_skips():
    hp = AdamW(max_grad_norm=1e-9, inv_loss_scale=2.0 ** -10)
    n = 20_000
    c = _adam_case(n, "f16", "f16", 0, 0, (0, 0, 0), hp, seed=5, stats_mode="none")
    s, th, m, v, p = _oracle_step(c, hp, "f16", "f16", False)
    assert s.coef == 1.0
    check_adam_one_step(hp, s, oracle.value16(c["gb"], "f16"), c["th0"], c["m0"], c["v0"],
                        c["th"].host(), c["m"].host(), c["v"].host(), th, m, v)
    sa = z.read_adam_state(c["state"])
    assert sa.step == 1 and sa.coef == 1.0


_DEGENERATE = {
    "beta1_0": dict(beta1=0.0),
    "beta2_0": dict(beta2=0.0),
    "betas_0": dict(beta1=0.0, beta2=0.0),
    "no_decay": dict(weight_decay=0.0),
    "lr_0": dict(lr=0.0, weight_decay=0.5),
    "heavy_decay": dict(lr=1e-2, weight_decay=50.0),
    "eps_1": dict(eps=1.0),
    "clip_inf": dict(max_grad_norm=float("inf")),
    "zero_grads_clip": dict(max_grad_norm=1.0),
}


@pytest.mark.parametrize("case", list(_DEGENERATE))
def test_adam_degenerate_hyperparameters(case):
    """The edge values the update formula admits: either beta 0 (no history,
    no bias correction), no decay, lr 0 (master unchanged), lr*wd near 1, a
    large eps, an infinite clip threshold (coefficient 1), and an all-zero
    gradient under clipping (norm 0: c / 0 is +inf, so coefficient 1)."""
    kw = dict(max_grad_norm=0.05, inv_loss_scale=2.0 ** -10)
    kw.update(_DEGENERATE[case])
    hp = AdamW(**kw)
    n = 8 * 700 + 5
    inject = [(i, 0) for i in range(n)] if case == "zero_grads_clip" else None
    c = _adam_case(n, "bf16", "f16", 2, 5, (1, 1, 1), hp, seed=len(case), inject=inject)
    st = z.read_grad_stats(c["stats"])
    s, th, m, v, p = _oracle_step(c, hp, "bf16", "f16", True, st.sq_norm, st.overflow)
    if case == "zero_grads_clip":
        assert st.sq_norm == 0.0 and s.coef == 1.0
    if case == "clip_inf":
        assert s.coef == 1.0
    e = check_adam_one_step(hp, s, oracle.value16(c["gb"], "bf16"), c["th0"], c["m0"],
                            c["v0"], c["th"].host(), c["m"].host(), c["v"].host(), th, m, v,
                            label=case)
    check_params16(c["p"].host(), c["th"].host(), th, "f16")
    if case == "lr_0":
        assert np.array_equal(c["th"].host(), c["th0"] + np.float32(0.0))
    sa = z.read_adam_state(c["state"])
    assert sa.step == 1 and sa.skip == 0 and abs(sa.coef - s.coef) <= 1e-12
    for b in ("g", "th", "m", "v", "p"):
        assert c[b].canaries_intact(), b


@pytest.mark.parametrize("pos", ["head", "middle", "tail"])
def test_adam_skip_on_overflow(pos):
    hp = AdamW(max_grad_norm=1.0, inv_loss_scale=2.0 ** -16)
    n = 70_001
    i = {"head": 0, "middle": n // 2, "tail": n - 1}[pos]
    c = _adam_case(n, "f16", "f16", 1, 1, (0, 0, 0), hp, seed=9, inject=[(i, gen.F16_NAN)])
    assert z.read_grad_stats(c["stats"]).overflow == 1
    sa = z.read_adam_state(c["state"])
    assert sa.skip == 1 and sa.step == 0
    assert np.array_equal(c["th"].host(), c["th0"])
    assert np.array_equal(c["m"].host(), c["m0"])
    assert np.array_equal(c["v"].host(), c["v0"])
    assert (c["p"].host() == 0x5A5A).all()  # never written
    for b in ("g", "th", "m", "v", "p"):
        assert c[b].canaries_intact(), b


def test_adam_zero_length_advances_step():
    hp = AdamW()
    state = z.new_adam_state(dev())
    for _ in range(3):
        z.zero_adam_step(z.adamw(**hp.__dict__), None, "f16", None, None, None, None, "f16", 0,
                         None, state)
    assert z.read_adam_state(state).step == 3


def test_adam_step_counter_and_determinism():
    """Several steps from one state, twice: bitwise identical results, and
    the step counter equals the number of non-skipped steps."""
    hp = AdamW(max_grad_norm=0.5, inv_loss_scale=2.0 ** -8)
    n = 123_457
    rng = np.random.default_rng(4)
    th0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    grads = [gen.f32_to_bits16((rng.standard_normal(n) * 0.5).astype(np.float32), "f16")
             for _ in range(4)]
    grads[2][77] = gen.F16_POS_INF
    outs = []
    for _ in range(2):
        th = torch.from_numpy(th0.copy()).to(dev())
        m = torch.zeros_like(th)
        v = torch.zeros_like(th)
        p = torch.zeros(n, dtype=torch.int16, device=dev())
        state, stats = z.new_adam_state(dev()), z.new_grad_stats(dev())
        ws = z.new_workspace(n, dev())
        for gb in grads:
            g = torch.from_numpy(gb.view(np.int16)).to(dev())
            z.zero_grad_stats(g, "f16", n, hp.inv_loss_scale, ws, ws.numel(), stats)
            z.zero_adam_step(z.adamw(**hp.__dict__), g, "f16", th, m, v, p, "f16", n, stats,
                             state)
        outs.append([x.cpu().numpy().copy() for x in (th, m, v, p)])
        assert z.read_adam_state(state).step == 3
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_param_rounding_every_tie(dtype):
    """With lr = wd = 0 the master is unchanged, so the param must be the
    round-to-nearest-even of the given fp32 master.  Inputs: every finite
    16-bit value, every exact midpoint between neighbours (ties), +-1 fp32
    ulp around each midpoint, and values past the largest finite one.
    Reference: numpy (binary16) and torch (bfloat16) rounding."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    if dtype == "f16":
        v = b.view(np.float16).astype(np.float32)
    else:
        v = (b.astype(np.uint32) << 16).view(np.float32)
    v = v[np.isfinite(v)]
    pos = np.sort(v[v >= 0].astype(np.float64))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)  # exact ties
    x = np.concatenate([v, mids, -mids, np.nextafter(mids, np.float32(np.inf)),
                        np.nextafter(mids, np.float32(0)),
                        np.float32([65519.99, 65520.0, 1e5, 3.4e38, -3.4e38])])
    n = x.size
    hp = AdamW(lr=0.0, weight_decay=0.0)
    g = Guarded(n, np.uint16, phase=3, init=np.zeros(n, np.uint16))
    th = Guarded(n, np.float32, phase=0, init=x)
    m = Guarded(n, np.float32, phase=0, init=np.zeros(n, np.float32))
    v_ = Guarded(n, np.float32, phase=0, init=np.zeros(n, np.float32))
    p = Guarded(n, np.uint16, phase=5)
    state = z.new_adam_state(dev())
    z.zero_adam_step(z.adamw(**hp.__dict__), g.ptr(), dtype, th.ptr(), m.ptr(), v_.ptr(), p.ptr(),
                     dtype, n, None, state)
    torch.cuda.synchronize()
    # master unchanged in value (IEEE arithmetic maps -0 - 0*(-0) to +0)
    assert np.array_equal(th.host(), x)
    xr = x + np.float32(0.0)  # the same -0 -> +0 mapping for the reference
    with np.errstate(over="ignore"):
        ref = (xr.astype(np.float16).view(np.uint16) if dtype == "f16" else
               torch.from_numpy(xr).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    got = p.host()
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]
    assert p.canaries_intact()


# ------------------------------------------------- gather fused with stats
def _fused(srcs, numels, dtype, lo, hi, dst, inv):
    ws_bytes = z.zero_bucket_flatten_stats_workspace(numels, lo, hi - lo)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev())
    stats = z.new_grad_stats(dev())
    z.zero_bucket_flatten_stats([s.ptr() if s is not None else None for s in srcs], numels, dtype,
                                lo, hi - lo, dst.ptr(), inv, ws, ws_bytes, stats)
    return z.read_grad_stats(stats)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("dst_phase", [0, 3, 7])
def test_flatten_stats_parity(dtype, dst_phase):
    rng = np.random.default_rng(200 + dst_phase)
    numels = [1, 7, 8, 9, 3, 1000, 4099, 70_001, 2, 16, 33, 262_145, 5, 600_000]
    host = [gen.f32_to_bits16((rng.standard_normal(k) * 5).astype(np.float32), dtype)
            for k in numels]
    srcs = [Guarded(k, np.uint16, phase=(i * 5) % 8, init=h) for i, (k, h) in
            enumerate(zip(numels, host))]
    psi = sum(numels)
    inv = 2.0 ** -3
    for lo, hi in [(0, psi), (3, psi - 2), (17, 17 + 5000), (psi - 1, psi), (1009, 1009 + 262_145)]:
        dst = Guarded(hi - lo, np.uint16, phase=dst_phase)
        st = _fused(srcs, numels, dtype, lo, hi, dst, inv)
        torch.cuda.synchronize()
        ref = oracle.flatten(host, lo, hi)
        assert np.array_equal(dst.host(), ref), (lo, hi)
        sq, ov = oracle.grad_stats(ref, dtype, inv)
        assert st.overflow == ov == 0 and abs(st.sq_norm - sq) <= 1e-12 * sq, (lo, hi)
        # the same value zero_grad_stats reports for the gathered buffer
        st2 = _stats(dst, dtype, hi - lo, inv)
        assert abs(st2.sq_norm - st.sq_norm) <= 1e-14 * sq and st2.overflow == 0
        assert dst.canaries_intact()
        st3 = _fused(srcs, numels, dtype, lo, hi, dst, inv)  # bit-reproducible
        assert st3.sq_norm == st.sq_norm
    assert all(s.canaries_intact() for s in srcs)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_flatten_stats_overflow_and_many_segments(dtype):
    rng = np.random.default_rng(9)
    numels = [int(k) for k in rng.integers(1, 3000, 300)]   # several launches of segments
    host = [gen.f32_to_bits16(rng.standard_normal(k).astype(np.float32), dtype) for k in numels]
    psi = sum(numels)
    pinf, ninf, nan = gen.specials(dtype)
    srcs = [Guarded(k, np.uint16, phase=i % 8, init=h) for i, (k, h) in enumerate(zip(numels, host))]
    dst = Guarded(psi, np.uint16, phase=1)
    st = _fused(srcs, numels, dtype, 0, psi, dst, 1.0)
    sq, ov = oracle.grad_stats(oracle.flatten(host, 0, psi), dtype, 1.0)
    assert st.overflow == ov == 0 and abs(st.sq_norm - sq) <= 1e-12 * sq
    offs = np.cumsum([0] + numels)
    for ti, pos, special in [(0, 0, pinf), (150, numels[150] // 2, nan), (299, numels[299] - 1, ninf),
                             (77, 0, nan | 0x8000)]:
        h = host[ti].copy()
        h[pos] = special
        src = Guarded(numels[ti], np.uint16, phase=ti % 8, init=h)
        ss = list(srcs)
        ss[ti] = src
        st = _fused(ss, numels, dtype, 0, psi, dst, 1.0)
        assert st.overflow == 1, (ti, pos)
        g = dst.host()
        assert g[offs[ti] + pos] == special
    # empty range writes {0, 0}
    st = _fused(srcs, numels, dtype, 10, 10, dst, 1.0)
    assert st.overflow == 0 and st.sq_norm == 0.0
