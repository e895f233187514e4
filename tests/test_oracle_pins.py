"""Pins of the oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  None re-types the oracle's own formula:
each compares it against a printed value from the pages (tests/golden), a
closed form that follows from the update, a library routine (numpy, torch),
an exact-rational brute force, or an invariant.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from oracle import brute
from synth import AdamW

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- partition
@pytest.mark.parametrize("psi", list(range(0, 301, 7)) + [299, 300])
def test_partition_tiles_and_matches_array_split(psi):
    for nd in range(1, 34):
        ranges = [oracle.partition(psi, nd, r) for r in range(nd)]
        assert ranges[0][0] == 0 and ranges[-1][1] == psi
        for (b0, e0), (b1, e1) in zip(ranges, ranges[1:]):
            assert e0 == b1
        lens = [e - b for b, e in ranges]
        assert max(lens) - min(lens) <= 1
        # numpy documents array_split: the first (l mod n) parts have l//n + 1
        parts = np.array_split(np.arange(psi), nd)
        assert [len(p) for p in parts] == lens
        for (b, e), p in zip(ranges, parts):
            assert list(range(b, e)) == list(p)


def test_partition_single_rank_and_errors():
    assert oracle.partition(12345, 1, 0) == (0, 12345)
    with pytest.raises(ValueError):
        oracle.partition(10, 0, 0)
    with pytest.raises(ValueError):
        oracle.partition(10, 4, 4)


@pytest.mark.parametrize("psi,nd", [(7_459_729_408, 8), (100_291_305_472, 400),
                                    (12_848_143_360, 1), ((1 << 40) + 3, 1024)])
def test_partition_at_workload_scale(psi, nd):
    ranges = [oracle.partition(psi, nd, r) for r in range(nd)]
    assert ranges[0][0] == 0 and ranges[-1][1] == psi
    assert all(a[1] == b[0] for a, b in zip(ranges, ranges[1:]))
    q, rem = divmod(psi, nd)
    assert [e - b for b, e in ranges] == [q + 1] * rem + [q] * (nd - rem)


# ---------------------------------------------------------------- accounting
def test_accounting_reproduces_the_papers_table():
    g = golden("zero_dp_memory_table.json")
    for nd, row in g["rows"].items():
        for stage, printed in zip(g["stage_of_column"], row):
            val = oracle.mem_bytes(stage, g["psi"], int(nd), g["K"]) / g["unit_bytes"]
            decimals = len(printed.split(".")[1]) if "." in printed else 0
            assert f"{val:.{decimals}f}" == printed, (nd, stage, val, printed)


def test_accounting_sixteen_bytes_per_param_and_gpt2():
    g = golden("memory_model.json")
    bpp = g["bytes_per_param"]
    assert bpp["fp16_params"] + bpp["fp16_grads"] + bpp["K"] == bpp["total"]
    for psi in (1, 1000, 7_500_000_000):
        assert oracle.mem_bytes(0, psi, 1, bpp["K"]) == bpp["total"] * psi
        for stage in range(4):  # with one rank nothing is sharded
            assert oracle.mem_bytes(stage, psi, 1, bpp["K"]) == bpp["total"] * psi
    gp = g["gpt2_1p5b"]
    assert oracle.mem_bytes(0, gp["psi"], 1, 12) >= gp["at_least_bytes"]


def test_accounting_large_nd_limits():
    g = golden("memory_model.json")["large_nd_reduction"]
    psi = 7_500_000_000
    nd = 1 << 20
    full = oracle.mem_bytes(0, psi, nd, 12)
    assert abs(full / oracle.mem_bytes(1, psi, nd, 12) - g["stage1_factor"]) < 1e-4
    assert abs(full / oracle.mem_bytes(2, psi, nd, 12) - g["stage2_factor"]) < 1e-3
    for nd in (2, 4, 64, 1000):  # stage 3 divides everything exactly when nd | psi
        assert oracle.mem_bytes(3, psi, nd, 12) * nd == full


def test_accounting_stage1_formula_and_ceil():
    g = golden("memory_model.json")["stage1_formula"]
    for psi, nd, k in [(7_500_000_000, 64, 12), (1000, 7, 12), (999, 1000, 8)]:
        largest = -(-psi // nd)
        assert oracle.mem_bytes(1, psi, nd, k) == g["params_plus_grads_bytes_per_param"] * psi + k * largest
    # the busiest rank: ceil, so that rank 0 of a ragged split is covered
    b, e = oracle.partition(1001, 10, 0)
    assert oracle.mem_bytes(3, 1001, 10, 12) == 16 * (e - b)


def test_accounting_monotone_in_stage_and_errors():
    for psi, nd in [(10**9, 8), (12345, 7), (5, 9)]:
        vals = [oracle.mem_bytes(s, psi, nd, 12) for s in range(4)]
        assert vals == sorted(vals, reverse=True)
    with pytest.raises(ValueError):
        oracle.mem_bytes(4, 10, 1, 12)
    with pytest.raises(ValueError):
        oracle.mem_bytes(1, 10, 0, 12)


# ----------------------------------------------------- bucket plan / flatten
def _apply_plan(tensors, segs, count):
    out = np.zeros(count, dtype=tensors[0].dtype)
    for s in segs:
        out[s.dst_off:s.dst_off + s.len] = tensors[s.tensor][s.src_off:s.src_off + s.len]
    return out


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(1, 40), min_size=1, max_size=12), st.integers(1, 50),
       st.data())
def test_bucket_plan_matches_torch_cat(numels, bucket, data):
    psi = sum(numels)
    lo = data.draw(st.integers(0, psi))
    hi = data.draw(st.integers(lo, psi))
    rng = np.random.default_rng(len(numels) * 1000 + bucket)
    tensors = [rng.integers(0, 1 << 16, k).astype(np.uint16) for k in numels]
    segs = oracle.bucket_plan(numels, bucket, lo, hi)
    ref = torch.cat([torch.from_numpy(t.view(np.int16)) for t in tensors]).numpy()[lo:hi]
    assert np.array_equal(_apply_plan(tensors, segs, hi - lo).view(np.int16), ref)
    # segments tile [0, hi-lo) in order and never straddle a window
    off = 0
    for s in segs:
        assert s.dst_off == off and s.len > 0
        g0 = lo + s.dst_off
        assert g0 // bucket == s.bucket == (g0 + s.len - 1) // bucket
        off += s.len
    assert off == hi - lo


def test_buckets_concatenate_to_the_flat_stream():
    numels = [7, 1, 130, 64, 3]
    psi = sum(numels)
    tensors = [np.arange(k, dtype=np.float32) + 1000 * i for i, k in enumerate(numels)]
    for bucket in (1, 5, 64, 65, 204, 205, 10_000):
        nb = -(-psi // bucket)
        parts = []
        for b in range(nb):
            lo, hi = b * bucket, min((b + 1) * bucket, psi)
            segs = oracle.bucket_plan(numels, bucket, lo, hi)
            assert all(s.bucket == b for s in segs)
            parts.append(_apply_plan(tensors, segs, hi - lo))
        assert np.array_equal(np.concatenate(parts), np.concatenate(tensors))
        assert np.array_equal(np.concatenate(parts), oracle.flatten(tensors, 0, psi))


def test_bucket_plan_errors():
    with pytest.raises(ValueError):
        oracle.bucket_plan([3, 4], 0, 0, 7)
    with pytest.raises(ValueError):
        oracle.bucket_plan([3, 4], 2, 5, 4)
    with pytest.raises(ValueError):
        oracle.bucket_plan([3, 4], 2, 0, 8)
    assert oracle.bucket_plan([3, 4], 2, 3, 3) == []


# ------------------------------------------------------- 16-bit conversions
def _all16():
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def test_decode_f16_matches_numpy_for_every_pattern():
    b = _all16()
    ref = b.view(np.float16).astype(np.float64)
    got = oracle.value16(b, "f16")
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_bf16_matches_torch_for_every_pattern():
    b = _all16()
    ref = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = oracle.value16(b, "bf16")
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _probe_f32(dtype):
    """fp32 values around every 16-bit grid point and midpoint, plus random
    values over the whole range (normal, subnormal, overflowing)."""
    b = _all16()
    if dtype == "f16":
        v = b.view(np.float16).astype(np.float32)
    else:
        v = (b.astype(np.uint32) << 16).view(np.float32)
    v = v[np.isfinite(v)]
    s = np.sort(v[v >= 0].astype(np.float64))
    mids = ((s[:-1] + s[1:]) / 2).astype(np.float32)
    pts = np.concatenate([v, mids, -mids])
    near = np.concatenate([np.nextafter(pts, np.float32(np.inf)),
                           np.nextafter(pts, np.float32(-np.inf))])
    rng = np.random.default_rng(7)
    rnd = rng.integers(0, 1 << 32, 2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    rnd = rnd[np.isfinite(rnd)]
    return np.concatenate([pts, near, rnd, np.float32([np.inf, -np.inf, 0.0, -0.0])])


def test_round_to_f16_matches_numpy():
    x = _probe_f32("f16")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.bits16(x, "f16"), ref)
    assert oracle.bits16(np.float32([np.nan]), "f16")[0] & 0x7C00 == 0x7C00


def test_round_to_bf16_matches_torch():
    x = _probe_f32("bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bits16(x, "bf16"), ref)


# --------------------------------------------------------------- grad stats
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n,inv", [(1, 1.0), (977, 2.0**-10), (10_000, 2.0**-16), (4096, 0.3)])
def test_grad_stats_exact_rational(dtype, n, inv):
    rng = np.random.default_rng(n)
    bits = rng.integers(0, 1 << 16, n).astype(np.uint16)
    # keep finite values
    vals = oracle.value16(bits, dtype)
    bits = bits[np.isfinite(vals)]
    sq, ov = oracle.grad_stats(bits, dtype, inv)
    assert ov == 0
    exact = brute.sq_norm(bits, dtype, inv)
    assert abs(Fraction(sq) - exact) <= exact * Fraction(1, 10**15)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_grad_stats_constant_and_library(dtype):
    g = np.float32(0.125)
    bits = np.full(100_003, oracle.bits16(np.float32([g]), dtype)[0], dtype=np.uint16)
    sq, ov = oracle.grad_stats(bits, dtype, 2.0**-3)
    assert ov == 0 and sq == 100_003 * (0.125 * 2.0**-3) ** 2
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(300_000) * 40).astype(np.float32)
    bits = oracle.bits16(x, dtype)
    vals = torch.from_numpy(bits.view(np.int16).copy()).view(
        torch.float16 if dtype == "f16" else torch.bfloat16).double()
    ref = float(torch.linalg.vector_norm(vals * 2.0**-6) ** 2)
    sq, _ = oracle.grad_stats(bits, dtype, 2.0**-6)
    assert abs(sq - ref) <= 1e-12 * ref


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_grad_stats_overflow_flag(dtype):
    rng = np.random.default_rng(11)
    n = 5000
    x = rng.standard_normal(n).astype(np.float32)
    bits = oracle.bits16(x, dtype)
    assert oracle.grad_stats(bits, dtype, 1.0)[1] == 0
    pinf, ninf, nan = (0x7C00, 0xFC00, 0x7E00) if dtype == "f16" else (0x7F80, 0xFF80, 0x7FC0)
    for pos in (0, n // 2, n - 1):
        for special in (pinf, ninf, nan, nan | 0x8000, nan | 1):
            b = bits.copy()
            b[pos] = special
            ref = not np.isfinite(oracle.value16(b, dtype)).all()
            assert ref and oracle.grad_stats(b, dtype, 1.0)[1] == 1
    # largest finite values do not overflow
    big = 0x7BFF if dtype == "f16" else 0x7F7F
    assert oracle.grad_stats(np.full(10, big, np.uint16), dtype, 1.0)[1] == 0


def test_grad_stats_sharding_additivity():
    rng = np.random.default_rng(5)
    bits = oracle.bits16(rng.standard_normal(100_000).astype(np.float32), "f16")
    whole, _ = oracle.grad_stats(bits, "f16", 0.5)
    for nd in (2, 3, 7):
        parts = [oracle.grad_stats(bits[slice(*oracle.partition(bits.size, nd, r))], "f16", 0.5)[0]
                 for r in range(nd)]
        assert abs(math.fsum(parts) - whole) <= 1e-14 * whole


def test_grad_stats_empty():
    assert oracle.grad_stats(np.zeros(0, np.uint16), "f16", 1.0) == (0.0, 0)


# ------------------------------------------------------------ step scalars
def test_step_scalars_clip_and_skip():
    hp = AdamW(max_grad_norm=1.0, inv_loss_scale=2.0**-16)
    s = oracle.step_scalars(hp, True, 16.0, 0, 4)
    assert s.t == 5 and s.skip == 0 and s.coef == 0.25
    assert s.bc1 == 1 - 0.9**5 and abs(s.bc2 - (1 - 0.999**5)) < 1e-16
    s = oracle.step_scalars(hp, True, 0.25, 0, 4)   # norm 0.5 <= c: no clip
    assert s.coef == 1.0
    s = oracle.step_scalars(hp, True, 0.0, 0, 0)    # zero grads: no clip
    assert s.coef == 1.0 and s.t == 1
    s = oracle.step_scalars(hp, True, 123.0, 1, 7)  # overflow: skipped, t unchanged
    assert s.skip == 1 and s.t == 7
    s = oracle.step_scalars(hp, False, 123.0, 1, 7)  # no statistics: never skip, no clip
    assert s.skip == 0 and s.t == 8 and s.coef == 1.0
    s = oracle.step_scalars(AdamW(max_grad_norm=0.0), True, 1e6, 0, 0)
    assert s.coef == 1.0


def test_clipped_gradient_has_norm_c():
    rng = np.random.default_rng(9)
    bits = oracle.bits16((rng.standard_normal(50_000) * 0.5).astype(np.float32), "f16")
    inv = 2.0**-4
    hp = AdamW(max_grad_norm=1.0, inv_loss_scale=inv)
    sq, ov = oracle.grad_stats(bits, "f16", inv)
    s = oracle.step_scalars(hp, True, sq, ov, 0)
    g_eff = oracle.value16(bits, "f16") * inv * s.coef
    assert abs(np.linalg.norm(g_eff) - 1.0) < 1e-7


# ----------------------------------------------------------------- AdamW
def _state(n, seed, scale=0.02, mv=True):
    rng = np.random.default_rng(seed)
    p = (rng.standard_normal(n) * scale).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32) if mv else np.zeros(n, np.float32)
    v = (rng.random(n) * 1e-6).astype(np.float32) if mv else np.zeros(n, np.float32)
    return p, m, v


def test_adamw_first_step_closed_form():
    """From m = v = 0, m_hat = g and v_hat = g^2 exactly, so
    p1 = p0 (1 - lr wd) - lr g / (|g| + eps)."""
    hp = AdamW(lr=3e-3, weight_decay=0.1, inv_loss_scale=2.0**-10)
    n = 4096
    p, m, v = _state(n, 1, mv=False)
    rng = np.random.default_rng(2)
    bits = oracle.bits16((rng.standard_normal(n) * 1e-3 * 1024).astype(np.float32), "f16")
    s = oracle.step_scalars(hp, False, 0.0, 0, 0)
    pn, mn, vn = oracle.adamw_f64(s, bits, "f16", p, m, v)
    g = oracle.value16(bits, "f16") * hp.inv_loss_scale
    a = 1 - hp.lr * hp.weight_decay
    expect = p.astype(np.float64) * a - hp.lr * g / (np.abs(g) + hp.eps)
    scale = np.abs(p) * a + hp.lr
    assert np.all(np.abs(pn - expect) <= 1e-14 * scale)
    assert np.all(np.abs(mn - (1 - hp.beta1) * g) <= 1e-16 * np.abs(g))
    assert np.all(np.abs(vn - (1 - hp.beta2) * g * g) <= 1e-15 * g * g)


@pytest.mark.parametrize("gval", [0.01, -2.5e-3, 7.0])
def test_adamw_constant_gradient_closed_form(gval):
    """Constant g: m_hat_t = g and v_hat_t = g^2 for every t, so
    p_t = a^t p0 - lr s (1 - a^t) / (1 - a), a = 1 - lr wd, s = g/(|g|+eps).
    The oracle stores fp32 between steps; the bound allows that rounding."""
    hp = AdamW(lr=1e-2, weight_decay=0.05)
    n, steps = 1000, 10
    p, m, v = _state(n, 3, mv=False)
    p0 = p.astype(np.float64).copy()
    gbits = oracle.bits16(np.full(n, gval, np.float32), "bf16")
    g = oracle.value16(gbits, "bf16")
    p16 = np.zeros(n, np.uint16)
    for t in range(steps):
        s = oracle.step_scalars(hp, False, 0.0, 0, t)
        oracle.adamw_(s, gbits, "bf16", p, m, v, p16, "bf16")
    a = 1 - hp.lr * hp.weight_decay
    sgn = g / (np.abs(g) + hp.eps)
    expect = a**steps * p0 - hp.lr * sgn * (1 - a**steps) / (1 - a)
    scale = np.abs(p0) + hp.lr * steps
    assert np.all(np.abs(p - expect) <= 2e-6 * scale)
    # m_t = (1 - b1^t) g, v_t = (1 - b2^t) g^2
    assert np.allclose(m, (1 - hp.beta1**steps) * g, rtol=2e-6, atol=0)
    assert np.allclose(v, (1 - hp.beta2**steps) * g * g, rtol=2e-6, atol=0)


def test_adamw_zero_gradient_is_pure_decay():
    hp = AdamW(lr=1e-2, weight_decay=0.3)
    p, m, v = _state(777, 4, mv=False)
    p0 = p.astype(np.float64).copy()
    zeros = np.zeros(777, np.uint16)
    p16 = np.zeros(777, np.uint16)
    for t in range(6):
        s = oracle.step_scalars(hp, False, 0.0, 0, t)
        oracle.adamw_(s, zeros, "f16", p, m, v, p16, "f16")
    assert not m.any() and not v.any()
    a = 1 - hp.lr * hp.weight_decay
    assert np.all(np.abs(p - a**6 * p0) <= 6 * 2.0**-24 * np.abs(p0))


def _torch_step(opt_cls, hp, p, m, v, t_prev, g, **kw):
    """One step of a torch.optim optimizer in fp64 from the given state."""
    x = torch.nn.Parameter(torch.from_numpy(p.astype(np.float64)))
    opt = opt_cls([x], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps,
                  weight_decay=hp.weight_decay, foreach=False, **kw)
    opt.state[x] = {"step": torch.tensor(float(t_prev), dtype=torch.float64),
                    "exp_avg": torch.from_numpy(m.astype(np.float64)),
                    "exp_avg_sq": torch.from_numpy(v.astype(np.float64))}
    x.grad = torch.from_numpy(g)
    opt.step()
    st_ = opt.state[x]
    return x.detach().numpy(), st_["exp_avg"].numpy(), st_["exp_avg_sq"].numpy()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_adamw_matches_torch_adamw(dtype):
    hp = AdamW(lr=2e-3, weight_decay=0.02, max_grad_norm=0.5, inv_loss_scale=2.0**-8)
    n = 20_000
    p, m, v = _state(n, 6)
    rng = np.random.default_rng(8)
    p16 = np.zeros(n, np.uint16)
    for t in range(5):
        bits = oracle.bits16((rng.standard_normal(n) * 3.0).astype(np.float32), dtype)
        sq, ov = oracle.grad_stats(bits, dtype, hp.inv_loss_scale)
        s = oracle.step_scalars(hp, True, sq, ov, t)
        assert s.coef < 1.0
        g_eff = oracle.value16(bits, dtype) * hp.inv_loss_scale * s.coef
        tp, tm, tv = _torch_step(torch.optim.AdamW, hp, p, m, v, t, g_eff)
        op, om, ov_ = oracle.adamw_f64(s, bits, dtype, p, m, v)
        m_scale = hp.beta1 * np.abs(m) + (1 - hp.beta1) * np.abs(g_eff)
        assert np.all(np.abs(om - tm) <= 1e-14 * m_scale)
        assert np.all(np.abs(ov_ - tv) <= 1e-14 * tv)
        upd = np.abs(tm / s.bc1) / (np.sqrt(tv / s.bc2) + hp.eps)
        p_scale = np.abs(p) + hp.lr * upd
        assert np.all(np.abs(op - tp) <= 1e-13 * p_scale)
        oracle.adamw_(s, bits, dtype, p, m, v, p16, dtype)


def test_adamw_without_decay_is_textbook_adam():
    hp = AdamW(lr=1e-3, weight_decay=0.0)
    n = 5000
    p, m, v = _state(n, 12)
    rng = np.random.default_rng(13)
    bits = oracle.bits16((rng.standard_normal(n) * 1e-2).astype(np.float32), "f16")
    s = oracle.step_scalars(hp, False, 0.0, 0, 3)
    g = oracle.value16(bits, "f16")
    tp, tm, tv = _torch_step(torch.optim.Adam, hp, p, m, v, 3, g)
    op, om, ov_ = oracle.adamw_f64(s, bits, "f16", p, m, v)
    upd = np.abs(tm / s.bc1) / (np.sqrt(tv / s.bc2) + hp.eps)
    assert np.all(np.abs(op - tp) <= 1e-13 * (np.abs(p) + hp.lr * upd))


@pytest.mark.parametrize("dtype,clip", [("f16", 0.0), ("f16", 0.005), ("bf16", 0.005)])
def test_adamw_brute_force_rational(dtype, clip):
    """64 elements x 3 steps against exact rational arithmetic."""
    hp = AdamW(lr=1e-3, weight_decay=0.01, max_grad_norm=clip, inv_loss_scale=2.0**-10)
    n = 64
    p, m, v = _state(n, 21, mv=False)
    rng = np.random.default_rng(22)
    p16 = np.zeros(n, np.uint16)
    for t in range(3):
        bits = oracle.bits16((rng.standard_normal(n) * 1.0).astype(np.float32), dtype)
        sq, ov = oracle.grad_stats(bits, dtype, hp.inv_loss_scale)
        exact_sq = brute.sq_norm(bits, dtype, hp.inv_loss_scale)
        assert abs(Fraction(sq) - exact_sq) <= exact_sq * Fraction(1, 10**15)
        s = oracle.step_scalars(hp, True, sq, ov, t)
        if clip:
            assert s.coef < 1.0
        P, M, V = brute.adamw(hp, exact_sq, t + 1, bits, dtype, p, m, v)
        op, om, ov_ = oracle.adamw_f64(s, bits, dtype, p, m, v)
        graw = brute.decode16(bits, dtype)
        for i in range(n):
            # m' = b1 m + (1 - b1) g may cancel: bound by the size of its terms
            m_scale = Fraction(hp.beta1) * abs(Fraction(float(m[i]))) + \
                (1 - Fraction(hp.beta1)) * abs(Fraction(graw[i]) * Fraction(hp.inv_loss_scale))
            assert abs(Fraction(om[i]) - M[i]) <= Fraction(1, 10**14) * m_scale
            assert abs(Fraction(ov_[i]) - V[i]) <= Fraction(1, 10**14) * V[i]
            assert abs(Fraction(op[i]) - P[i]) <= Fraction(1, 10**13) * (abs(P[i]) + Fraction(hp.lr))
        oracle.adamw_(s, bits, dtype, p, m, v, p16, dtype)
        # stored fp32 values are the rounding of the exact values (or one ulp off at a tie)
        for arr, ex in ((p, P), (m, M), (v, V)):
            exf = np.float32([float(e) for e in ex])
            ulps = np.abs(arr.view(np.int32).astype(np.int64) - exf.view(np.int32).astype(np.int64))
            assert ulps.max() <= 1


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_adamw_param_is_rounded_master(dtype):
    hp = AdamW()
    n = 50_000
    p, m, v = _state(n, 30, scale=3.0)
    bits = oracle.bits16(np.random.default_rng(31).standard_normal(n).astype(np.float32), dtype)
    p16 = np.zeros(n, np.uint16)
    s = oracle.step_scalars(hp, False, 0.0, 0, 0)
    oracle.adamw_(s, bits, dtype, p, m, v, p16, dtype)
    if dtype == "f16":
        ref = p.astype(np.float16).view(np.uint16)
    else:
        ref = torch.from_numpy(p).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(p16, ref)


def test_adamw_sharding_invariance():
    """Same update whether the flat vector is updated whole or as Nd
    contiguous shards that share the global norm: sharding changes where
    the state lives, not the math."""
    hp = AdamW(max_grad_norm=1.0, inv_loss_scale=2.0**-16)
    n = 30_011
    rng = np.random.default_rng(40)
    bits = oracle.bits16((rng.standard_normal(n) * 1e-3 * 65536).astype(np.float32), "f16")
    p, m, v = _state(n, 41)
    sq, ov = oracle.grad_stats(bits, "f16", hp.inv_loss_scale)
    s = oracle.step_scalars(hp, True, sq, ov, 2)
    whole = [a.copy() for a in (p, m, v)]
    p16w = np.zeros(n, np.uint16)
    oracle.adamw_(s, bits, "f16", *whole, p16w, "f16")
    for nd in (2, 5, 8):
        parts = [a.copy() for a in (p, m, v)]
        p16 = np.zeros(n, np.uint16)
        shard_sq = []
        for r in range(nd):
            b, e = oracle.partition(n, nd, r)
            shard_sq.append(oracle.grad_stats(bits[b:e], "f16", hp.inv_loss_scale)[0])
        assert abs(math.fsum(shard_sq) - sq) <= 1e-14 * sq
        for r in range(nd):
            b, e = oracle.partition(n, nd, r)
            sl = [np.ascontiguousarray(a[b:e]) for a in parts]
            pp = np.zeros(e - b, np.uint16)
            oracle.adamw_(s, np.ascontiguousarray(bits[b:e]), "f16", *sl, pp, "f16")
            for a, x in zip(parts, sl):
                a[b:e] = x
            p16[b:e] = pp
        for a, w in zip(parts, whole):
            assert np.array_equal(a, w)
        assert np.array_equal(p16, p16w)


def test_adamw_skip_leaves_everything_untouched():
    hp = AdamW(max_grad_norm=1.0)
    n = 1000
    p, m, v = _state(n, 50)
    bits = oracle.bits16(np.random.default_rng(51).standard_normal(n).astype(np.float32), "f16")
    bits[123] = 0x7C00
    sq, ov = oracle.grad_stats(bits, "f16", 1.0)
    assert ov == 1
    s = oracle.step_scalars(hp, True, sq, ov, 9)
    assert s.skip == 1 and s.t == 9
    before = [a.copy() for a in (p, m, v)]
    p16 = np.full(n, 0xABCD, np.uint16)
    oracle.adamw_(s, bits, "f16", p, m, v, p16, "f16")
    for a, b in zip((p, m, v), before):
        assert np.array_equal(a, b)
    assert (p16 == 0xABCD).all()


# ------------------------------------------------------ dynamic loss scaling
def _scaler(init=1024.0, growth=2.0, backoff=0.5, interval=3, lo=2.0 ** -100,
            hi=float("inf")):
    return oracle.Scaler(init, growth, backoff, interval, lo, hi)


@pytest.mark.parametrize("interval", [1, 2, 3, 7])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_loss_scale_matches_torch_amp_update(interval, seed):
    """Library pin: torch's own loss-scale update (CPU, fp32 scale), which
    halves the scale on an overflow and doubles it after `interval` steps
    without one; with power-of-two factors both are exact."""
    rng = np.random.default_rng(seed)
    flags = (rng.random(60) < 0.2).astype(int).tolist()
    got = oracle.loss_scale_sequence(_scaler(interval=interval), flags)
    scale = torch.tensor([1024.0])
    tracker = torch.tensor([0], dtype=torch.int32)
    found = torch.tensor([0.0])
    for k, ov in enumerate(flags):
        found.fill_(float(ov))
        torch._amp_update_scale_(scale, tracker, found, 2.0, 0.5, interval)
        assert got[k][0] == scale.item(), (k, got[k], scale.item())
        assert got[k][2] == tracker.item(), (k, got[k], tracker.item())
        assert got[k][1] == 1.0 / got[k][0]
    assert got[-1][3] == sum(flags)


def test_loss_scale_closed_forms():
    # k overflows in a row: S0 * b^k, floored at min_scale
    got = oracle.loss_scale_sequence(_scaler(init=2.0 ** 16, lo=2.0 ** 10), [1] * 9)
    assert [g[0] for g in got] == [2.0 ** max(16 - k, 10) for k in range(1, 10)]
    assert [g[3] for g in got] == list(range(1, 10)) and all(g[2] == 0 for g in got)
    # N good steps: S0 * g^floor(N / I), capped at max_scale; good = N mod I
    got = oracle.loss_scale_sequence(_scaler(init=8.0, interval=4, hi=2.0 ** 6), [0] * 30)
    for n, g in enumerate(got, start=1):
        assert g[0] == min(8.0 * 2.0 ** (n // 4), 2.0 ** 6), (n, g)
        assert g[2] == n % 4 and g[3] == 0
    # a non-power-of-two rule, by hand: 1000 -> (x0.25) 250 -> 3 good (x3) 750
    c = _scaler(init=1000.0, growth=3.0, backoff=0.25, interval=3, lo=1.0)
    got = oracle.loss_scale_sequence(c, [1, 0, 0, 0, 1, 1, 1, 1, 1])
    assert [g[0] for g in got] == [250.0, 250.0, 250.0, 750.0, 187.5, 46.875, 11.71875,
                                   2.9296875, 1.0]
    # growth that would overflow leaves the scale unchanged but restarts the count
    big = 2.0 ** 1023
    got = oracle.loss_scale_sequence(_scaler(init=big, interval=1), [0, 0])
    assert got == [(big, 1.0 / big, 0, 0)] * 2
