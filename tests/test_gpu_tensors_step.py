"""The step read from the per-tensor gradients in place (no gathered shard):
zero_grad_stats_tensors, then zero_adam_step_tensors ("ZeRO: Memory
Optimizations Toward Training Trillion Parameter Models", paper summary page,
section ZeRO-R > CB; ZeRO-DP Stage 1).  Checks:
  - the statistics equal, bit for bit, those of the fused gather
    (zero_bucket_flatten_stats into an aligned buffer) over the same range;
  - every output of the step (master, m, v, param shard, step state) equals,
    bit for bit, the step on the gathered shard, at every 16-bit param phase
    and fp32 phase, for all dtype pairs;
  - workloads 1 and 5 against the oracle on every element (one-step and
    free-running, the injected overflow step skipped), workload 2 on the
    whole shard against the gathered path and on a sample against the
    oracle."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_grads_amd as z
from synth import AdamW, WORKLOADS, gen
from test_gpu_configs import NP16, Rank, _dev16, _free, _sample_indices, _to_host16
from util import FreeRunScales, check_adam_one_step, check_params16, dev, progress

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _release_memory():
    yield
    _free()


def _host_list(numels, dtype, seed, scale):
    rng = np.random.default_rng(seed)
    return [gen.f32_to_bits16((rng.standard_normal(k) * 1e-3 * scale).astype(np.float32), dtype)
            for k in numels]


def _dev_list(host):
    return [torch.from_numpy(h.view(np.int16)).to(dev()) for h in host]


# --------------------------------------------------------------- statistics
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("case", ["tiny_r0", "tiny_r1", "tiny_r3", "ragged", "nan"])
def test_tensor_stats_equal_fused_gather(dtype, case):
    if case.startswith("tiny"):
        cfg = WORKLOADS[1]
        numels = cfg.numels
        lo, hi = oracle.partition(cfg.psi, 4, int(case[-1]))
    else:
        numels = [1, 7, 8, 9, 1000, 4097, 33_333, 3, 100_000]
        lo, hi = 5, sum(numels) - 2
    host = _host_list(numels, dtype, 7, 1024.0)
    if case == "nan":
        host[5][11] = gen.specials(dtype)[2]
    ts = _dev_list(host)
    n = hi - lo
    nb = z.zero_bucket_flatten_stats_workspace(numels, lo, n)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev())
    st_t, st_f = z.new_grad_stats(dev()), z.new_grad_stats(dev())
    z.zero_grad_stats_tensors(ts, numels, dtype, lo, n, 1.0 / 1024, ws, nb, st_t)
    dst = torch.empty(n + 8, dtype=torch.int16, device=dev())
    assert dst.data_ptr() % 16 == 0
    z.zero_bucket_flatten_stats(ts, numels, dtype, lo, n, dst, 1.0 / 1024, ws, nb, st_f)
    torch.cuda.synchronize()
    a, b = z.read_grad_stats(st_t), z.read_grad_stats(st_f)
    assert a.overflow == b.overflow == (case == "nan")
    if not a.overflow:
        assert a.sq_norm == b.sq_norm
        sq, ov = oracle.grad_stats(oracle.flatten(host, lo, hi), dtype, 1.0 / 1024)
        assert ov == 0 and abs(a.sq_norm - sq) <= 1e-12 * sq


def test_tensor_stats_empty_range():
    ts = _dev_list(_host_list([10, 20], "f16", 1, 1.0))
    nb = z.zero_bucket_flatten_stats_workspace([10, 20], 30, 0)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev())
    st = z.new_grad_stats(dev())
    st.fill_(0x7F)
    z.zero_grad_stats_tensors(ts, [10, 20], "f16", 30, 0, 1.0, ws, nb, st)
    r = z.read_grad_stats(st)
    assert r.sq_norm == 0.0 and r.overflow == 0


# ------------------------------------------------- step: bitwise vs gathered
def _state(n, f_phase, p_phase, seed, pdt):
    rng = np.random.default_rng(seed)
    raw = [torch.from_numpy(np.zeros(n + 8, np.float32)).to(dev()) for _ in range(3)]
    th, m, v = (r[f_phase:f_phase + n] for r in raw)
    th.copy_(torch.from_numpy((rng.standard_normal(n) * 0.02).astype(np.float32)))
    m.copy_(torch.from_numpy((rng.standard_normal(n) * 1e-4).astype(np.float32)))
    v.copy_(torch.from_numpy((rng.random(n) * 1e-8).astype(np.float32)))
    p_raw = torch.full((n + 8,), 0x5A5A, dtype=torch.int16, device=dev())
    return raw, (th, m, v), p_raw, p_raw[p_phase:p_phase + n]


@pytest.mark.parametrize("gdt,pdt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "bf16")])
@pytest.mark.parametrize("f_phase", [0, 1, 3])
@pytest.mark.parametrize("p_phase", range(8))
def test_tensor_step_equals_gathered_step(gdt, pdt, f_phase, p_phase):
    numels = [1, 7, 8, 9, 1000, 4097, 33_333, 3, 100_000, 2]
    lo, hi = 5, sum(numels) - 2
    n = hi - lo
    hp = AdamW(max_grad_norm=0.5, inv_loss_scale=1.0 / 1024)
    ahp = z.adamw(**hp.__dict__)
    seed = 100 * f_phase + 10 * p_phase + len(gdt + pdt)
    a_raw, (a_th, a_m, a_v), a_praw, a_p = _state(n, f_phase, p_phase, seed, pdt)
    b_raw, (b_th, b_m, b_v), b_praw, b_p = _state(n, f_phase, p_phase, seed, pdt)
    a_st, b_st = z.new_adam_state(dev()), z.new_adam_state(dev())
    a_gs, b_gs = z.new_grad_stats(dev()), z.new_grad_stats(dev())
    nb = z.zero_bucket_flatten_stats_workspace(numels, lo, n)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev())
    # the gathered shard, 16-byte aligned: its statistics then sum the same
    # tiles in the same order as the in-place statistics
    g = torch.empty(n, dtype=torch.int16, device=dev())
    for k in range(3):
        ts = _dev_list(_host_list(numels, gdt, seed + k, 1024.0))
        z.zero_grad_stats_tensors(ts, numels, gdt, lo, n, hp.inv_loss_scale, ws, nb, a_gs)
        z.zero_adam_step_tensors(ahp, ts, numels, gdt, lo, n, a_th, a_m, a_v, a_p, pdt, a_gs, a_st)
        z.zero_bucket_flatten_stats(ts, numels, gdt, lo, n, g, hp.inv_loss_scale, ws, nb, b_gs)
        z.zero_adam_step(ahp, g, gdt, b_th, b_m, b_v, b_p, pdt, n, b_gs, b_st)
        torch.cuda.synchronize()
        sa, sb = z.read_grad_stats(a_gs), z.read_grad_stats(b_gs)
        assert sa.overflow == sb.overflow == 0 and sa.sq_norm == sb.sq_norm
        for x, y in zip(a_raw + [a_praw], b_raw + [b_praw]):  # guard bands included
            assert torch.equal(x.view(torch.int32 if x.dtype == torch.float32 else torch.int16),
                               y.view(torch.int32 if y.dtype == torch.float32 else torch.int16)), k
        assert torch.equal(a_st, b_st)
    assert int((a_praw[:p_phase] == 0x5A5A).sum()) == p_phase
    assert bool((a_praw[p_phase + n:] == 0x5A5A).all())


def test_tensor_step_rejects_split_fp32_phases_and_overlap():
    numels = [1000, 200]
    ts = _dev_list(_host_list(numels, "f16", 1, 1.0))
    st = z.new_adam_state(dev())
    buf = torch.zeros(4 * 400, dtype=torch.float32, device=dev())
    th, m, v = buf[0:300], buf[400:700], buf[801:1101]
    p = torch.zeros(300, dtype=torch.int16, device=dev())
    with pytest.raises(z.ZeroError) as e:  # v at another position within 16 bytes
        z.zero_adam_step_tensors(z.adamw(), ts, numels, "f16", 0, 300, th, m, v, p, "f16", None,
                                 st)
    assert e.value.status == z.ZERO_EALIGN
    with pytest.raises(z.ZeroError) as e:  # param_out over gradients the step reads
        z.zero_adam_step_tensors(z.adamw(), ts, numels, "f16", 0, 300, th, m, buf[1200:1500],
                                 ts[0][100:400], "f16", None, st)
    assert e.value.status == z.ZERO_EINVAL and "param_out overlaps tensor 0" in str(e.value)
    assert z.read_adam_state(st).step == 0  # nothing ran


@pytest.mark.parametrize("case", ["empty_tensors", "short", "empty_range", "one_tensor_middle"])
def test_tensor_step_edge_ranges(case):
    """Zero-size tensors in the list, ranges shorter than a chunk, an empty
    range (the step counter still advances), and a range inside one tensor:
    equal to the step on the gathered shard, bit for bit."""
    numels = {"empty_tensors": [0, 1000, 0, 0, 37, 0, 5000],
              "short": [3, 2, 4, 1],
              "empty_range": [100, 200],
              "one_tensor_middle": [50, 100_000, 70]}[case]
    lo, hi = {"empty_tensors": (1, 6036), "short": (1, 7), "empty_range": (150, 150),
              "one_tensor_middle": (1001, 60_003)}[case]
    n = hi - lo
    hp = AdamW(max_grad_norm=0.5, inv_loss_scale=1.0 / 1024)
    ahp = z.adamw(**hp.__dict__)
    host = _host_list(numels, "bf16", 5, 1024.0)
    ts = [torch.from_numpy(h.view(np.int16)).to(dev()) if h.size else None for h in host]
    a_raw, (a_th, a_m, a_v), a_praw, a_p = _state(max(n, 1), 1, 5, 7, "bf16")
    b_raw, (b_th, b_m, b_v), b_praw, b_p = _state(max(n, 1), 1, 5, 7, "bf16")
    a_st, b_st = z.new_adam_state(dev()), z.new_adam_state(dev())
    a_gs, b_gs = z.new_grad_stats(dev()), z.new_grad_stats(dev())
    nb = z.zero_bucket_flatten_stats_workspace(numels, lo, n)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev())
    g = torch.empty(max(n, 1), dtype=torch.int16, device=dev())
    z.zero_grad_stats_tensors(ts, numels, "bf16", lo, n, hp.inv_loss_scale, ws, nb, a_gs)
    z.zero_adam_step_tensors(ahp, ts, numels, "bf16", lo, n, a_th, a_m, a_v, a_p, "bf16", a_gs,
                             a_st)
    z.zero_bucket_flatten_stats(ts, numels, "bf16", lo, n, g, hp.inv_loss_scale, ws, nb, b_gs)
    z.zero_adam_step(ahp, g, "bf16", b_th, b_m, b_v, b_p, "bf16", n, b_gs, b_st)
    torch.cuda.synchronize()
    sa, sb = z.read_grad_stats(a_gs), z.read_grad_stats(b_gs)
    assert sa.overflow == sb.overflow == 0 and sa.sq_norm == sb.sq_norm
    if n == 0:
        assert sa.sq_norm == 0.0
    for x, y in zip(a_raw + [a_praw], b_raw + [b_praw]):
        assert torch.equal(x.view(torch.int32 if x.dtype == torch.float32 else torch.int16),
                           y.view(torch.int32 if y.dtype == torch.float32 else torch.int16))
    assert torch.equal(a_st, b_st) and z.read_adam_state(a_st).step == 1


# --------------------------------------------------- workloads vs the oracle
def _step_both(rt, rg, grads):
    rt.tensors_step(grads)
    rg.gather_with_stats(grads)
    rg.stats_and_step(fused=True)
    torch.cuda.synchronize()
    a, b = z.read_grad_stats(rt.stats), z.read_grad_stats(rg.stats)
    assert a.overflow == b.overflow
    if not a.overflow:
        assert a.sq_norm == b.sq_norm  # the same tiles, the same order
    for x, y in ((rt.master, rg.master), (rt.m, rg.m), (rt.v, rg.v)):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    assert torch.equal(rt.p_raw.view(torch.int16), rg.p_raw.view(torch.int16))
    assert torch.equal(rt.state, rg.state)
    return a


def test_workload1_tensors_full():
    cfg = WORKLOADS[1]
    rt, rg = Rank(cfg), Rank(cfg)
    n, b, e = rt.n, rt.begin, rt.end
    masters = gen.host_master_list(cfg)
    th_o = oracle.flatten(masters, b, e).copy()
    for r in (rt, rg):
        r.master.copy_(torch.from_numpy(th_o))
    m_o, v_o, p_o = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, NP16)
    scales = FreeRunScales(cfg.hp, th_o)
    for k in range(cfg.steps):
        host = gen.host_grad_list(cfg, k)
        grads = {i: torch.from_numpy(h.view(np.int16)).to(dev()) for i, h in enumerate(host)}
        th0, m0, v0 = (a.cpu().numpy().copy() for a in (rt.master, rt.m, rt.v))
        st = _step_both(rt, rg, grads)
        g_ref = oracle.flatten(host, b, e)
        sq, ov = oracle.grad_stats(g_ref, cfg.dtype, cfg.hp.inv_loss_scale)
        assert st.overflow == ov == 0 and abs(st.sq_norm - sq) <= 1e-5 * sq
        s1 = oracle.step_scalars(cfg.hp, True, st.sq_norm, st.overflow, k)
        th1, m1, v1, p1 = th0.copy(), m0.copy(), v0.copy(), np.zeros(n, NP16)
        oracle.adamw_(s1, g_ref, cfg.dtype, th1, m1, v1, p1, cfg.dtype)
        th_g, m_g, v_g = (a.cpu().numpy() for a in (rt.master, rt.m, rt.v))
        p_g = _to_host16(rt.p)
        gv = oracle.value16(g_ref, cfg.dtype)
        e1 = check_adam_one_step(cfg.hp, s1, gv, th0, m0, v0, th_g, m_g, v_g, th1, m1, v1,
                                 label=f"step {k}")
        d1 = check_params16(p_g, th_g, th1, cfg.dtype, f"step {k}")
        s = oracle.step_scalars(cfg.hp, True, sq, ov, k)
        oracle.adamw_(s, g_ref, cfg.dtype, th_o, m_o, v_o, p_o, cfg.dtype)
        scales.update(s, gv, m_o, v_o)
        e2 = scales.check(th_g, m_g, v_g, th_o, m_o, v_o, label=f"step {k}")
        d2 = check_params16(p_g, th_g, th_o, cfg.dtype, f"step {k}")
        progress(f"workload 1 tensors step {k}: one-step {e1} params differ {d1}; "
                 f"free {e2} params differ {d2} (of {n})")
    assert z.read_adam_state(rt.state).step == cfg.steps


@pytest.mark.timeout(900)
def test_workload5_tensors_skip_full():
    cfg = WORKLOADS[5]
    ph = oracle.partition(cfg.psi, cfg.nd, cfg.rank)[0] % 8
    rt, rg = Rank(cfg, p_phase=ph), Rank(cfg, p_phase=ph)
    n, b = rt.n, rt.begin
    assert ph == 1 and len(rt.tensor_ids) == 4
    gen.device_fill_normal_(rt.master, cfg.master_seed(), cfg.master_sigma)
    rg.master.copy_(rt.master)
    th_o = rt.master.cpu().numpy().copy()
    m_o, v_o, p_o = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, NP16)
    scales = FreeRunScales(cfg.hp, th_o)
    inj_step, inj = gen.inject_plan(cfg, n)
    offs = np.cumsum([0] + cfg.numels)
    lo_t = int(offs[rt.tensor_ids[0]])
    t_expect = 0
    for k in range(cfg.steps):
        grads = gen.device_grad_list(cfg, k, dev(), which=rt.tensor_ids)
        if k == inj_step:
            for i, bits in inj:
                ti = int(np.searchsorted(offs, b + i, side="right") - 1)
                o = b + i - int(offs[ti])
                grads[ti][o:o + 1] = _dev16(bits, grads[ti])
        th0, m0, v0 = (a.cpu().numpy().copy() for a in (rt.master, rt.m, rt.v))
        p_before = _to_host16(rt.p).copy()
        st = _step_both(rt, rg, grads)
        g_ref = oracle.flatten([_to_host16(grads[i]) for i in rt.tensor_ids], b - lo_t,
                               rt.end - lo_t)
        sq, ov = oracle.grad_stats(g_ref, cfg.dtype, cfg.hp.inv_loss_scale)
        assert st.overflow == ov
        state = z.read_adam_state(rt.state)
        th_g, m_g, v_g = (a.cpu().numpy() for a in (rt.master, rt.m, rt.v))
        p_g = _to_host16(rt.p)
        if ov:
            assert k == inj_step and state.skip == 1 and state.step == t_expect
            for a, a0 in ((th_g, th0), (m_g, m0), (v_g, v0), (p_g, p_before)):
                assert np.array_equal(a.view(np.uint8), a0.view(np.uint8))
            progress(f"workload 5 tensors step {k}: overflow -> skipped")
            continue
        t_expect += 1
        assert state.step == t_expect and abs(st.sq_norm - sq) <= 1e-5 * sq
        gv = oracle.value16(g_ref, cfg.dtype)
        s1 = oracle.step_scalars(cfg.hp, True, st.sq_norm, st.overflow, t_expect - 1)
        assert s1.coef < 1.0
        th1, m1, v1, p1 = th0.copy(), m0.copy(), v0.copy(), np.zeros(n, NP16)
        oracle.adamw_(s1, g_ref, cfg.dtype, th1, m1, v1, p1, cfg.dtype)
        e1 = check_adam_one_step(cfg.hp, s1, gv, th0, m0, v0, th_g, m_g, v_g, th1, m1, v1,
                                 label=f"step {k}")
        d1 = check_params16(p_g, th_g, th1, cfg.dtype, f"step {k}")
        del th1, m1, v1, p1
        s = oracle.step_scalars(cfg.hp, True, sq, ov, t_expect - 1)
        oracle.adamw_(s, g_ref, cfg.dtype, th_o, m_o, v_o, p_o, cfg.dtype)
        scales.update(s, gv, m_o, v_o)
        e2 = scales.check(th_g, m_g, v_g, th_o, m_o, v_o, label=f"step {k}")
        d2 = check_params16(p_g, th_g, th_o, cfg.dtype, f"step {k}")
        progress(f"workload 5 tensors step {k}: one-step {e1} params differ {d1}; "
                 f"free {e2} params differ {d2} (of {n})")
    assert t_expect == cfg.steps - 1
    assert int(rt.p_raw[0].view(torch.int16).item()) == 0  # the lead pad was never written


@pytest.mark.timeout(900)
def test_workload2_tensors_whole_shard_and_sample():
    cfg = WORKLOADS[2]
    rt, rg = Rank(cfg), Rank(cfg)
    n = rt.n
    gen.device_fill_normal_(rt.master, cfg.master_seed(), cfg.master_sigma)
    rg.master.copy_(rt.master)
    idx = _sample_indices(cfg, rt.begin, rt.end, 1 << 20, 77)
    idx_t = torch.from_numpy(idx).to(dev())
    for k in range(3):
        grads = gen.device_grad_list(cfg, k, dev())
        th0, m0, v0 = (a[idx_t].cpu().numpy() for a in (rt.master, rt.m, rt.v))
        st = _step_both(rt, rg, grads)  # whole shard, bit for bit
        # the sample against the oracle (one step from the GPU's state and norm)
        starts = np.cumsum([0] + cfg.numels)
        k_t = np.searchsorted(starts, idx, side="right") - 1
        g_s = np.empty(idx.size, NP16)
        for ti in np.unique(k_t):
            sel = np.nonzero(k_t == ti)[0]
            g_s[sel] = _to_host16(grads[int(ti)][torch.from_numpy(idx[sel] - starts[ti]).to(dev())])
        s1 = oracle.step_scalars(cfg.hp, True, st.sq_norm, st.overflow, k)
        th1, m1, v1, p1 = th0.copy(), m0.copy(), v0.copy(), np.zeros(idx.size, NP16)
        oracle.adamw_(s1, g_s, cfg.dtype, th1, m1, v1, p1, cfg.dtype)
        th_g, m_g, v_g = (a[idx_t].cpu().numpy() for a in (rt.master, rt.m, rt.v))
        e1 = check_adam_one_step(cfg.hp, s1, oracle.value16(g_s, cfg.dtype), th0, m0, v0, th_g,
                                 m_g, v_g, th1, m1, v1, label=f"step {k}")
        d1 = check_params16(_to_host16(rt.p[idx_t]), th_g, th1, cfg.dtype, f"step {k}")
        progress(f"workload 2 tensors step {k}: whole shard equal to the gathered path; "
                 f"sample of {idx.size}: {e1} params differ {d1}")
        del grads
