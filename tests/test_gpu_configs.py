"""Parity on the five synthetic workloads, at their full sizes, through the
C ABI, in the launch configuration that bench.py times.

Each step runs the whole hot path on the device: the rank's part of every
fused bucket is gathered from the per-tensor gradients (zero_bucket_flatten),
then zero_grad_stats and zero_adam_step.  Checks per step:
  - the gathered gradient shard is bit-exact (full or sampled);
  - overflow flag bit-exact, squared norm within 1e-5 of the oracle's own
    fp64 norm over every gradient of the shard;
  - one-step mode: the oracle restarts from the GPU's state and uses the GPU's
    norm; master/m/v within 1e-6 of the size of the update's terms, params
    within 1 ulp;
  - free-running: the oracle's own trajectory (its own norm), master/m/v
    within 1e-5 of the shadow-recursion scales, params within 1 ulp.
Workloads 1 and 5 are verified on every element; 2, 3 and 4 on a seeded sample
(every tensor and bucket boundary +-64, the shard's head and tail, and
random positions), which is exact because the update is elementwise once the
step scalars are fixed.
"""
import gc
import math

import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_grads_amd as z
from synth import WORKLOADS, gen
from util import FreeRunScales, check_adam_one_step, check_params16, dev, progress

pytestmark = pytest.mark.gpu

NP16 = np.uint16


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _to_host16(t):
    return t.view(torch.int16).cpu().numpy().view(NP16)


def _dev16(bits, like):
    """A one-element device tensor holding the 16-bit pattern `bits`."""
    return torch.from_numpy(np.array([bits], NP16).view(np.int16)).view(like.dtype).to(dev())


def _sample_indices(cfg, begin, end, n_random, seed, bucket=None):
    n = end - begin
    pts = [np.arange(0, min(64, n)), np.arange(max(0, n - 64), n)]
    offs = np.cumsum([0] + cfg.numels)
    cuts = [int(o) for o in offs if begin < o < end]
    if bucket:
        cuts += list(range((begin // bucket + 1) * bucket, end, bucket))
    for c in cuts:
        lo = c - begin
        pts.append(np.arange(max(0, lo - 64), min(n, lo + 64)))
    pts.append(np.random.default_rng(seed).integers(0, n, n_random))
    return np.unique(np.concatenate(pts)).astype(np.int64)


class Rank:
    """Device state of one rank's shard plus the calls of one step."""

    def __init__(self, cfg, p_phase=0, grads_list=True, spread=False):
        """spread: the five state arrays are placed in one pool exactly as the
        benchmark places them (zero_state_layout); otherwise separate tensors."""
        self.cfg = cfg
        self.begin, self.end = z.zero_partition(cfg.psi, cfg.nd, cfg.rank)
        assert (self.begin, self.end) == oracle.partition(cfg.psi, cfg.nd, cfg.rank)
        n = self.n = self.end - self.begin
        d = dev()
        tdt = gen.torch_dtype(cfg.dtype)
        if spread:
            import bench
            g, master, m, v, self.p_raw, self.layout = bench.state_arrays(n + 8, tdt, d)
            assert self.layout["kind"] == "spread", self.layout
            self.g, self.master, self.m, self.v = g[:n], master[:n], m[:n], v[:n]
            self.m.zero_()
            self.v.zero_()
            self.p_raw.zero_()
        else:
            self.g = torch.empty(n, dtype=tdt, device=d)
            self.master = torch.empty(n, dtype=torch.float32, device=d)
            self.m = torch.zeros(n, dtype=torch.float32, device=d)
            self.v = torch.zeros(n, dtype=torch.float32, device=d)
            self.p_raw = torch.zeros(n + 8, dtype=tdt, device=d)
        # the 16-bit param shard keeps the phase it has in the full flat buffer
        self.p = self.p_raw[p_phase:p_phase + n]
        self.stats = z.new_grad_stats(d)
        self.state = z.new_adam_state(d)
        self.ws = z.new_workspace(n, d)
        self.hp = z.adamw(**cfg.hp.__dict__)
        plan = oracle.bucket_plan(cfg.numels, cfg.psi, self.begin, self.end)
        self.tensor_ids = sorted({s.tensor for s in plan})

    def gather(self, grads):
        """The rank's part of every fused bucket, into the grad shard."""
        cfg = self.cfg
        B = cfg.bucket_elems or cfg.psi
        ptrs = [grads[i].data_ptr() if i in grads else None for i in range(len(cfg.numels))]
        lo = self.begin
        while lo < self.end:
            hi = min((lo // B + 1) * B, self.end)
            z.zero_bucket_flatten(ptrs, cfg.numels, cfg.dtype, lo, hi - lo,
                                  self.g.data_ptr() + 2 * (lo - self.begin))
            lo = hi

    def gather_with_stats(self, grads):
        """The whole shard gathered in one pass that also writes the
        statistics (the path of a rank whose per-tensor gradients are final)."""
        cfg = self.cfg
        ptrs = [grads[i].data_ptr() if i in grads else None for i in range(len(cfg.numels))]
        nb = z.zero_bucket_flatten_stats_workspace(cfg.numels, self.begin, self.n)
        self.fws = torch.empty(nb, dtype=torch.uint8, device=dev())
        z.zero_bucket_flatten_stats(ptrs, cfg.numels, cfg.dtype, self.begin, self.n, self.g,
                                    cfg.hp.inv_loss_scale, self.fws, nb, self.stats)

    def tensors_step(self, grads):
        """The step read from the per-tensor gradients in place: statistics,
        then AdamW, with no gathered shard (30 bytes per parameter)."""
        cfg = self.cfg
        ptrs = [grads[i].data_ptr() if i in grads else None for i in range(len(cfg.numels))]
        nb = z.zero_bucket_flatten_stats_workspace(cfg.numels, self.begin, self.n)
        self.fws = torch.empty(nb, dtype=torch.uint8, device=dev())
        z.zero_grad_stats_tensors(ptrs, cfg.numels, cfg.dtype, self.begin, self.n,
                                  cfg.hp.inv_loss_scale, self.fws, nb, self.stats)
        z.zero_adam_step_tensors(self.hp, ptrs, cfg.numels, cfg.dtype, self.begin, self.n,
                                 self.master, self.m, self.v, self.p, cfg.dtype, self.stats,
                                 self.state)

    def stats_and_step(self, fused=False):
        cfg = self.cfg
        if not fused:
            z.zero_grad_stats(self.g, cfg.dtype, self.n, cfg.hp.inv_loss_scale, self.ws,
                              self.ws.numel(), self.stats)
        z.zero_adam_step(self.hp, self.g, cfg.dtype, self.master, self.m, self.v, self.p,
                         cfg.dtype, self.n, self.stats, self.state)


def _oracle_norm_streamed(g_dev, dtype, inv, chunk=1 << 29):
    """The oracle's norm over every gradient, streamed to the host in chunks
    (partial sums combined exactly with math.fsum)."""
    parts, ov = [], 0
    for lo in range(0, g_dev.numel(), chunk):
        h = _to_host16(g_dev[lo:lo + chunk])
        sq, o = oracle.grad_stats(h, dtype, inv)
        parts.append(sq)
        ov |= o
    return math.fsum(parts), ov


# ------------------------------------------------------------ workload 1
@pytest.mark.parametrize("fused", [False, True])
def test_workload1_tiny_full(fused):
    cfg = WORKLOADS[1]
    r = Rank(cfg)
    n, b, e = r.n, r.begin, r.end
    assert (b, e, n) == (0, 262_144, 262_144)
    # master initialised from the fp32 parameter list (fp32 gather)
    masters = gen.host_master_list(cfg)
    src = [torch.from_numpy(a).to(dev()) for a in masters]
    z.zero_bucket_flatten(src, None, "f32", b, n, r.master)
    th_o = oracle.flatten(masters, b, e).copy()
    assert np.array_equal(r.master.cpu().numpy().view(np.uint32), th_o.view(np.uint32))
    m_o, v_o, p_o = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, NP16)
    scales = FreeRunScales(cfg.hp, th_o)
    worst, worst1, norm_rel, far = {}, {}, 0.0, [0, 0]
    for k in range(cfg.steps):
        host = gen.host_grad_list(cfg, k)
        grads = {i: torch.from_numpy(h.view(np.int16)).to(dev()) for i, h in enumerate(host)}
        if fused:
            r.gather_with_stats(grads)
        else:
            r.gather(grads)
        g_ref = oracle.flatten(host, b, e)
        assert np.array_equal(_to_host16(r.g), g_ref), k
        th0, m0, v0 = (a.cpu().numpy().copy() for a in (r.master, r.m, r.v))
        r.stats_and_step(fused)
        torch.cuda.synchronize()
        st = z.read_grad_stats(r.stats)
        sq, ov = oracle.grad_stats(g_ref, cfg.dtype, cfg.hp.inv_loss_scale)
        assert st.overflow == ov == 0 and abs(st.sq_norm - sq) <= 1e-5 * sq
        norm_rel = max(norm_rel, abs(st.sq_norm - sq) / sq)
        gv = oracle.value16(g_ref, cfg.dtype)
        # one-step mode
        s1 = oracle.step_scalars(cfg.hp, True, st.sq_norm, st.overflow, k)
        th1, m1, v1, p1 = th0.copy(), m0.copy(), v0.copy(), np.zeros(n, NP16)
        oracle.adamw_(s1, g_ref, cfg.dtype, th1, m1, v1, p1, cfg.dtype)
        th_g, m_g, v_g = (a.cpu().numpy() for a in (r.master, r.m, r.v))
        p_g = _to_host16(r.p)
        e1 = check_adam_one_step(cfg.hp, s1, gv, th0, m0, v0, th_g, m_g, v_g, th1, m1, v1,
                                 label=f"step {k}")
        far[0] = max(far[0], check_params16(p_g, th_g, th1,
                                            cfg.dtype, f"step {k}"))
        worst1 = {key: max(worst1.get(key, 0), val) for key, val in e1.items()}
        # free-running
        s = oracle.step_scalars(cfg.hp, True, sq, ov, k)
        oracle.adamw_(s, g_ref, cfg.dtype, th_o, m_o, v_o, p_o, cfg.dtype)
        scales.update(s, gv, m_o, v_o)
        errs = scales.check(th_g, m_g, v_g, th_o, m_o, v_o, label=f"step {k}")
        far[1] = max(far[1], check_params16(p_g, th_g, th_o,
                                            cfg.dtype, f"step {k}"))
        worst = {key: max(worst.get(key, 0), val) for key, val in errs.items()}
    assert z.read_adam_state(r.state).step == cfg.steps
    progress(f"workload 1 {'fused' if fused else 'unfused'}: {cfg.steps} steps, worst norm "
             f"rel.err {norm_rel:.1e}, worst error / scale one-step {worst1} free {worst}, "
             f"params beyond 1 ulp: {far[0]}/{far[1]} of {n}")


# ------------------------------------------------------------ workload 5
def _w5_grads(cfg, r, step):
    return gen.device_grad_list(cfg, step, dev(), which=r.tensor_ids)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("fused", [False, True])
def test_workload5_shard_skip_full(fused):
    cfg = WORKLOADS[5]
    r = Rank(cfg, p_phase=oracle.partition(cfg.psi, cfg.nd, cfg.rank)[0] % 8)
    n, b = r.n, r.begin
    assert n == 250_728_263 and b % 8 == 1 and r.p.data_ptr() % 16 == 2
    assert len(r.tensor_ids) == 4
    gen.device_fill_normal_(r.master, cfg.master_seed(), cfg.master_sigma)
    th_o = r.master.cpu().numpy().copy()
    m_o, v_o, p_o = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, NP16)
    scales = FreeRunScales(cfg.hp, th_o)
    inj_step, inj = gen.inject_plan(cfg, n)
    t_expect = 0
    for k in range(cfg.steps):
        grads = _w5_grads(cfg, r, k)
        if k == inj_step:  # the non-finite values are planted in the per-tensor inputs
            offs = np.cumsum([0] + cfg.numels)
            for i, bits in inj:
                gi = b + i  # flat position -> tensor and offset
                ti = int(np.searchsorted(offs, gi, side="right") - 1)
                o = gi - int(offs[ti])
                grads[ti][o:o + 1] = _dev16(bits, grads[ti])
        if fused:
            r.gather_with_stats(grads)
        else:
            r.gather(grads)
        # the gathered shard against the oracle's flatten of the same tensors
        host = {i: _to_host16(t) for i, t in grads.items()}
        lo_t = int(np.cumsum([0] + cfg.numels)[r.tensor_ids[0]])
        sub = [host[i] for i in r.tensor_ids]
        g_ref = oracle.flatten(sub, b - lo_t, r.end - lo_t)
        del host, sub
        if k == inj_step:
            assert all(g_ref[i] == bits for i, bits in inj)
        assert np.array_equal(_to_host16(r.g), g_ref), k
        th0, m0, v0 = (a.cpu().numpy().copy() for a in (r.master, r.m, r.v))
        p_before = _to_host16(r.p).copy()
        r.stats_and_step(fused)
        torch.cuda.synchronize()
        st = z.read_grad_stats(r.stats)
        sq, ov = oracle.grad_stats(g_ref, cfg.dtype, cfg.hp.inv_loss_scale)
        assert st.overflow == ov
        state = z.read_adam_state(r.state)
        th_g, m_g, v_g = (a.cpu().numpy() for a in (r.master, r.m, r.v))
        p_g = _to_host16(r.p)
        if ov:
            assert k == inj_step and state.skip == 1 and state.step == t_expect
            for a, a0 in ((th_g, th0), (m_g, m0), (v_g, v0), (p_g, p_before)):
                assert np.array_equal(a.view(np.uint8), a0.view(np.uint8))
            progress(f"workload 5 step {k}: overflow -> skipped, step counter {state.step}")
            continue
        t_expect += 1
        assert state.step == t_expect and abs(st.sq_norm - sq) <= 1e-5 * sq
        gv = oracle.value16(g_ref, cfg.dtype)
        s1 = oracle.step_scalars(cfg.hp, True, st.sq_norm, st.overflow, t_expect - 1)
        assert s1.coef < 1.0  # clipping is active on this workload
        th1, m1, v1, p1 = th0.copy(), m0.copy(), v0.copy(), np.zeros(n, NP16)
        oracle.adamw_(s1, g_ref, cfg.dtype, th1, m1, v1, p1, cfg.dtype)
        e1 = check_adam_one_step(cfg.hp, s1, gv, th0, m0, v0, th_g, m_g, v_g, th1, m1, v1,
                                 label=f"step {k}")
        far1 = check_params16(p_g, th_g, th1, cfg.dtype,
                              f"step {k}")
        del th1, m1, v1, p1
        s = oracle.step_scalars(cfg.hp, True, sq, ov, t_expect - 1)
        oracle.adamw_(s, g_ref, cfg.dtype, th_o, m_o, v_o, p_o, cfg.dtype)
        scales.update(s, gv, m_o, v_o)
        e2 = scales.check(th_g, m_g, v_g, th_o, m_o, v_o, label=f"step {k}")
        far = check_params16(p_g, th_g, th_o, cfg.dtype,
                             f"step {k}")
        rel = abs(st.sq_norm - sq) / sq
        progress(f"workload 5 step {k}: sq {st.sq_norm:.9e} rel.err {rel:.1e} one-step {e1} "
                 f"free {e2} params beyond 1 ulp: {far1}/{far} of {n}")
        del grads
    assert t_expect == cfg.steps - 1
    # the 16-bit lead pad before the phase-faithful slice was never written
    assert int(r.p_raw[0].view(torch.int16).item()) == 0


def test_workload5_single_nan_at_last_element():
    cfg = WORKLOADS[5]
    r = Rank(cfg, p_phase=oracle.partition(cfg.psi, cfg.nd, cfg.rank)[0] % 8)
    gen.device_fill_normal_(r.master, cfg.master_seed(), cfg.master_sigma)
    r.gather(_w5_grads(cfg, r, 0))
    r.g[r.n - 1:] = _dev16(gen.F16_NAN, r.g)
    before = [a.clone() for a in (r.master, r.m, r.v, r.p_raw)]
    r.stats_and_step()
    torch.cuda.synchronize()
    assert z.read_grad_stats(r.stats).overflow == 1
    st = z.read_adam_state(r.state)
    assert st.skip == 1 and st.step == 0
    for a, b in zip((r.master, r.m, r.v, r.p_raw), before):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.fixture(autouse=True)
def _release_memory():
    yield
    _free()


# ------------------------------------------------ sampled full-size workloads
def _plan_map(cfg, lo, hi, bucket):
    """dst offset -> (tensor, src offset) lookup arrays from the oracle's plan."""
    segs = oracle.bucket_plan(cfg.numels, bucket or cfg.psi, lo, hi)
    return (np.array([s.dst_off for s in segs], np.int64), np.array([s.tensor for s in segs]),
            np.array([s.src_off for s in segs], np.int64))


def _expected_from_sources(grads, plan, idx):
    """Values the gather must produce at local positions idx, read from the
    per-tensor inputs at the positions the oracle's plan assigns."""
    dst_off, tens, src_off = plan
    k = np.searchsorted(dst_off, idx, side="right") - 1
    out = np.empty(idx.size, NP16)
    for ti in np.unique(tens[k]):
        sel = np.nonzero(tens[k] == ti)[0]
        offs = src_off[k[sel]] + (idx[sel] - dst_off[k[sel]])
        out[sel] = _to_host16(grads[int(ti)][torch.from_numpy(offs).to(dev())])
    return out


def _run_sampled(cfg, r, idx, fill_grads, label, fused=False):
    """cfg.steps steps on the full-size shard; oracle on the sampled indices
    with its own norm over every gradient."""
    idx_t = torch.from_numpy(idx).to(dev())
    th_o = r.master[idx_t].cpu().numpy()
    m_o, v_o = np.zeros(idx.size, np.float32), np.zeros(idx.size, np.float32)
    p_o = np.zeros(idx.size, NP16)
    scales = FreeRunScales(cfg.hp, th_o)
    for k in range(cfg.steps):
        fill_grads(k)
        th0, m0, v0 = (a[idx_t].cpu().numpy() for a in (r.master, r.m, r.v))
        r.stats_and_step(fused)
        torch.cuda.synchronize()
        st = z.read_grad_stats(r.stats)
        sq, ov = _oracle_norm_streamed(r.g, cfg.dtype, cfg.hp.inv_loss_scale)
        assert st.overflow == ov == 0
        assert abs(st.sq_norm - sq) <= 1e-5 * sq, (k, st.sq_norm, sq)
        g_s = _to_host16(r.g[idx_t])
        gv = oracle.value16(g_s, cfg.dtype)
        s1 = oracle.step_scalars(cfg.hp, True, st.sq_norm, st.overflow, k)
        th1, m1, v1, p1 = th0.copy(), m0.copy(), v0.copy(), np.zeros(idx.size, NP16)
        oracle.adamw_(s1, g_s, cfg.dtype, th1, m1, v1, p1, cfg.dtype)
        th_g, m_g, v_g = (a[idx_t].cpu().numpy() for a in (r.master, r.m, r.v))
        p_g = _to_host16(r.p[idx_t])
        e1 = check_adam_one_step(cfg.hp, s1, gv, th0, m0, v0, th_g, m_g, v_g, th1, m1, v1,
                                 label=f"{label} step {k}")
        f1 = check_params16(p_g, th_g, th1, cfg.dtype,
                            f"{label} step {k}")
        s = oracle.step_scalars(cfg.hp, True, sq, ov, k)
        oracle.adamw_(s, g_s, cfg.dtype, th_o, m_o, v_o, p_o, cfg.dtype)
        scales.update(s, gv, m_o, v_o)
        e2 = scales.check(th_g, m_g, v_g, th_o, m_o, v_o, label=f"{label} step {k}")
        f2 = check_params16(p_g, th_g, th_o, cfg.dtype,
                            f"{label} step {k}")
        progress(f"{label} step {k}: sq {st.sq_norm:.9e} rel.err {abs(st.sq_norm - sq) / sq:.1e} "
                 f"coef {s.coef:.6f} one-step {e1} free {e2} params beyond 1 ulp: {f1}/{f2} "
                 f"of {idx.size}")
    assert z.read_adam_state(r.state).step == cfg.steps


@pytest.mark.timeout(900)
@pytest.mark.parametrize("fused", [True, False])
def test_workload2_gpt2_1p5b_sampled(fused):
    """The bench's workload, launch configuration and state layout (fused:
    the bench's default step; unfused: one gather per 500M-element buffer,
    then stats)."""
    cfg = WORKLOADS[2]
    r = Rank(cfg, spread=True)
    assert r.n == cfg.psi == 1_557_611_200
    gen.device_fill_normal_(r.master, cfg.master_seed(), cfg.master_sigma)
    idx = _sample_indices(cfg, r.begin, r.end, 4_000_000, 4242, cfg.bucket_elems)
    plan = _plan_map(cfg, r.begin, r.end, cfg.bucket_elems)

    def fill(k):
        grads = gen.device_grad_list(cfg, k, dev())
        if fused:
            r.gather_with_stats(grads)
        else:
            r.gather(grads)
        exp = _expected_from_sources(grads, plan, idx)
        assert np.array_equal(_to_host16(r.g[torch.from_numpy(idx).to(dev())]), exp), k

    _run_sampled(cfg, r, idx, fill, f"workload 2 {'fused' if fused else 'unfused'}", fused)
    st = z.read_adam_state(r.state)
    assert st.coef < 0.1  # clipping at 1.0 is active on this workload


@pytest.mark.timeout(900)
def test_workload3_gpt_7p5b_rank3_buckets_sampled():
    cfg = WORKLOADS[3]
    r = Rank(cfg)
    assert (r.begin, r.end) == (2_797_398_528, 3_729_864_704)
    B = cfg.bucket_elems
    cb = torch.empty(B, dtype=gen.torch_dtype(cfg.dtype), device=dev())  # one fused buffer
    gen.device_fill_normal_(r.master, cfg.master_seed(), cfg.master_sigma)
    idx = _sample_indices(cfg, r.begin, r.end, 4_000_000, 4343, B)
    idx_t = torch.from_numpy(idx).to(dev())
    shard_plan = _plan_map(cfg, r.begin, r.end, B)
    n_buckets = -(-cfg.psi // B)
    assert n_buckets == 15

    def fill(k):
        grads = gen.device_grad_list(cfg, k, dev())
        ptrs = [grads[i] for i in range(len(cfg.numels))]
        for b in range(n_buckets):
            lo, hi = b * B, min((b + 1) * B, cfg.psi)
            owns = lo < r.end and r.begin < hi
            if not owns and k > 0:
                continue  # every window is checked on the first step
            z.zero_bucket_flatten(ptrs, cfg.numels, cfg.dtype, lo, hi - lo, cb)
            if k == 0:  # the fused buffer itself, sampled
                bi = _sample_indices(cfg, lo, hi, 100_000, 5000 + b)
                exp = _expected_from_sources(grads, _plan_map(cfg, lo, hi, B), bi)
                got = _to_host16(cb[torch.from_numpy(bi).to(dev())])
                assert np.array_equal(got, exp), b
            if owns:  # this rank's part of the window, out of the fused buffer
                a, e = max(lo, r.begin), min(hi, r.end)
                z.zero_bucket_flatten([cb], [hi - lo], cfg.dtype, a - lo, e - a,
                                      r.g.data_ptr() + 2 * (a - r.begin))
        exp = _expected_from_sources(grads, shard_plan, idx)
        assert np.array_equal(_to_host16(r.g[idx_t]), exp), k
        del grads, ptrs

    _run_sampled(cfg, r, idx, fill, "workload 3")
    # the accounting pins of this model size
    assert z.zero_mem_bytes(2, 7_500_000_000, 64, 12) == oracle.mem_bytes(2, 7_500_000_000, 64, 12)


@pytest.mark.timeout(900)
def test_workload4_gpt_13b_full_state_sampled():
    cfg = WORKLOADS[4]
    need = 16 * cfg.psi + (1 << 30)
    free, total = torch.cuda.mem_get_info()
    if free < need:
        pytest.skip(f"needs {need / 1e9:.1f} GB of device memory, {free / 1e9:.1f} GB free")
    r = Rank(cfg)
    assert r.n == 12_848_143_360
    gen.device_fill_normal_(r.master, cfg.master_seed(), cfg.master_sigma)
    idx = _sample_indices(cfg, r.begin, r.end, 4_000_000, 4444)
    progress(f"workload 4: {torch.cuda.memory_allocated() / 1e9:.1f} GB resident")

    def fill(k):
        gen.device_fill_normal_(r.g, cfg.grad_seed(k), cfg.grad_sigma, cfg.loss_scale)

    _run_sampled(cfg, r, idx, fill, "workload 4")
