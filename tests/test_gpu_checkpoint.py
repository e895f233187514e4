"""Sharded checkpoints on the GPU: bit-exact round trip, re-sharding to a
different number of ranks (checked against the oracle's partition of the
concatenated shards), and bit-exact resume of training."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_grads_amd as z
from synth import AdamW, gen
from util import dev

pytestmark = pytest.mark.gpu


def _state_bufs(n):
    return [torch.empty(n, dtype=torch.float32, device=dev()) for _ in range(3)]


def _save_run(tmp_path, psi, nd, host_arrays, step):
    paths = []
    for r in range(nd):
        b, e = oracle.partition(psi, nd, r)
        bufs = [torch.from_numpy(a[b:e].copy()).to(dev()) for a in host_arrays]
        st = z.new_adam_state(dev())
        st.copy_(torch.from_numpy(np.frombuffer(bytes(z.AdamState(step=step)), np.uint8).copy()))
        p = str(tmp_path / f"nd{nd}_r{r}.zck")
        z.zero_ckpt_save(p, psi, nd, r, *bufs, st)
        paths.append(p)
    return paths


def test_ckpt_roundtrip_and_reshard(tmp_path):
    psi = 1_000_003
    rng = np.random.default_rng(0)
    full = [rng.standard_normal(psi).astype(np.float32) for _ in range(3)]
    full[1][::7] = np.float32(-0.0)
    full[2][5] = np.float32(np.inf)  # bytes are bytes
    paths = _save_run(tmp_path, psi, 3, full, step=17)
    for nd_new in (1, 2, 3, 5, 7):
        for r in range(nd_new):
            b, e = oracle.partition(psi, nd_new, r)
            bufs = _state_bufs(e - b)
            st = z.new_adam_state(dev())
            z.zero_ckpt_load(list(reversed(paths)), psi, nd_new, r, *bufs, st)
            for got, ref in zip(bufs, full):
                assert np.array_equal(got.cpu().numpy().view(np.uint32),
                                      ref[b:e].view(np.uint32)), (nd_new, r)
            s = z.read_adam_state(st)
            assert s.step == 17 and s.skip == 0 and s.bc1 == 0.0 and s.bc2 == 0.0


def _train(bufs, p, grads, hp, state, stats_mode):
    """Steps of the whole path on one rank's buffers with the given grads."""
    th, m, v = bufs
    n = th.numel()
    stats = z.new_grad_stats(dev())
    ws = z.new_workspace(n, dev())
    for g in grads:
        if stats_mode:
            z.zero_grad_stats(g, "f16", n, hp.inv_loss_scale, ws, ws.numel(), stats)
        z.zero_adam_step(z.adamw(**hp.__dict__), g, "f16", th, m, v, p, "f16", n,
                         stats if stats_mode else None, state)


def test_ckpt_resume_is_bit_exact(tmp_path):
    n = 777_777
    hp = AdamW(max_grad_norm=0.5, inv_loss_scale=2.0 ** -10)
    rng = np.random.default_rng(1)
    grads = [torch.from_numpy(gen.f32_to_bits16((rng.standard_normal(n) * 300).astype(np.float32),
                                                "f16").view(np.int16)).to(dev()) for _ in range(5)]
    th0 = rng.standard_normal(n).astype(np.float32) * 0.02
    bufs = [torch.from_numpy(th0.copy()).to(dev()), torch.zeros(n, device=dev()),
            torch.zeros(n, device=dev())]
    p = torch.zeros(n, dtype=torch.int16, device=dev())
    st = z.new_adam_state(dev())
    _train(bufs, p, grads[:3], hp, st, True)
    path = str(tmp_path / "r0.zck")
    z.zero_ckpt_save(path, n, 1, 0, *bufs, st)
    _train(bufs, p, grads[3:], hp, st, True)
    # resume into fresh buffers
    bufs2 = _state_bufs(n)
    p2 = torch.zeros(n, dtype=torch.int16, device=dev())
    st2 = z.new_adam_state(dev())
    z.zero_ckpt_load([path], n, 1, 0, *bufs2, st2)
    assert z.read_adam_state(st2).step == 3
    _train(bufs2, p2, grads[3:], hp, st2, True)
    for a, b in zip(bufs + [p], bufs2 + [p2]):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b)
    assert z.read_adam_state(st2).step == 5


def test_ckpt_reshard_mid_training_matches_unsharded(tmp_path):
    """2 ranks train 2 steps, save, resume as 3 ranks for 2 more steps: the
    result equals 4 steps on one rank bit for bit (no clipping, so each
    element's update depends on that element alone)."""
    psi = 300_007
    hp = AdamW(inv_loss_scale=2.0 ** -10)
    rng = np.random.default_rng(2)
    g_all = [gen.f32_to_bits16((rng.standard_normal(psi) * 300).astype(np.float32), "f16")
             for _ in range(4)]
    th0 = rng.standard_normal(psi).astype(np.float32) * 0.02
    # reference: one rank, 4 steps
    ref = [torch.from_numpy(th0.copy()).to(dev()), torch.zeros(psi, device=dev()),
           torch.zeros(psi, device=dev())]
    pref = torch.zeros(psi, dtype=torch.int16, device=dev())
    _train(ref, pref, [torch.from_numpy(g.view(np.int16)).to(dev()) for g in g_all], hp,
           z.new_adam_state(dev()), False)
    # 2 ranks, 2 steps, save
    paths = []
    for r in range(2):
        b, e = oracle.partition(psi, 2, r)
        bufs = [torch.from_numpy(th0[b:e].copy()).to(dev()), torch.zeros(e - b, device=dev()),
                torch.zeros(e - b, device=dev())]
        p = torch.zeros(e - b, dtype=torch.int16, device=dev())
        st = z.new_adam_state(dev())
        _train(bufs, p, [torch.from_numpy(g[b:e].view(np.int16).copy()).to(dev())
                         for g in g_all[:2]], hp, st, False)
        paths.append(str(tmp_path / f"r{r}.zck"))
        z.zero_ckpt_save(paths[-1], psi, 2, r, *bufs, st)
    # resume as 3 ranks, 2 more steps
    for r in range(3):
        b, e = oracle.partition(psi, 3, r)
        bufs = _state_bufs(e - b)
        p = torch.zeros(e - b, dtype=torch.int16, device=dev())
        st = z.new_adam_state(dev())
        z.zero_ckpt_load(paths, psi, 3, r, *bufs, st)
        _train(bufs, p, [torch.from_numpy(g[b:e].view(np.int16).copy()).to(dev())
                         for g in g_all[2:]], hp, st, False)
        for a, rf in zip(bufs, ref):
            assert torch.equal(a.view(torch.int32), rf[b:e].view(torch.int32)), r
        assert torch.equal(p, pref[b:e])
        assert z.read_adam_state(st).step == 4


def test_ckpt_save_errors(tmp_path):
    n = 1000
    bufs = _state_bufs(n)
    st = z.new_adam_state(dev())
    with pytest.raises(z.ZeroError) as e:
        z.zero_ckpt_save(str(tmp_path / "no_such_dir" / "x.zck"), n, 1, 0, *bufs, st)
    assert e.value.status == z.ZERO_EIO
    with pytest.raises(z.ZeroError) as e:
        z.zero_ckpt_save(str(tmp_path / "x.zck"), n, 2, 2, *bufs, st)
    assert e.value.status == z.ZERO_EINVAL
    # a save that fails after writing (the target is a directory, so the final
    # rename fails) leaves neither the target nor its temporary file behind
    target = tmp_path / "taken"
    target.mkdir()
    with pytest.raises(z.ZeroError) as e:
        z.zero_ckpt_save(str(target), n, 1, 0, *bufs, st)
    assert e.value.status == z.ZERO_EIO
    assert target.is_dir() and not (tmp_path / "taken.tmp").exists()


def _dyn_steps(bufs, p, grads, st, d_scale, cfg, overflow_at=()):
    """Steps with dynamic loss scaling on one shard: statistics and AdamW read
    the scale from the device; the scale is advanced after each step."""
    n = bufs[0].numel()
    stats, ws = z.new_grad_stats(dev()), z.new_workspace(n, dev())
    hp = z.adamw(max_grad_norm=1.0, inv_loss_scale=float("nan"))
    for k, g in enumerate(grads):
        if k in overflow_at:
            g = g.clone()
            g[n // 2] = 0x7C00  # +inf
        z.zero_grad_stats(g, "f16", n, float("nan"), ws, ws.numel(), stats, d_scale=d_scale)
        z.zero_adam_step(hp, g, "f16", *bufs, p, "f16", n, stats, st, d_scale=d_scale)
        z.zero_loss_scale_update(cfg, stats, d_scale)
    torch.cuda.synchronize()


def test_ckpt_resume_with_dynamic_loss_scale_is_bit_exact(tmp_path):
    """Two ranks save state and the (identical) loss-scale state; one rank
    resumes from both files and continues exactly like the run that never
    stopped, loss scale included.  A load that asks for the loss scale from
    files without it, or with differing ones, is refused."""
    n = 300_007
    cfg = z.loss_scaler(init_scale=2.0 ** 12, growth_interval=2, min_scale=1.0)
    rng = np.random.default_rng(2)
    grads = [torch.from_numpy(gen.f32_to_bits16((rng.standard_normal(n) * 3).astype(np.float32),
                                                "f16").view(np.int16)).to(dev()) for _ in range(6)]
    th0 = rng.standard_normal(n).astype(np.float32) * 0.02
    bufs = [torch.from_numpy(th0.copy()).to(dev()), torch.zeros(n, device=dev()),
            torch.zeros(n, device=dev())]
    p = torch.zeros(n, dtype=torch.int16, device=dev())
    st, sc = z.new_adam_state(dev()), z.new_loss_scale(dev())
    z.zero_loss_scale_init(cfg, sc)
    _dyn_steps(bufs, p, grads[:3], st, sc, cfg, overflow_at=(1,))
    paths = []
    for r in range(2):
        b, e = oracle.partition(n, 2, r)
        paths.append(str(tmp_path / f"dyn_r{r}.zck"))
        z.zero_ckpt_save(paths[-1], n, 2, r, *[x[b:e] for x in bufs], st, d_scale=sc)
    saved_scale = z.read_loss_scale(sc)
    saved_step = z.read_adam_state(st).step
    assert saved_scale.overflows == 1 and saved_step == 2
    _dyn_steps(bufs, p, grads[3:], st, sc, cfg)
    # resume as one rank from the two shards
    bufs2 = _state_bufs(n)
    p2 = torch.zeros(n, dtype=torch.int16, device=dev())
    st2, sc2 = z.new_adam_state(dev()), z.new_loss_scale(dev())
    z.zero_ckpt_load(paths, n, 1, 0, *bufs2, st2, d_scale=sc2)
    got = z.read_loss_scale(sc2)
    assert bytes(got) == bytes(saved_scale)
    _dyn_steps(bufs2, p2, grads[3:], st2, sc2, cfg)
    for a, b in zip(bufs, bufs2):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(p, p2)
    assert bytes(z.read_loss_scale(sc)) == bytes(z.read_loss_scale(sc2))
    assert z.read_adam_state(st2).step == z.read_adam_state(st).step
    # refusals: no record in one file; records that differ between files (the
    # re-saved shard keeps the save's step, so only the record differs)
    b, e = oracle.partition(n, 2, 1)
    st_saved = z.new_adam_state(dev())
    st_saved.copy_(torch.from_numpy(
        np.frombuffer(bytes(z.AdamState(step=saved_step)), np.uint8).copy()))
    z.zero_ckpt_save(paths[1], n, 2, 1, *[x[b:e] for x in bufs2], st_saved)  # no d_scale
    with pytest.raises(z.ZeroError) as ex:
        z.zero_ckpt_load(paths, n, 1, 0, *bufs2, st2, d_scale=sc2)
    assert ex.value.status == z.ZERO_EINVAL and "no loss-scale" in str(ex.value)
    z.zero_ckpt_load(paths, n, 1, 0, *bufs2, st2)  # without asking for it: fine
    z.zero_ckpt_save(paths[1], n, 2, 1, *[x[b:e] for x in bufs2], st_saved, d_scale=sc2)
    with pytest.raises(z.ZeroError) as ex:
        z.zero_ckpt_load(paths, n, 1, 0, *bufs2, st2, d_scale=sc2)
    assert ex.value.status == z.ZERO_EINVAL and "different loss-scale" in str(ex.value)
