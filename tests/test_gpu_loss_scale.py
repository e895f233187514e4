"""Dynamic loss scaling on the device: the scale state follows the oracle's
rule bit for bit over runs with overflows, and every call that unscales
gradients gives bit-identical results whether the inverse scale comes from
the device state or from the host."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_grads_amd as z
from synth import gen
from util import dev

pytestmark = pytest.mark.gpu


def _dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(dev())


def _scale_state(scale):
    """A device zero_loss_scale_t holding `scale` (set through the init call)."""
    d = z.new_loss_scale(dev())
    z.zero_loss_scale_init(z.loss_scaler(init_scale=scale, min_scale=min(scale, 1.0)), d)
    return d


@pytest.mark.parametrize("rule", [
    dict(init_scale=2.0 ** 10, growth_factor=2.0, backoff_factor=0.5, growth_interval=3,
         min_scale=2.0 ** 6, max_scale=2.0 ** 13),
    dict(init_scale=1000.0, growth_factor=3.0, backoff_factor=0.3, growth_interval=2,
         min_scale=0.7, max_scale=1e6),
    dict(init_scale=2.0 ** 15, growth_factor=2.0, backoff_factor=0.5, growth_interval=1,
         min_scale=1.0, max_scale=float("inf")),
])
def test_loss_scale_sequence_matches_oracle(rule):
    """A run of real steps (statistics, AdamW, scale update) with overflows
    injected at seeded steps: after every step the device state equals the
    oracle's, bit for bit, and the AdamW step counter counts the good steps."""
    cfg = z.loss_scaler(**rule)
    ocfg = oracle.Scaler(rule["init_scale"], rule["growth_factor"], rule["backoff_factor"],
                         rule["growth_interval"], rule["min_scale"], rule["max_scale"])
    rng = np.random.default_rng(7)
    steps = 40
    flags = (rng.random(steps) < 0.25).astype(int)
    flags[:2] = [0, 1]
    expect = oracle.loss_scale_sequence(ocfg, flags.tolist())
    n = 10_007
    d_scale = z.new_loss_scale(dev())
    z.zero_loss_scale_init(cfg, d_scale)
    st = z.read_loss_scale(d_scale)
    assert (st.scale, st.inv_scale, st.good_steps, st.overflows) == \
        (rule["init_scale"], 1.0 / rule["init_scale"], 0, 0)
    th = torch.zeros(n, device=dev())
    m, v = torch.zeros_like(th), torch.zeros_like(th)
    p = torch.zeros(n, dtype=torch.int16, device=dev())
    stats, state = z.new_grad_stats(dev()), z.new_adam_state(dev())
    ws = z.new_workspace(n, dev())
    hp = z.adamw(max_grad_norm=1.0, inv_loss_scale=float("nan"))  # ignored: d_scale given
    for k in range(steps):
        gb = gen.f32_to_bits16(rng.standard_normal(n).astype(np.float32) * 1e-2, "f16")
        if flags[k]:
            gb[rng.integers(n)] = gen.F16_POS_INF
        g = _dev16(gb)
        z.zero_grad_stats(g, "f16", n, float("nan"), ws, ws.numel(), stats, d_scale=d_scale)
        z.zero_adam_step(hp, g, "f16", th, m, v, p, "f16", n, stats, state, d_scale=d_scale)
        z.zero_loss_scale_update(cfg, stats, d_scale)
        got = z.read_loss_scale(d_scale)
        assert (got.scale, got.inv_scale, got.good_steps, got.overflows) == expect[k], (k, flags[k])
        assert z.read_adam_state(state).step == k + 1 - int(flags[:k + 1].sum())


def test_device_scale_equals_host_scale():
    """zero_grad_stats, zero_bucket_flatten_stats, zero_adam_step and
    zero_offload_adam_step read the inverse scale from the device state when
    it is given, with results identical to passing the same value on the host."""
    scale = 2.0 ** 12 * 3  # not a power of two: its inverse is rounded
    inv = 1.0 / scale
    d_scale = _scale_state(scale)
    assert z.read_loss_scale(d_scale).inv_scale == inv
    rng = np.random.default_rng(3)
    numels = [1000, 4099, 17, 30_000]
    n = sum(numels)
    gbs = [gen.f32_to_bits16(rng.standard_normal(k).astype(np.float32) * 30.0, "bf16")
           for k in numels]
    srcs = [_dev16(b) for b in gbs]
    gall = _dev16(np.concatenate(gbs))
    ws = z.new_workspace(n, dev())
    outs = {}
    for mode in ("host", "device"):
        kw = dict(d_scale=d_scale) if mode == "device" else {}
        hinv = inv if mode == "host" else float("nan")
        s1, s2 = z.new_grad_stats(dev()), z.new_grad_stats(dev())
        z.zero_grad_stats(gall, "bf16", n, hinv, ws, ws.numel(), s1, **kw)
        dst = torch.zeros(n, dtype=torch.int16, device=dev())
        fwb = z.zero_bucket_flatten_stats_workspace(numels, 0, n)
        fws = torch.empty(fwb, dtype=torch.uint8, device=dev())
        z.zero_bucket_flatten_stats(srcs, numels, "bf16", 0, n, dst, hinv, fws, fwb, s2, **kw)
        th0 = rng.standard_normal(n).astype(np.float32) if mode == "host" else outs["th0"]
        outs["th0"] = th0
        hp = z.adamw(max_grad_norm=0.5, inv_loss_scale=hinv)
        dstate = [torch.from_numpy(th0.copy()).to(dev()), torch.zeros(n, device=dev()),
                  torch.zeros(n, device=dev())]
        pdv = torch.zeros(n, dtype=torch.int16, device=dev())
        sd = z.new_adam_state(dev())
        hstate = [torch.from_numpy(th0.copy()), torch.zeros(n), torch.zeros(n)]
        phv = torch.zeros(n, dtype=torch.int16, device=dev())
        sh = z.new_adam_state(dev())
        nb = z.zero_offload_staging_bytes(4096)
        stg = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
        for _ in range(2):
            z.zero_adam_step(hp, gall, "bf16", *dstate, pdv, "bf16", n, s1, sd, **kw)
            z.zero_offload_adam_step(hp, gall, "bf16", *hstate, phv, "bf16", n, s1, sh, stg, nb,
                                     **kw)
        torch.cuda.synchronize()
        outs[mode] = [bytes(s1.cpu().numpy()), bytes(s2.cpu().numpy()),
                      dst.cpu().numpy().tobytes(), bytes(sd.cpu().numpy()),
                      *[x.cpu().numpy().tobytes() for x in (*dstate, pdv)],
                      *[x.numpy().tobytes() for x in hstate], phv.cpu().numpy().tobytes(),
                      bytes(sh.cpu().numpy())]
    names = ["grad_stats", "flatten_stats", "flatten_dst", "adam_state", "master", "m", "v",
             "param", "offload_master", "offload_m", "offload_v", "offload_param",
             "offload_state"]
    for name, a, b in zip(names, outs["host"], outs["device"]):
        assert a == b, name
    # the norm is of the unscaled gradients
    sq, ov = oracle.grad_stats(np.concatenate(gbs), "bf16", inv)
    got = z.read_grad_stats(torch.frombuffer(bytearray(outs["device"][0]), dtype=torch.uint8))
    assert ov == 0 and got.overflow == 0 and abs(got.sq_norm - sq) <= 1e-12 * sq
