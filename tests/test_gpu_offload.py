"""AdamW with the optimizer state in host memory: the same results as the
device step (bit for bit: the host loop performs the same fp32 operations in
the same order), within the oracle's bounds, the skip path, and chunking."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_grads_amd as z
from synth import AdamW, gen
from util import check_adam_one_step, check_params16, dev

pytestmark = pytest.mark.gpu


def _staging(chunk):
    nb = z.zero_offload_staging_bytes(chunk)
    return torch.empty(nb, dtype=torch.uint8, pin_memory=True), nb


def _run_both(n, gdt, pdt, hp, grads, th0, m0, v0, chunk, with_stats=True):
    """Runs the same steps on the device path and on the offload path."""
    d = [torch.from_numpy(a.copy()).to(dev()) for a in (th0, m0, v0)]
    h = [torch.from_numpy(a.copy()) for a in (th0, m0, v0)]
    pd = torch.zeros(n, dtype=torch.int16, device=dev())
    ph = torch.zeros(n, dtype=torch.int16, device=dev())
    sd, sh = z.new_adam_state(dev()), z.new_adam_state(dev())
    stats = z.new_grad_stats(dev()) if with_stats else None
    ws = z.new_workspace(n, dev())
    stg, nb = _staging(chunk)
    hw = z.adamw(**hp.__dict__)
    for gb in grads:
        g = torch.from_numpy(gb.view(np.int16)).to(dev())
        if with_stats:
            z.zero_grad_stats(g, gdt, n, hp.inv_loss_scale, ws, ws.numel(), stats)
        z.zero_adam_step(hw, g, gdt, *d, pd, pdt, n, stats, sd)
        z.zero_offload_adam_step(hw, g, gdt, *h, ph, pdt, n, stats, sh, stg, nb)
    torch.cuda.synchronize()
    return d, pd, sd, h, ph, sh, stats


@pytest.mark.parametrize("gdt,pdt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "bf16"),
                                     ("bf16", "f16")])
@pytest.mark.parametrize("n,chunk", [(1, 4096), (4097, 4096), (100_003, 4096),
                                     (1_000_003, 1 << 18)])
def test_offload_matches_device_step_bit_for_bit(gdt, pdt, n, chunk):
    hp = AdamW(max_grad_norm=0.3, inv_loss_scale=2.0 ** -8)
    rng = np.random.default_rng(n)
    th0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = (rng.random(n) * 1e-8).astype(np.float32)
    grads = [gen.f32_to_bits16((rng.standard_normal(n) * 0.5).astype(np.float32), gdt)
             for _ in range(3)]
    d, pd, sd, h, ph, sh, _ = _run_both(n, gdt, pdt, hp, grads, th0, m0, v0, chunk)
    for a, b in zip(d, h):
        assert np.array_equal(a.cpu().numpy().view(np.uint32), b.numpy().view(np.uint32))
    assert torch.equal(pd, ph)
    assert z.read_adam_state(sd).step == z.read_adam_state(sh).step == 3


def test_offload_against_oracle_one_step():
    n = 300_001
    hp = AdamW(max_grad_norm=0.05, inv_loss_scale=2.0 ** -10)
    rng = np.random.default_rng(5)
    th0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = (rng.random(n) * 1e-8).astype(np.float32)
    gb = gen.f32_to_bits16((rng.standard_normal(n)).astype(np.float32), "f16")
    _, _, _, h, ph, sh, stats = _run_both(n, "f16", "f16", hp, [gb], th0, m0, v0, 1 << 16)
    st = z.read_grad_stats(stats)
    sq, ov = oracle.grad_stats(gb, "f16", hp.inv_loss_scale)
    assert abs(st.sq_norm - sq) <= 1e-12 * sq
    s = oracle.step_scalars(hp, True, st.sq_norm, st.overflow, 0)
    assert s.coef < 1.0
    th, m, v, p = th0.copy(), m0.copy(), v0.copy(), np.zeros(n, np.uint16)
    oracle.adamw_(s, gb, "f16", th, m, v, p, "f16")
    e = check_adam_one_step(hp, s, oracle.value16(gb, "f16"), th0, m0, v0, h[0].numpy(),
                            h[1].numpy(), h[2].numpy(), th, m, v)
    check_params16(ph.cpu().numpy().view(np.uint16), h[0].numpy(), th,
                   "f16")


def test_offload_skip_and_empty():
    n = 50_000
    hp = AdamW(max_grad_norm=1.0)
    rng = np.random.default_rng(6)
    th0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    z0 = np.zeros(n, np.float32)
    gb = gen.f32_to_bits16(rng.standard_normal(n).astype(np.float32), "f16")
    gb[n - 1] = gen.F16_NAN
    _, _, _, h, ph, sh, _ = _run_both(n, "f16", "f16", hp, [gb], th0, z0, z0, 4096)
    assert np.array_equal(h[0].numpy(), th0) and not h[1].numpy().any()
    assert not ph.any()  # params never written
    st = z.read_adam_state(sh)
    assert st.skip == 1 and st.step == 0
    # n == 0 still advances the step state, like the device step
    sh0 = z.new_adam_state(dev())
    stg, nb = _staging(4096)
    z.zero_offload_adam_step(z.adamw(), None, "f16", None, None, None, None, "f16", 0, None, sh0,
                             stg, nb)
    assert z.read_adam_state(sh0).step == 1


def test_offload_errors():
    n = 10_000
    h = [torch.zeros(n) for _ in range(3)]
    g = torch.zeros(n, dtype=torch.int16, device=dev())
    p = torch.zeros(n, dtype=torch.int16, device=dev())
    st = z.new_adam_state(dev())
    stg, nb = _staging(4096)
    with pytest.raises(z.ZeroError) as e:
        z.zero_offload_adam_step(z.adamw(), g, "f16", *h, p, "f16", n, None, st, stg, 4096 * 8 - 1)
    assert e.value.status == z.ZERO_ENOSPC
    with pytest.raises(z.ZeroError) as e:
        z.zero_offload_adam_step(z.adamw(), g, "f16", h[0], h[0], h[2], p, "f16", n, None, st,
                                 stg, nb)
    assert e.value.status == z.ZERO_EINVAL
    with pytest.raises(z.ZeroError) as e:
        z.zero_offload_staging_bytes(100)
    assert e.value.status == z.ZERO_EINVAL
