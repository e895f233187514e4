"""One whole step captured in a HIP graph: the fused gather+stats, AdamW and
the loss-scale update record only kernels (no memset, allocation or
synchronisation), so replaying the graph must give, replay after replay,
bit for bit what the same calls give eagerly.  The same for the step read in
place from the per-tensor gradients, and for the step whose statistics use
the library's own scratch (zero_grad_stats_noalloc, meant for callers under
graph capture)."""
import numpy as np
import pytest
import torch

import zero_sharded_mixed_grads_amd as z
from synth import gen
from util import dev

pytestmark = pytest.mark.gpu


class _Rank:
    """One rank's buffers for a shard of three gradient tensors."""

    def __init__(self, numels, th0, cfg):
        n = sum(numels)
        self.numels, self.n, self.cfg = numels, n, cfg
        self.grads = [torch.zeros(k, dtype=torch.int16, device=dev()) for k in numels]
        self.g = torch.zeros(n, dtype=torch.int16, device=dev())
        self.th = torch.from_numpy(th0.copy()).to(dev())
        self.m, self.v = torch.zeros_like(self.th), torch.zeros_like(self.th)
        self.p = torch.zeros(n, dtype=torch.int16, device=dev())
        self.stats, self.state = z.new_grad_stats(dev()), z.new_adam_state(dev())
        self.scale = z.new_loss_scale(dev())
        z.zero_loss_scale_init(cfg, self.scale)
        nb = z.zero_bucket_flatten_stats_workspace(numels, 0, n)
        self.ws = torch.empty(nb, dtype=torch.uint8, device=dev())
        self.hp = z.adamw(max_grad_norm=1.0, inv_loss_scale=float("nan"))  # scale from device

    def step(self, kind="gathered"):
        if kind == "tensors":  # read in place: no gathered shard
            z.zero_grad_stats_tensors(self.grads, self.numels, "f16", 0, self.n, float("nan"),
                                      self.ws, self.ws.numel(), self.stats, d_scale=self.scale)
            z.zero_adam_step_tensors(self.hp, self.grads, self.numels, "f16", 0, self.n, self.th,
                                     self.m, self.v, self.p, "f16", self.stats, self.state,
                                     d_scale=self.scale)
        else:
            if kind == "noalloc":  # gather, then statistics in the library's scratch
                z.zero_bucket_flatten(self.grads, self.numels, "f16", 0, self.n, self.g)
                z.zero_grad_stats_noalloc(self.g, "f16", self.n, float("nan"), self.stats,
                                          d_scale=self.scale)
            else:
                z.zero_bucket_flatten_stats(self.grads, self.numels, "f16", 0, self.n, self.g,
                                            float("nan"), self.ws, self.ws.numel(), self.stats,
                                            d_scale=self.scale)
            z.zero_adam_step(self.hp, self.g, "f16", self.th, self.m, self.v, self.p, "f16",
                             self.n, self.stats, self.state, d_scale=self.scale)
        z.zero_loss_scale_update(self.cfg, self.stats, self.scale)

    def snapshot(self):
        return [x.cpu().numpy().tobytes() for x in
                (self.g, self.th, self.m, self.v, self.p, self.stats, self.state, self.scale)]


@pytest.mark.parametrize("kind", ["gathered", "tensors", "noalloc"])
def test_step_replays_in_a_graph_bit_for_bit(kind):
    numels = [70_001, 13, 30_003]
    n = sum(numels)
    rng = np.random.default_rng(11)
    th0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    cfg = z.loss_scaler(init_scale=2.0 ** 12, growth_interval=2, min_scale=1.0)
    eager, graphed = _Rank(numels, th0, cfg), _Rank(numels, th0, cfg)

    def load_grads(k):
        gb = gen.f32_to_bits16((rng.standard_normal(n) * 2.0 ** 2).astype(np.float32), "f16")
        if k == 2:
            gb[n // 3] = gen.F16_POS_INF  # an overflowing step: skipped, the scale backs off
        pieces = np.split(gb.view(np.int16), np.cumsum(numels)[:-1])
        for r in (eager, graphed):
            for t, piece in zip(r.grads, pieces):
                t.copy_(torch.from_numpy(piece.copy()))

    # warm up on a side stream (first-call host caches), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        warm = _Rank(numels, th0, cfg)
        warm.step(kind)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        graphed.step(kind)
    torch.cuda.synchronize()
    assert z.read_adam_state(graphed.state).step == 0  # capture ran nothing

    for k in range(6):
        load_grads(k)
        torch.cuda.synchronize()
        graph.replay()
        eager.step(kind)
        torch.cuda.synchronize()
        a, b = eager.snapshot(), graphed.snapshot()
        names = ["g", "master", "m", "v", "param", "stats", "state", "scale"]
        for name, x, y in zip(names, a, b):
            assert x == y, (k, name)
    st = z.read_adam_state(eager.state)
    sc = z.read_loss_scale(eager.scale)
    assert st.step == 5 and sc.overflows == 1
