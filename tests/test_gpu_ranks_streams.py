"""Nd ranks of one flat model state in one process, each on its own stream.

Each rank runs the statistics and the AdamW step on its contiguous part of
the flat state (ZeRO paper summary page, section ZeRO-DP, Stage 1: each rank
updates only its 1/Nd).  Between the two calls the ranks' 16-byte statistics
are combined as a multi-rank caller would all-reduce them (sum of the squared
norms, maximum of the overflow flags); here a device-side torch reduction
stands in for that collective.  The concatenated rank updates must equal the
unsharded step bit for bit when both use the same combined statistics, and an
overflow in one rank's part must skip the step on every rank."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_mixed_grads_amd as z
from synth import gen
from util import dev, progress

pytestmark = pytest.mark.gpu

PSI, ND = 1_000_003, 7  # ragged parts: their starts lie at several 16-byte phases


class _State:
    """Flat fp16 grad, fp32 master/m/v and fp16 param of PSI elements."""

    def __init__(self, th0):
        self.g = torch.zeros(PSI, dtype=torch.int16, device=dev())
        self.th = torch.from_numpy(th0.copy()).to(dev())
        self.m, self.v = torch.zeros_like(self.th), torch.zeros_like(self.th)
        self.p = torch.zeros(PSI, dtype=torch.int16, device=dev())

    def host(self):
        return [x.cpu().numpy().tobytes() for x in (self.th, self.m, self.v, self.p)]


def _combine(rank_stats, out):
    """out <- {sum of sq_norm, max of overflow} over the ranks, on the device."""
    sq = torch.stack([s[0:8].view(torch.float64) for s in rank_stats]).sum(0)
    ov = torch.stack([s[8:12].view(torch.int32) for s in rank_stats]).amax(0)
    out[0:8].view(torch.float64).copy_(sq)
    out[8:12].view(torch.int32).copy_(ov)


def test_ranks_on_streams_equal_the_unsharded_step():
    ranges = [z.zero_partition(PSI, ND, r) for r in range(ND)]
    assert ranges[0][0] == 0 and ranges[-1][1] == PSI
    assert len({b % 8 for b, _ in ranges}) > 3  # several 16-byte phases of the 16-bit arrays

    rng = np.random.default_rng(31)
    th0 = (rng.standard_normal(PSI) * 0.02).astype(np.float32)
    hp = z.adamw(max_grad_norm=1.0, inv_loss_scale=1.0 / 1024)
    whole, ranked = _State(th0), _State(th0)
    whole_state = z.new_adam_state(dev())
    whole_stats = z.new_grad_stats(dev())
    ws_whole = z.new_workspace(PSI, dev())
    streams = [torch.cuda.Stream() for _ in range(ND)]
    rank_stats = [z.new_grad_stats(dev()) for _ in range(ND)]
    rank_comb = [z.new_grad_stats(dev()) for _ in range(ND)]
    rank_state = [z.new_adam_state(dev()) for _ in range(ND)]
    rank_ws = [z.new_workspace(e - b, dev()) for b, e in ranges]
    comb = z.new_grad_stats(dev())
    cur = torch.cuda.current_stream()
    inj_step, inj_rank = 2, 4

    for k in range(5):
        # ||g|| is about 3 after unscaling, so the clip at 1.0 is active
        gb = gen.f32_to_bits16((rng.standard_normal(PSI) * 3e-3 * 1024).astype(np.float32),
                               "f16")
        if k == inj_step:  # one non-finite gradient inside one rank's part
            b, e = ranges[inj_rank]
            gb[(b + e) // 2] = gen.F16_POS_INF
        gt = torch.from_numpy(gb.view(np.int16)).to(dev())
        whole.g.copy_(gt)
        ranked.g.copy_(gt)

        # each rank's statistics on its own stream
        for r, (b, e) in enumerate(ranges):
            streams[r].wait_stream(cur)
            with torch.cuda.stream(streams[r]):
                z.zero_grad_stats(ranked.g[b:e], "f16", e - b, hp.inv_loss_scale, rank_ws[r],
                                  rank_ws[r].numel(), rank_stats[r], stream=streams[r])
        for s in streams:
            cur.wait_stream(s)
        _combine(rank_stats, comb)
        # the combined result goes to every rank and to the unsharded step
        for r in range(ND):
            rank_comb[r].copy_(comb)
        z.zero_grad_stats(whole.g, "f16", PSI, hp.inv_loss_scale, ws_whole, ws_whole.numel(),
                          whole_stats)
        own = z.read_grad_stats(whole_stats)
        whole_stats.copy_(comb)

        # each rank's AdamW on its own stream, the unsharded step on the current one
        for r, (b, e) in enumerate(ranges):
            streams[r].wait_stream(cur)
            with torch.cuda.stream(streams[r]):
                z.zero_adam_step(hp, ranked.g[b:e], "f16", ranked.th[b:e], ranked.m[b:e],
                                 ranked.v[b:e], ranked.p[b:e], "f16", e - b, rank_comb[r],
                                 rank_state[r], stream=streams[r])
        z.zero_adam_step(hp, whole.g, "f16", whole.th, whole.m, whole.v, whole.p, "f16", PSI,
                         whole_stats, whole_state)
        for s in streams:
            cur.wait_stream(s)
        torch.cuda.synchronize()

        c = z.read_grad_stats(comb)
        per_rank = [z.read_grad_stats(s) for s in rank_stats]
        assert [s.overflow for s in per_rank] == [int(k == inj_step and r == inj_rank)
                                                  for r in range(ND)], k
        assert c.overflow == own.overflow == int(k == inj_step)
        if k != inj_step:
            sq_ref, ov_ref = oracle.grad_stats(gb, "f16", hp.inv_loss_scale)
            assert ov_ref == 0
            assert abs(c.sq_norm - sq_ref) <= 1e-9 * sq_ref, (k, c.sq_norm, sq_ref)
            assert abs(own.sq_norm - sq_ref) <= 1e-9 * sq_ref, (k, own.sq_norm, sq_ref)
            assert 4.0 < c.sq_norm < 16.0  # clipping is active
        a, b_ = whole.host(), ranked.host()
        for name, x, y in zip(("master", "m", "v", "param"), a, b_):
            assert x == y, (k, name)
        t_expect = k + 1 - int(k >= inj_step)
        whole_st = z.read_adam_state(whole_state)
        assert whole_st.step == t_expect and whole_st.skip == int(k == inj_step)
        for r in range(ND):
            st = z.read_adam_state(rank_state[r])
            assert st.step == t_expect and st.skip == whole_st.skip, (k, r)
        progress(f"ranks on streams, step {k}: step counter {t_expect}, "
                 f"{'skipped on every rank' if k == inj_step else 'equal to the unsharded step'}")
