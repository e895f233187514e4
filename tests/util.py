"""Helpers shared by the GPU parity tests: phase-controlled device buffers
with canary guard bands, 16-bit ordered distance, and the AdamW comparison
criteria (per-step bounds scaled by the size of each update's terms)."""
import sys

import numpy as np
import torch

CANARY16 = 0x5A5A
CANARY32 = 0x3C3C3C3C
GUARD = 64  # elements of guard band on each side


def dev():
    return torch.device("cuda:0")


class Guarded:
    """A 1-D device buffer of n elements whose first element sits `phase`
    elements past a 256-byte boundary, with canary-filled guard bands."""

    def __init__(self, n, dtype, phase=0, init=None):
        self.n, self.phase, self.dtype = n, phase, dtype
        tdt = {np.uint16: torch.int16, np.float32: torch.float32}[dtype]
        self.es = 2 if dtype == np.uint16 else 4
        self.lead = GUARD + phase
        total = self.lead + n + GUARD
        can = np.full(total, CANARY16 if self.es == 2 else CANARY32,
                      dtype=np.uint16 if self.es == 2 else np.uint32)
        if init is not None:
            can[self.lead:self.lead + n] = np.asarray(init).view(can.dtype)
        self.raw = torch.from_numpy(can.view(np.int16 if self.es == 2 else np.float32)).to(dev())
        assert self.raw.data_ptr() % 256 == 0
        self.t = self.raw[self.lead:self.lead + n]

    def ptr(self):
        return self.raw.data_ptr() + self.lead * self.es

    def host(self):
        a = self.t.cpu().numpy()
        return a.view(np.uint16) if self.es == 2 else a.view(np.float32)

    def canaries_intact(self):
        a = self.raw.cpu().numpy().view(np.uint16 if self.es == 2 else np.uint32)
        c = CANARY16 if self.es == 2 else CANARY32
        return bool((a[:self.lead] == c).all() and (a[self.lead + self.n:] == c).all())


def ordered16(bits):
    b = np.asarray(bits).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ulp16_dist(a, b):
    return np.abs(ordered16(a) - ordered16(b))


def ordered32(x):
    """fp32 values -> integers in value order (adjacent floats differ by 1;
    +0 and -0 both map to 0)."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.int64)
    return np.where(b & 0x80000000, -(b & 0x7FFFFFFF), b)


def ulp32_dist(a, b):
    return np.abs(ordered32(a) - ordered32(b))


def check_params16(p, th, th_ref, dtype, label=""):
    """16-bit params: exactly the round-to-nearest-even of the GPU's own fp32
    master, and within 1 ulp of the oracle's param (the rounding of the
    oracle's master).  Returns how many params differ from the oracle's."""
    import oracle
    exact = oracle.bits16(np.asarray(th, np.float32), dtype)
    if not np.array_equal(p, exact):
        i = int(np.argmax(p != exact))
        raise AssertionError(f"{label} param[{i}] {p[i]:#06x} is not RNE of its master "
                             f"{th[i]!r} ({exact[i]:#06x})")
    p_ref = oracle.bits16(np.asarray(th_ref, np.float32), dtype)
    d = ulp16_dist(p, p_ref)
    if (d > 1).any():
        i = int(np.argmax(d > 1))
        raise AssertionError(f"{label} param[{i}] {p[i]:#06x} vs oracle {p_ref[i]:#06x}: "
                             f"{d[i]} ulp (master {th[i]!r}, oracle master {th_ref[i]!r})")
    return int((d != 0).sum())


def check_adam_one_step(hp, s, g_val, th0, m0, v0, th, m, v, th_ref, m_ref, v_ref, label=""):
    """One step from a common state (th0, m0, v0), both sides with the same
    step scalars: every fp32 result of the GPU (m, v, master) within 1 ulp
    of the oracle's rounding of its fp64 result, which is also within 1e-6
    relative.  Returns, per array, the largest distance in ulps and how many
    elements differ at all."""
    out = {}
    for name, a, r in (("m", m, m_ref), ("v", v, v_ref), ("master", th, th_ref)):
        d = ulp32_dist(a, r)
        if (d > 1).any():
            i = int(np.argmax(d > 1))
            raise AssertionError(f"{label} {name}[{i}]: gpu {a[i]!r} ref {r[i]!r} "
                                 f"({d[i]} ulp apart)")
        out[name] = int(d.max()) if d.size else 0
        out[name + "_differ"] = int((d != 0).sum())
    return out


class FreeRunScales:
    """Shadow recursions that bound how far two independently computed AdamW
    trajectories may drift: M_t = b1 M + (1 - b1)|g_t| for the momentum,
    T_t = (1 - lr wd) T + lr (M_t/bc1)/(sqrt(v_hat)+eps) for the master
    (T_0 = |p_0|); the variance has no cancellation and is compared relative
    to itself.  Two trajectories part where a rounding differs by one ulp (a
    clip coefficient or bias correction that differs in its last fp64 bit),
    and a later step whose terms cancel turns that ulp into a large relative
    error of a small result; it stays small against the size of the terms."""

    def __init__(self, hp, th0):
        self.hp = hp
        self.M = np.zeros(th0.size)
        self.T = np.abs(th0.astype(np.float64))

    def update(self, s, g_val, m_ref, v_ref):
        hp = self.hp
        g = np.abs(g_val) * hp.inv_loss_scale * s.coef
        self.M = hp.beta1 * self.M + (1 - hp.beta1) * g
        upd = (np.maximum(self.M, np.abs(m_ref)) / s.bc1) / \
            (np.sqrt(np.abs(v_ref) / s.bc2) + hp.eps)
        self.T = (1 - hp.lr * hp.weight_decay) * self.T + hp.lr * upd

    def check(self, th, m, v, th_ref, m_ref, v_ref, tol=1e-5, label=""):
        out = {}
        for name, a, r, sc in (("m", m, m_ref, np.maximum(self.M, np.abs(m_ref))),
                               ("v", v, v_ref, np.abs(v_ref)),
                               ("master", th, th_ref, np.maximum(self.T, np.abs(th_ref)))):
            d = np.abs(a.astype(np.float64) - r.astype(np.float64))
            ok = d <= tol * sc
            if not ok.all():
                i = int(np.argmax(~ok))
                raise AssertionError(f"{label} free-running {name}[{i}]: gpu {a[i]!r} "
                                     f"ref {r[i]!r} err {d[i]:.3e} bound {tol * sc[i]:.3e}")
            with np.errstate(divide="ignore", invalid="ignore"):
                out[name] = float(np.nanmax(np.where(sc > 0, d / sc, 0.0))) if d.size else 0.0
            out[name + "_differ"] = int((a.view(np.uint32) != r.view(np.uint32)).sum())
        return out


_reporter = None  # pytest's terminal reporter, set by conftest
_capman = None    # pytest's capture manager, set by conftest


def progress(msg):
    """A progress line that reaches the terminal even while output is captured.
    pytest captures file descriptors 1 and 2 during a test, the terminal
    reporter's own writes included, so capture is suspended around the write."""
    line = f"    [progress] {msg}"
    if _reporter is not None and _capman is not None:
        with _capman.global_and_fixture_disabled():
            _reporter.write_line(line)
            _reporter._tw.flush()
    else:
        print(line, file=sys.stderr, flush=True)
