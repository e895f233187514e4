"""Benchmark of one data-parallel rank's shard-local mixed-precision AdamW step.

A step is one pass of the whole hot path over one batch of synthetic
gradients already resident in HBM:
  zero_partition (host)
  -> zero_bucket_flatten_stats: the rank's per-tensor 16-bit grads gathered
     into the flat grad shard, with the overflow flag and squared norm (fp64)
     computed in the same pass (at Nd = 1 the per-tensor grads are final)
  -> zero_adam_step: fused AdamW on fp32 master/m/v, writes 16-bit params
With --unfused the gather runs once per 500M-element fused buffer
(zero_bucket_flatten) followed by a separate zero_grad_stats pass.
Workload (default): the 13B-parameter GPT-style list (40 layers, hidden 5120,
vocab 50257, bf16 grads and params) at Nd=1, so the rank's shard is all
12,848,143,360 parameters and its whole 16-byte-per-parameter model state
(205.6 GB) is resident in one MI355X's HBM; loss scale 1, no clipping.
--config 2 runs the GPT-2-1.5B-like list (48 layers, hidden 1600, fp16) at
Nd=1 instead (1,557,611,200 parameters, loss scale 2^16, clip 1.0).

Prints one JSON line.  `value` is parameters per second of the whole step
(32 B/param fused, 34 unfused); `step_tensors` times, after it, the step that
reads the per-tensor gradients in place (zero_grad_stats_tensors, then
zero_adam_step_tensors: 30 B/param) on the same workload;
the roofline object covers the fused AdamW kernel (28 algorithmic bytes per
parameter: read grad 2 + master/m/v 12, write master/m/v 12 + param 2).
copy_ceiling times the library's own plain copy of 4 GiB in the same process
after the timed steps, and gives AdamW's and the whole step's bandwidth as
fractions of it.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E
ADAM_BYTES_PER_PARAM = 28
STATS_BYTES_PER_PARAM = 2
FLATTEN_BYTES_PER_PARAM = 4  # 16-bit read + write
METRIC = "Adam-shard params/sec + achieved HBM GB/s vs peak (28 B/param)"
ARITH_DTYPE = "f64"  # the update and the norm are computed in fp64; storage is 16-bit / fp32
TARGET_FRAC = 0.80   # the AdamW step's target fraction of the HBM peak
PROFILES = os.path.join(ROOT, "profiles")
CPU_SAMPLE_CAP = 1_000_000_000  # elements: the largest oracle sample (16 GB of host arrays)
# the AdamW kernel's sources: its own file and the device helpers it includes
KERNEL_SRCS = [os.path.join(ROOT, "zero_sharded_mixed_grads_amd", "csrc", f)
               for f in ("zero_adam.hip", "zero_device.h")]


def kernel_source_hash() -> str:
    """Hash of the AdamW kernel sources' code: line comments, trailing blanks
    and empty lines are dropped, so that editing comments keeps the stored
    counter results valid while any change to the code invalidates them."""
    code = []
    for path in KERNEL_SRCS:
        for line in open(path, encoding="utf-8"):
            line = line.split("//", 1)[0].rstrip()
            if line:
                code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


POOL_CAP = 200 << 30    # bytes: the widest pool the state arrays are spread over
POOL_MARGIN = 8 << 30  # bytes of device memory left free beside the pool


def state_arrays(n: int, dt16, device, spread: bool = True):
    """The five state arrays of an n-element shard (16-bit grad, fp32 master,
    m, v, 16-bit param).  spread: views of one pool, placed by
    zero_state_layout (as far apart as the pool allows; AdamW streams the five
    at once and runs fastest when they lie far apart in HBM).  The pool takes
    the free device memory, capped at POOL_CAP when that holds the arrays
    apart, and leaves POOL_MARGIN free; if it cannot hold the arrays apart,
    or spread is False, they are separate allocations.  Returns the arrays and a description of the layout."""
    import torch
    import zero_sharded_mixed_grads_amd as z
    sizes = (2 * n, 4 * n, 4 * n, 4 * n, 2 * n)
    dts = (dt16, torch.float32, torch.float32, torch.float32, dt16)
    if spread:
        free, _ = torch.cuda.mem_get_info(device)
        most = (free - POOL_MARGIN) // (2 << 20) * (2 << 20)
        offs = None
        # a pool of POOL_CAP bytes if it holds the arrays apart, else the
        # largest one that fits (the 13B shard's 206 GB of state)
        for pool_bytes in (min(POOL_CAP, most), most):
            try:
                offs = z.zero_state_layout(n, pool_bytes)
                break
            except z.ZeroError:
                continue
        pool = None
        if offs is not None:
            try:
                pool = torch.empty(pool_bytes, dtype=torch.uint8, device=device)
            except torch.OutOfMemoryError:
                log(f"[bench] no {pool_bytes} B pool available; separate allocations")
        if pool is not None:
            arrays = [pool[o:o + nb].view(dt) for o, nb, dt in zip(offs, sizes, dts)]
            return (*arrays, {"kind": "spread", "pool_bytes": pool_bytes,
                              "spacing_bytes": offs[1]})
    arrays = [torch.empty(nb // (2 if dt != torch.float32 else 4), dtype=dt, device=device)
              for nb, dt in zip(sizes, dts)]
    return (*arrays, {"kind": "separate"})


class Workload:
    def __init__(self, cfg_idx: int, device, spread: bool = True):
        import torch
        import zero_sharded_mixed_grads_amd as z
        from synth import WORKLOADS, gen

        self.z, self.torch = z, torch
        self.cfg_idx = cfg_idx
        cfg = self.cfg = WORKLOADS[cfg_idx]
        self.dev = device
        self.begin, self.end = z.zero_partition(cfg.psi, cfg.nd, cfg.rank)
        n = self.n = self.end - self.begin
        tdt = gen.torch_dtype(cfg.dtype)
        log(f"[bench] workload {cfg.name}: psi={cfg.psi} nd={cfg.nd} rank={cfg.rank} n={n}")
        t0 = time.time()
        # per-tensor gradients as backward would leave them (only those in the shard)
        plan = z.zero_bucket_plan(cfg.numels, cfg.psi, self.begin, self.end)
        self.tensor_ids = sorted({s[1] for s in plan})
        self.grads = [None] * len(cfg.numels)
        for i in self.tensor_ids:
            t = torch.empty(cfg.numels[i], dtype=tdt, device=device)
            gen.device_fill_normal_(t, cfg.grad_seed(0) * 100003 + i, cfg.grad_sigma,
                                    cfg.loss_scale)
            self.grads[i] = t
        # the five state arrays: flat grad shard, master, m, v, param shard
        self.g, self.master, self.m, self.v, self.p, self.layout = state_arrays(
            n, tdt, device, spread)
        gen.device_fill_normal_(self.master, cfg.master_seed(), cfg.master_sigma)
        self.m.zero_()
        self.v.zero_()
        self.stats = z.new_grad_stats(device)
        self.state = z.new_adam_state(device)
        self.ws = z.new_workspace(n, device)
        nb = z.zero_bucket_flatten_stats_workspace(cfg.numels, self.begin, n)
        self.fws = torch.empty(nb, dtype=torch.uint8, device=device)
        self.hp = z.adamw(**cfg.hp.__dict__)
        # the gradient table, marshalled once (self.grads keeps the tensors alive)
        self.ptrs, self.numels = z.tensor_table(
            [t.data_ptr() if t is not None else None for t in self.grads], cfg.numels)
        torch.cuda.synchronize()
        log(f"[bench] inputs resident in HBM after {time.time() - t0:.1f}s "
            f"({torch.cuda.memory_allocated() / 1e9:.1f} GB allocated)")

    def step_tensors(self, marks=None):
        """The step read from the per-tensor gradients in place (the rank's
        per-tensor gradients are final at Nd = 1): statistics, then AdamW,
        with no gathered shard.  marks: optional one event recorded between
        the two."""
        z, cfg = self.z, self.cfg
        stream = self.torch.cuda.current_stream()
        s = stream.cuda_stream
        b, e = z.zero_partition(cfg.psi, cfg.nd, cfg.rank)
        z.zero_grad_stats_tensors(self.ptrs, self.numels, cfg.dtype, b, e - b,
                                  cfg.hp.inv_loss_scale, self.fws, self.fws.numel(), self.stats, s)
        if marks: marks[0].record(stream)
        z.zero_adam_step_tensors(self.hp, self.ptrs, self.numels, cfg.dtype, b, e - b, self.master,
                                 self.m, self.v, self.p, cfg.dtype, self.stats, self.state, s)

    def step(self, marks=None, fused=True):
        """One pass of the hot path.  fused: gather the rank's gradients and
        compute their statistics in one pass (the rank's per-tensor gradients
        are final at Nd = 1); otherwise gather one fused buffer at a time, then
        a separate statistics pass.  marks: optional events recorded on the
        launch stream between the phases: after the gather and statistics
        (fused, one event), or after the gather and after the statistics
        (unfused, two events)."""
        z, cfg = self.z, self.cfg
        stream = self.torch.cuda.current_stream()
        s = stream.cuda_stream
        b, e = z.zero_partition(cfg.psi, cfg.nd, cfg.rank)
        B = cfg.bucket_elems or cfg.psi
        if fused:
            z.zero_bucket_flatten_stats(self.ptrs, self.numels, cfg.dtype, b, e - b, self.g,
                                        cfg.hp.inv_loss_scale, self.fws, self.fws.numel(),
                                        self.stats, s)
        else:
            lo = b
            while lo < e:  # one fused buffer at a time, this rank's part of it
                hi = min((lo // B + 1) * B, e)
                z.zero_bucket_flatten(self.ptrs, self.numels, cfg.dtype, lo, hi - lo,
                                      self.g.data_ptr() + 2 * (lo - b), s)
                lo = hi
            if marks: marks[0].record(stream)
            z.zero_grad_stats(self.g, cfg.dtype, self.n, cfg.hp.inv_loss_scale, self.ws,
                              self.ws.numel(), self.stats, s)
        if marks: marks[-1].record(stream)
        z.zero_adam_step(self.hp, self.g, cfg.dtype, self.master, self.m, self.v, self.p,
                         cfg.dtype, self.n, self.stats, self.state, s)


def _host_bits(t, np_dt):
    """A host copy of a device tensor's bits, viewed as np_dt (numpy has no
    bfloat16, so 16-bit tensors travel as int16)."""
    import torch
    if t.element_size() == 2:
        t = t.view(torch.int16)
    return t.cpu().numpy().view(np_dt).copy()


def cpu_baseline(w, target_s: float = 12.0):
    """The oracle, as it is, on a bounded contiguous sample of the same shard
    (copied to host memory): grad stats + AdamW.  The sample is sized for
    about target_s seconds of work, capped at the whole shard and at
    CPU_SAMPLE_CAP elements, and repeated until target_s seconds have passed."""
    import oracle
    cfg = w.cfg

    def host(t, k, np_dt):
        return _host_bits(t[:k], np_dt)

    def once(gb, th, m, v, p):
        t0 = time.perf_counter()
        sq, ov = oracle.grad_stats(gb, cfg.dtype, cfg.hp.inv_loss_scale)
        s = oracle.step_scalars(cfg.hp, True, sq, ov, 0)
        oracle.adamw_(s, gb, cfg.dtype, th, m, v, p, cfg.dtype)
        return time.perf_counter() - t0

    def arrays(k):
        return (host(w.g, k, np.uint16), host(w.master, k, np.float32), host(w.m, k, np.float32),
                host(w.v, k, np.float32), np.zeros(k, np.uint16))

    k = min(w.n, 1 << 22)
    dt = once(*arrays(k))
    k = int(min(w.n, CPU_SAMPLE_CAP, max(k, k * target_s / max(dt, 1e-6))))
    a = arrays(k)
    total, reps = 0.0, 0
    while total < target_s:
        total += once(*a)
        reps += 1
    return {"value": k * reps / total, "unit": "params/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"first {k} elements of the same shard in host memory, fp64 grad stats "
                      f"+ AdamW, {reps} pass(es) in {total:.1f} s"}


_ONE_THREAD_SCRIPT = """
import json, sys, time
import numpy as np
sys.path.insert(0, sys.argv[1])
import oracle
from synth import WORKLOADS
cfg = WORKLOADS[int(sys.argv[2])]
a = np.load(sys.argv[3])
g, th, m, v, p = (a[k].copy() for k in ("g", "th", "m", "v", "p"))
total, reps = 0.0, 0
while total < float(sys.argv[4]):
    t0 = time.perf_counter()
    sq, ov = oracle.grad_stats(g, cfg.dtype, cfg.hp.inv_loss_scale)
    s = oracle.step_scalars(cfg.hp, True, sq, ov, 0)
    oracle.adamw_(s, g, cfg.dtype, th, m, v, p, cfg.dtype)
    total += time.perf_counter() - t0
    reps += 1
print(json.dumps({"threads": oracle.num_threads(), "n": int(g.size), "reps": reps, "s": total}))
"""


def cpu_baseline_one_thread(w, k: int = 1 << 24, target_s: float = 4.0):
    """The same oracle pass on one host thread (a child process started with
    OMP_NUM_THREADS=1), on the first k elements of the shard, repeated for
    about target_s seconds; plus the host's CPU model and memory."""
    import subprocess
    import tempfile
    k = min(k, w.n)

    def host(t, np_dt):
        return _host_bits(t[:k], np_dt)

    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "sample.npz")
        np.savez(path, g=host(w.g, np.uint16), th=host(w.master, np.float32),
                 m=host(w.m, np.float32), v=host(w.v, np.float32), p=np.zeros(k, np.uint16))
        env = dict(os.environ, OMP_NUM_THREADS="1")
        out = subprocess.run([sys.executable, "-c", _ONE_THREAD_SCRIPT, ROOT, str(w.cfg_idx), path,
                              str(target_s)], env=env, capture_output=True, text=True,
                             timeout=300, check=True).stdout
    r = json.loads(out.strip().splitlines()[-1])
    cpu = next((l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
                if l.startswith("model name")), "unknown")
    mem_kb = next((int(l.split()[1]) for l in open("/proc/meminfo") if l.startswith("MemTotal")), 0)
    return {"value": r["n"] * r["reps"] / r["s"], "unit": "params/s", "cores": r["threads"],
            "kind": "oracle",
            "sample": f"first {r['n']} elements of the same shard, fp64 grad stats + AdamW, "
                      f"{r['reps']} pass(es) in {r['s']:.1f} s",
            "host_cpu": cpu, "host_mem_gb": round(mem_kb / 1e6, 1)}


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"adamw_stream_{workload}_traffic.json")


def load_traffic(workload: str, n_params: int):
    """HBM bytes per AdamW launch on this workload from the committed
    rocprofv3 counter runs, or None if there are none for it or the kernel
    source changed since they were taken."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_source_sha256_16") != kernel_source_hash() or d.get("n") != n_params:
        return None
    return d.get("bytes_per_launch")


def time_tensor_step(w, steps: int, warmup: int):
    """Times `steps` passes of the 30 B/param step (statistics read in place,
    then AdamW reading the per-tensor gradients) on the same workload, after
    `warmup` untimed ones; every step must be a real update."""
    import torch
    taken0 = w.z.read_adam_state(w.state).step
    for _ in range(warmup):
        w.step_tensors()
    stream = torch.cuda.current_stream()
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks = [[torch.cuda.Event(enable_timing=True)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    bounds[0].record(stream)
    for k in range(steps):
        w.step_tensors(marks[k])
        bounds[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = w.z.read_adam_state(w.state)
    if st.step != taken0 + warmup + steps:
        raise SystemExit("bench: a step of the in-place step was skipped; timing invalid")
    ms = np.array([[bounds[k].elapsed_time(marks[k][0]), marks[k][0].elapsed_time(bounds[k + 1])]
                   for k in range(steps)])
    stats_ms, adam_ms = ms.mean(axis=0)
    step_ms = wall * 1e3 / steps
    n = w.n
    log(f"[bench] in-place step: {step_ms:.3f} ms/step (stats {stats_ms:.3f} ms, "
        f"adam {adam_ms:.3f} ms)")
    return {"steps": steps, "ms_per_step": step_ms, "params_per_s": n / (step_ms * 1e-3),
            "bytes_per_param": ADAM_BYTES_PER_PARAM + STATS_BYTES_PER_PARAM,
            "kernels": {"grad_stats_tensors": {"ms": stats_ms,
                                               "GB/s": STATS_BYTES_PER_PARAM * n / stats_ms / 1e6},
                        "adam_step_tensors": {"ms": adam_ms,
                                              "GB/s": ADAM_BYTES_PER_PARAM * n / adam_ms / 1e6,
                                              "frac": ADAM_BYTES_PER_PARAM * n / adam_ms / 1e6
                                              / HBM_PEAK_GBS}}}


def copy_ceiling(device, reps: int = 20):
    """The part's streaming ceiling for a read + write mix, measured in this
    process: the library's own gather of one aligned 4 GiB fp32 tensor (a
    plain copy with the path's 16-byte access pattern), median of reps calls.
    None when the device has no room for the two buffers."""
    import torch
    import zero_sharded_mixed_grads_amd as z
    n = 1 << 30
    try:
        src = torch.empty(n, dtype=torch.float32, device=device)
        dst = torch.empty_like(src)
    except torch.OutOfMemoryError:
        return None
    src.fill_(1.0)
    for _ in range(3):
        z.zero_bucket_flatten([src], [n], "f32", 0, n, dst)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(reps):
        z.zero_bucket_flatten([src], [n], "f32", 0, n, dst)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([evs[i].elapsed_time(evs[i + 1]) for i in range(reps)]))
    del src, dst
    torch.cuda.empty_cache()
    return {"kernel": "zero_bucket_flatten of one aligned 4 GiB fp32 tensor (a plain copy)",
            "ms": ms, "GB/s": 8 * n / (ms * 1e-3) / 1e9}


def copy_probe(steps: int):
    """Streaming kernels of a known size: plain copies (the achievable ceiling
    for a read + write mix like the AdamW step, and the reference dispatch for
    calibrating the HBM byte counters), plus a write-only fill, an in-place
    read-modify-write and a read-only pass.  Prints one JSON line."""
    import torch
    n = 1 << 30  # fp32 elements: 4 GiB read + 4 GiB written per copy
    src = torch.empty(n, dtype=torch.float32, device="cuda:0").normal_()
    dst = torch.empty_like(src)
    import zero_sharded_mixed_grads_amd as z
    res = {}
    g16 = src.view(torch.float16)  # the same 4 GiB read as 2^31 fp16 gradients
    stats = z.new_grad_stats(src.device)
    ws = z.new_workspace(g16.numel(), src.device)
    nb = 4 * n
    for name, fn, rd, wr in (
            ("copy_", lambda: dst.copy_(src), nb, nb),
            ("mul_out", lambda: torch.mul(src, 1.0, out=dst), nb, nb),
            # the library's own gather of one aligned fp32 tensor: a plain copy
            # with the same 16-byte load/store pattern as the path's kernels
            ("zero_bucket_flatten", lambda: z.zero_bucket_flatten([src], [n], "f32", 0, n, dst),
             nb, nb),
            # other access mixes: write only, read and write back in place (as
            # AdamW does to master, m and v), and read only (the library's
            # statistics pass over the buffer as fp16 gradients, and torch's sum)
            ("fill_", lambda: dst.fill_(1.0), 0, nb),
            ("mul_ in place", lambda: dst.mul_(1.0), nb, nb),
            ("zero_grad_stats", lambda: z.zero_grad_stats(g16, "f16", g16.numel(), 1.0, ws,
                                                          ws.numel(), stats), nb, 0),
            ("sum", lambda: torch.sum(src), nb, 0)):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        res[name] = {"ms": ms, "GB/s": (rd + wr) / (ms * 1e-3) / 1e9,
                     "bytes_read": rd, "bytes_written": wr}
    print(json.dumps({"copy_probe": res}), flush=True)


def time_calls(fn, nbytes: int, steps: int, warmup: int) -> dict:
    """Median and minimum of `steps` HIP-event-timed calls of fn after `warmup`
    untimed ones, with the bandwidth that moving nbytes per call gives."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = []
    for _ in range(steps):
        a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        c.record()
        evs.append((a, c))
    torch.cuda.synchronize()
    ms = sorted(x.elapsed_time(y) for x, y in evs)
    med = ms[len(ms) // 2]
    return {"ms_median": med, "ms_min": ms[0], "GB/s": nbytes / med / 1e6,
            "frac": nbytes / med / 1e6 / HBM_PEAK_GBS}


def time_calls_alternating(fns: dict, nbytes: int, steps: int, warmup: int) -> dict:
    """time_calls for several calls at once, alternating them call by call
    (a, b, a, b, ...) so that each sees the same state of the part."""
    import torch
    for _ in range(warmup):
        for fn in fns.values():
            fn()
    torch.cuda.synchronize()
    evs = {k: [] for k in fns}
    for _ in range(steps):
        for k, fn in fns.items():
            a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            c.record()
            evs[k].append((a, c))
    torch.cuda.synchronize()
    out = {}
    for k, pairs in evs.items():
        ms = sorted(x.elapsed_time(y) for x, y in pairs)
        med = ms[len(ms) // 2]
        out[k] = {"ms_median": med, "ms_min": ms[0], "GB/s": nbytes / med / 1e6,
                  "frac": nbytes / med / 1e6 / HBM_PEAK_GBS}
    return out


def configs_sweep(steps: int, warmup: int, spread: bool = True, which=(2, 3, 4, 5)):
    """zero_grad_stats and zero_adam_step timed alone on the flat shard of each
    workload of at least 100M parameters (1.5B at Nd 1, 7.5B rank 3 of 8, 13B
    at Nd 1, 100B rank 399 of 400), with the 16-bit arrays at the element
    phase the shard has in the flat layout (for a shard off phase 0, AdamW
    again on the same arrays with the 16-bit views at phase 0); then a skipped
    (overflowing) step, and the fused gather + statistics of the shard from
    its per-tensor gradients.  Prints one JSON line."""
    import torch
    import zero_sharded_mixed_grads_amd as z
    from synth import WORKLOADS, gen
    dev = torch.device("cuda:0")
    out = {}
    for idx in which:
        cfg = WORKLOADS[idx]
        b, e = z.zero_partition(cfg.psi, cfg.nd, cfg.rank)
        n, ph = e - b, b % 8
        tdt = gen.torch_dtype(cfg.dtype)
        gbuf, master, m, v, pbuf, layout = state_arrays(n + 8, tdt, dev, spread)
        g, p = gbuf[ph:ph + n], pbuf[ph:ph + n]
        master, m, v = master[:n], m[:n], v[:n]
        # every element of gbuf finite: its phase-0 view is timed too
        gen.device_fill_normal_(gbuf, cfg.grad_seed(0), cfg.grad_sigma, cfg.loss_scale)
        gen.device_fill_normal_(master, cfg.master_seed(), cfg.master_sigma)
        m.zero_()
        v.zero_()
        stats, state = z.new_grad_stats(dev), z.new_adam_state(dev)
        ws = z.new_workspace(n, dev)
        hp = z.adamw(**cfg.hp.__dict__)
        calls = {
            "grad_stats": lambda: z.zero_grad_stats(g, cfg.dtype, n, cfg.hp.inv_loss_scale, ws,
                                                    ws.numel(), stats),
            "adam_step": lambda: z.zero_adam_step(hp, g, cfg.dtype, master, m, v, p, cfg.dtype,
                                                  n, stats, state),
        }
        res = {"n": n, "dtype": cfg.dtype, "phase16": ph, "state_layout": layout}
        res["grad_stats"] = time_calls(calls["grad_stats"], STATS_BYTES_PER_PARAM * n, steps,
                                       warmup)
        if ph:
            # the same arrays with the 16-bit views moved to phase 0, timed call
            # by call in turn with the shard's own phase: what the realigning
            # variant costs on these buffers
            g0, p0 = gbuf[:n], pbuf[:n]
            res.update(time_calls_alternating(
                {"adam_step": calls["adam_step"],
                 "adam_step_phase0": lambda: z.zero_adam_step(hp, g0, cfg.dtype, master, m, v,
                                                              p0, cfg.dtype, n, stats, state)},
                ADAM_BYTES_PER_PARAM * n, steps, warmup))
            del g0, p0
        else:
            res["adam_step"] = time_calls(calls["adam_step"], ADAM_BYTES_PER_PARAM * n, steps,
                                          warmup)
        st = z.read_adam_state(state)
        expect = (warmup + steps) * (2 if ph else 1)
        if st.skip or st.step != expect:
            raise SystemExit(f"{cfg.name}: a step was skipped; timing would be invalid")
        # the skip path: one non-finite gradient, then AdamW writes nothing
        g[0] = float("inf")
        calls["grad_stats"]()
        ms = []
        for _ in range(steps):
            a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            calls["adam_step"]()
            c.record()
            ms.append((a, c))
        torch.cuda.synchronize()
        ms = sorted(x.elapsed_time(y) for x, y in ms)
        st = z.read_adam_state(state)
        if not st.skip or st.step != expect:
            raise SystemExit(f"{cfg.name}: the overflowing steps were not skipped")
        res["adam_step_skipped"] = {"ms_median": ms[len(ms) // 2], "ms_min": ms[0]}
        # the fused gather + statistics of the shard from its per-tensor gradients,
        # each tensor that meets the shard in an allocation of its own
        starts = np.cumsum([0] + list(cfg.numels))
        which = [i for i in range(len(cfg.numels)) if starts[i] < e and starts[i + 1] > b]
        try:
            grads = gen.device_grad_list(cfg, 1, dev, which)
        except torch.OutOfMemoryError:
            grads = None
            res["gather_stats"] = "not measured: no room for the per-tensor gradients"
        if grads is not None:
            ptrs, nums = z.tensor_table([grads.get(i) for i in range(len(cfg.numels))],
                                        cfg.numels)
            fws_n = z.zero_bucket_flatten_stats_workspace(nums, b, n)
            fws = torch.empty(fws_n, dtype=torch.uint8, device=dev)

            def gather():
                z.zero_bucket_flatten_stats(ptrs, nums, cfg.dtype, b, n, g,
                                            cfg.hp.inv_loss_scale, fws, fws_n, stats)
            for _ in range(warmup):
                gather()
            torch.cuda.synchronize()
            evs = []
            for _ in range(steps):
                a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                gather()
                c.record()
                evs.append((a, c))
            torch.cuda.synchronize()
            ms = sorted(x.elapsed_time(y) for x, y in evs)
            med = ms[len(ms) // 2]
            res["gather_stats"] = {"tensors": len(which), "ms_median": med, "ms_min": ms[0],
                                   "GB/s": FLATTEN_BYTES_PER_PARAM * n / med / 1e6,
                                   "frac": FLATTEN_BYTES_PER_PARAM * n / med / 1e6 / HBM_PEAK_GBS}
            del grads, ptrs, nums, fws
        out[cfg.name] = res
        gs = res["gather_stats"]
        ph0 = (f"; at phase 0 {res['adam_step_phase0']['ms_median']:.3f} ms"
               if ph else "")
        log(f"[bench] {cfg.name}: n={n} adam {res['adam_step']['ms_median']:.3f} ms "
            f"({res['adam_step']['GB/s']:.0f} GB/s{ph0}); gather+stats "
            + (f"{gs['ms_median']:.3f} ms ({gs['GB/s']:.0f} GB/s, {gs['tensors']} tensors)"
               if isinstance(gs, dict) else gs))
        del gbuf, pbuf, g, p, master, m, v, ws, calls
        torch.cuda.empty_cache()
    print(json.dumps({"configs": out}), flush=True)


def ckpt_bench(cfg_idx: int = 5, reps: int = 2):
    """Checkpoint save and load of one rank's optimizer state (fp32 master, m,
    v) to the local temporary directory: save, then load into fresh arrays and
    compare bit for bit.  The state has the size of the 100B model's rank 399
    of 400 (250,728,263 params, 3.0 GB); it is saved as the single shard of a
    run of that size (Nd = 1), because a load needs every shard of a save and
    400 such files do not fit a local disk.  Prints one JSON line."""
    import shutil
    import tempfile
    import torch
    import zero_sharded_mixed_grads_amd as z
    from synth import WORKLOADS, gen
    cfg = WORKLOADS[cfg_idx]
    dev = torch.device("cuda:0")
    b, e = z.zero_partition(cfg.psi, cfg.nd, cfg.rank)
    n = e - b
    tmp = tempfile.mkdtemp(prefix="zero_ckpt_")
    need = 12 * n + 64
    if shutil.disk_usage(tmp).free < 2 * need:
        shutil.rmtree(tmp)
        print(json.dumps({"ckpt": {"skipped": f"less than {2 * need} bytes free in {tmp}"}}))
        return
    src = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(3)]
    for i, t in enumerate(src):
        gen.device_fill_normal_(t, cfg.master_seed() + i, 0.02)
    state = z.new_adam_state(dev)
    dst = [torch.empty_like(t) for t in src]
    state2 = z.new_adam_state(dev)
    path = os.path.join(tmp, "shard.zck")
    save_s, load_s = [], []
    try:
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            z.zero_ckpt_save(path, n, 1, 0, *src, state)
            save_s.append(time.perf_counter() - t0)
            t0 = time.perf_counter()
            z.zero_ckpt_load([path], n, 1, 0, *dst, state2)
            load_s.append(time.perf_counter() - t0)
        same = all(torch.equal(a.view(torch.int32), c.view(torch.int32))
                   for a, c in zip(src, dst))
    finally:
        shutil.rmtree(tmp)
    if not same:
        raise SystemExit("checkpoint round trip changed the state")
    by = 12 * n
    print(json.dumps({"ckpt": {"workload": f"{cfg.name} state as one shard",
                               "shard_params": n, "bytes": by,
                               "save_s": min(save_s), "load_s": min(load_s),
                               "save_GB/s": by / min(save_s) / 1e9,
                               "load_GB/s": by / min(load_s) / 1e9,
                               "round_trip_bit_exact": same}}), flush=True)


def host_stream_ceiling(reps: int = 5):
    """Host memory bandwidth with torch's intra-op threads on 4 GiB fp32 arrays,
    well beyond the host caches: an in-place scale (each element read and
    written back, as the offloaded update does to master, m and v) and an
    out-of-place copy (counted as 8 B per element, though its stores first
    read their lines for ownership).  Returns the best of `reps` passes of
    each, in GB/s."""
    import torch
    n = 1 << 30
    a = torch.ones(n, dtype=torch.float32)
    b = torch.empty_like(a)
    out = {"threads": torch.get_num_threads()}
    for name, fn in (("copy", lambda: torch.mul(a, 1.0, out=b)), ("in_place", lambda: a.mul_(1.0))):
        fn()
        best = min(_host_time(fn) for _ in range(reps))
        out[f"{name}_GB/s"] = 2 * 4 * n / best / 1e9
    return out


def _host_time(fn):
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


def offload_bench(cfg_idx: int, steps: int, warmup: int, chunk: int = 1 << 24):
    """The optimizer step with master/m/v in host memory (zero_offload_adam_step)
    on the same shard: gradients and params on the device, statistics on the
    device, AdamW on the host cores.  Prints one JSON line."""
    import torch
    import zero_sharded_mixed_grads_amd as z
    from synth import WORKLOADS, gen
    cfg = WORKLOADS[cfg_idx]
    dev = torch.device("cuda:0")
    b, e = z.zero_partition(cfg.psi, cfg.nd, cfg.rank)
    n = e - b
    g = torch.empty(n, dtype=gen.torch_dtype(cfg.dtype), device=dev)
    gen.device_fill_normal_(g, cfg.grad_seed(0), cfg.grad_sigma, cfg.loss_scale)
    p = torch.empty_like(g)
    dm = torch.empty(n, dtype=torch.float32, device=dev)
    gen.device_fill_normal_(dm, cfg.master_seed(), cfg.master_sigma)
    master = dm.cpu()
    del dm
    m, v = torch.zeros(n), torch.zeros(n)
    stats, state = z.new_grad_stats(dev), z.new_adam_state(dev)
    ws = z.new_workspace(n, dev)
    nb = z.zero_offload_staging_bytes(chunk)
    stg = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
    hp = z.adamw(**cfg.hp.__dict__)
    log(f"[bench] offload: n={n}, state {12 * n / 1e9:.1f} GB in host memory, "
        f"chunks of {chunk} elements")

    def step():
        z.zero_grad_stats(g, cfg.dtype, n, cfg.hp.inv_loss_scale, ws, ws.numel(), stats)
        z.zero_offload_adam_step(hp, g, cfg.dtype, master, m, v, p, cfg.dtype, n, stats, state,
                                 stg, nb)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    st = z.read_adam_state(state)
    if st.step != warmup + steps:
        print("bench: offloaded steps were skipped; the measurement is invalid", file=sys.stderr)
        sys.exit(3)
    cpu = next((l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
                if l.startswith("model name")), "unknown")
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    del master, m, v
    log("[bench] host memory ceiling")
    ceiling = host_stream_ceiling()
    # host DRAM bytes per param: master, m, v read and written (24), the staged
    # gradient written by DMA and read (4), the staged param written and read by DMA (4)
    host_gbs = 32 * n / (ms * 1e-3) / 1e9
    print(json.dumps({"offload": {
        "workload": cfg.name + f"-nd{cfg.nd}-rank{cfg.rank}", "shard_params": n,
        "steps": steps, "warmup": warmup, "ms_per_step": ms, "params_per_s": n / (ms * 1e-3),
        "pcie_GB/s": 4 * n / (ms * 1e-3) / 1e9,
        "host_state_GB/s": 24 * n / (ms * 1e-3) / 1e9,
        "host_dram_GB/s": host_gbs, "host_ceiling": ceiling,
        "frac_of_host_in_place": host_gbs / ceiling["in_place_GB/s"],
        "chunk_elems": chunk, "host_threads": threads, "host_cpu": cpu}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, choices=(1, 2, 3, 4, 5),
                    help="workload: 4 = 13B list at Nd 1 (default), 2 = GPT-2 1.5B list at "
                         "Nd 1, 3 = 7.5B rank 3 of 8, 5 = 100B rank 399 of 400, 1 = the tiny "
                         "ragged list (rank 0 of 4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="time plain device copies of a known size instead")
    ap.add_argument("--unfused", action="store_true",
                    help="gather per fused buffer, then a separate statistics pass")
    ap.add_argument("--offload", action="store_true",
                    help="time the step with the optimizer state in host memory instead")
    ap.add_argument("--chunk", type=int, default=1 << 24,
                    help="with --offload: elements per pinned staging slot")
    ap.add_argument("--ckpt", action="store_true",
                    help="time a sharded checkpoint save and load of one rank's state instead")
    ap.add_argument("--separate", action="store_true",
                    help="allocate the five state arrays separately instead of spreading "
                         "them over one pool")
    ap.add_argument("--configs", nargs="*", type=int, default=None,
                    help="time grad stats and AdamW alone on every workload of >= 100M params "
                         "(2 3 4 5), or on those listed")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one data-parallel rank's shard on one GPU; it does not "
              "run on more than one GPU (the exchanges between ranks are not implemented)",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.steps)
        return
    if args.offload:
        offload_bench(args.config, args.steps, args.warmup, chunk=args.chunk)
        return
    if args.ckpt:
        ckpt_bench()
        return
    if args.configs is not None:
        bad = [i for i in args.configs if i not in (2, 3, 4, 5)]
        if bad:
            ap.error(f"--configs takes workloads 2 3 4 5, not {bad}")
        configs_sweep(args.steps, args.warmup, spread=not args.separate,
                      which=tuple(args.configs) or (2, 3, 4, 5))
        return

    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = Workload(args.config, dev, spread=not args.separate)

    fused = not args.unfused
    for _ in range(args.warmup):
        w.step(fused=fused)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done")

    # HIP events on the launch stream: one at each step boundary (shared by
    # consecutive steps) and one (fused) or two (unfused) between the phases
    def event():
        return torch.cuda.Event(enable_timing=True)
    bounds = [event() for _ in range(args.steps + 1)]
    marks = [[event() for _ in range(1 if fused else 2)] for _ in range(args.steps)]
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    bounds[0].record(stream)
    for k in range(args.steps):
        w.step(marks[k], fused=fused)
        bounds[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per step: gather (+ stats when fused), stats (unfused), adam
    ms = np.array([[bounds[k].elapsed_time(marks[k][0]),
                    marks[k][0].elapsed_time(marks[k][-1]),
                    marks[k][-1].elapsed_time(bounds[k + 1])] for k in range(args.steps)])
    flat_ms, stats_ms, adam_ms = ms.mean(axis=0)
    log(f"[bench] timed {args.steps} steps in {wall:.3f}s ({'fused' if fused else 'unfused'}); "
        f"per step gather {flat_ms:.3f} ms, stats {stats_ms:.3f} ms, adam {adam_ms:.3f} ms "
        f"(adam min {ms[:, 2].min():.3f} max {ms[:, 2].max():.3f})")
    # every step must have been a real update: the device step counter counts them
    st = w.z.read_adam_state(w.state)
    gs = w.z.read_grad_stats(w.stats)
    taken = args.warmup + args.steps
    if st.step != taken or gs.overflow:
        print(f"bench: {taken - st.step} of {taken} steps were skipped (overflow={gs.overflow}); "
              "the measurement is invalid", file=sys.stderr)
        sys.exit(3)

    n = w.n
    step_ms = wall * 1e3 / args.steps
    kernels = {"adam_step": {"ms": adam_ms, "ms_min": float(ms[:, 2].min()),
                             "ms_max": float(ms[:, 2].max()), "params_per_s": n / (adam_ms * 1e-3),
                             "GB/s": ADAM_BYTES_PER_PARAM * n / (adam_ms * 1e-3) / 1e9,
                             "bytes_per_param": ADAM_BYTES_PER_PARAM}}
    if fused:  # gather + statistics in one pass: 2 B read + 2 B written per param
        kernels["bucket_flatten_stats"] = {
            "ms": flat_ms, "GB/s": FLATTEN_BYTES_PER_PARAM * n / (flat_ms * 1e-3) / 1e9,
            "bytes_per_param": FLATTEN_BYTES_PER_PARAM}
        step_bytes = ADAM_BYTES_PER_PARAM + FLATTEN_BYTES_PER_PARAM
    else:
        kernels["bucket_flatten"] = {
            "ms": flat_ms, "GB/s": FLATTEN_BYTES_PER_PARAM * n / (flat_ms * 1e-3) / 1e9,
            "bytes_per_param": FLATTEN_BYTES_PER_PARAM}
        kernels["grad_stats"] = {
            "ms": stats_ms, "GB/s": STATS_BYTES_PER_PARAM * n / (stats_ms * 1e-3) / 1e9,
            "bytes_per_param": STATS_BYTES_PER_PARAM}
        step_bytes = ADAM_BYTES_PER_PARAM + STATS_BYTES_PER_PARAM + FLATTEN_BYTES_PER_PARAM
    adam_gbs = ADAM_BYTES_PER_PARAM * n / (adam_ms * 1e-3) / 1e9
    workload = w.cfg.name + f"-nd{w.cfg.nd}-rank{w.cfg.rank}"
    traffic = load_traffic(workload, n)
    out = {
        "metric": METRIC,
        "value": n / (step_ms * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ARITH_DTYPE,
        "data": "synthetic",
        "config": {"workload": workload, "psi": w.cfg.psi,
                   "nd": w.cfg.nd, "rank": w.cfg.rank, "shard_params": n,
                   "grad_dtype": w.cfg.dtype, "param_dtype": w.cfg.dtype,
                   "bucket_elems": w.cfg.bucket_elems, "max_grad_norm": w.cfg.hp.max_grad_norm,
                   "loss_scale": w.cfg.loss_scale, "state_dtype": "f32",
                   "state_layout": w.layout},
        "roofline": {"bound": "hbm", "achieved": adam_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": adam_gbs / HBM_PEAK_GBS, "traffic": traffic},
        "target": {"what": "AdamW fraction of the 8 TB/s HBM peak", "frac": TARGET_FRAC,
                   "met": bool(adam_gbs / HBM_PEAK_GBS >= TARGET_FRAC)},
        "kernels": kernels,
        "step_bytes_per_param": step_bytes,
        "checks": {"device_steps_taken": int(st.step), "overflow": int(gs.overflow),
                   "sq_norm": gs.sq_norm, "clip_coef": st.coef},
    }
    # the step read from the per-tensor gradients in place, timed the same way
    out["step_tensors"] = time_tensor_step(w, min(args.steps, 20), args.warmup)
    # the same process's copy ceiling, for the fraction of what a plain copy reaches
    cc = copy_ceiling(dev)
    if cc is not None:
        cc["adam_frac_of_copy"] = adam_gbs / cc["GB/s"]
        cc["step_frac_of_copy"] = step_bytes * n / (step_ms * 1e-3) / 1e9 / cc["GB/s"]
        log(f"[bench] copy ceiling {cc['GB/s']:.0f} GB/s; AdamW at "
            f"{cc['adam_frac_of_copy']:.3f} of it")
    out["copy_ceiling"] = cc
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(w)
        log("[bench] timing the oracle on one host thread")
        out["cpu_baseline_one_thread"] = cpu_baseline_one_thread(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
