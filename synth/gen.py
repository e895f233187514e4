"""Seeded input generators.

Host side: numpy PCG64 (``np.random.default_rng(seed)``), fp64 normal draws
rounded once to fp32, multiplied by a power-of-two loss scale (exact in fp32)
and rounded to the 16-bit storage type by numpy (fp16) or torch (bf16).

Device side: torch's seeded device generator (Philox) fills fp32 chunks of a
fixed size that are then rounded to the 16-bit storage type by torch's copy.
The chunk size is part of the recipe: the same seed and chunk size give the
same bytes on every run.

Nothing here computes any part of the optimizer step.
"""
from typing import List, Sequence, Tuple

import numpy as np

# Special 16-bit encodings used to inject non-finite gradients.
F16_POS_INF, F16_NEG_INF, F16_NAN = 0x7C00, 0xFC00, 0x7E00
BF16_POS_INF, BF16_NEG_INF, BF16_NAN = 0x7F80, 0xFF80, 0x7FC0

DEVICE_CHUNK = 1 << 27  # elements per device fill chunk


def specials(dtype: str) -> Tuple[int, int, int]:
    return (F16_POS_INF, F16_NEG_INF, F16_NAN) if dtype == "f16" else \
        (BF16_POS_INF, BF16_NEG_INF, BF16_NAN)


# ----------------------------------------------------------------- host side
def normal_f32(seed: int, n: int, sigma: float) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(n) * sigma).astype(np.float32)


def f32_to_bits16(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to the 16-bit storage type (nearest-even) and
    return the raw bit patterns as uint16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    import torch
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def split(flat: np.ndarray, numels: Sequence[int]) -> List[np.ndarray]:
    out, off = [], 0
    for k in numels:
        out.append(flat[off:off + k])
        off += k
    return out


def host_master_list(cfg) -> List[np.ndarray]:
    """fp32 initial parameters of every tensor, one seeded stream in list order."""
    return split(normal_f32(cfg.master_seed(), cfg.psi, cfg.master_sigma), cfg.numels)


def host_grad_list(cfg, step: int) -> List[np.ndarray]:
    """16-bit gradient bits of every tensor for one step (scaled by the loss scale)."""
    g = normal_f32(cfg.grad_seed(step), cfg.psi, cfg.grad_sigma) * np.float32(cfg.loss_scale)
    return split(f32_to_bits16(g, cfg.dtype), cfg.numels)


def host_grad_flat(seed: int, n: int, sigma: float, scale: float, dtype: str) -> np.ndarray:
    g = normal_f32(seed, n, sigma) * np.float32(scale)
    return f32_to_bits16(g, dtype)


def inject_plan(cfg, n: int):
    """(step, [(local index, bits), ...]) of the non-finite values that the
    injection workload writes into its gradient shard: +inf and NaN at two
    seeded distinct positions and -inf at local index 0."""
    rng = np.random.default_rng(cfg.inject_seed())
    step = int(rng.integers(0, cfg.steps))
    a, b = (int(v) for v in rng.choice(np.arange(1, n), 2, replace=False))
    pinf, ninf, nan = specials(cfg.dtype)
    return step, [(a, pinf), (b, nan), (0, ninf)]


# --------------------------------------------------------------- device side
def torch_dtype(dtype: str):
    import torch
    return {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def device_fill_normal_(t, seed: int, sigma: float, scale: float = 1.0,
                        chunk: int = DEVICE_CHUNK):
    """Fill a 1-D device tensor (fp32, fp16 or bf16) with seeded N(0, sigma)*scale
    draws, rounded to the tensor's dtype, in fixed-size fp32 chunks."""
    import torch
    n = t.numel()
    gen = torch.Generator(device=t.device)
    gen.manual_seed(seed)
    tmp = torch.empty(min(chunk, max(n, 1)), dtype=torch.float32, device=t.device)
    for lo in range(0, n, chunk):
        k = min(chunk, n - lo)
        buf = tmp[:k]
        buf.normal_(0.0, sigma, generator=gen)
        if scale != 1.0:
            buf.mul_(scale)
        t[lo:lo + k].copy_(buf)
    del tmp
    return t


def device_grad_list(cfg, step: int, device, which=None):
    """Per-tensor 16-bit gradients for one step, drawn on the device.  Each
    tensor gets its own seed derived from the step seed and its index, so a
    subset of the list can be materialised alone."""
    import torch
    out = {}
    idxs = range(len(cfg.tensors)) if which is None else which
    for i in idxs:
        t = torch.empty(cfg.numels[i], dtype=torch_dtype(cfg.dtype), device=device)
        device_fill_normal_(t, cfg.grad_seed(step) * 100003 + i, cfg.grad_sigma, cfg.loss_scale)
        out[i] = t
    return out
