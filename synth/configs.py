"""The five synthetic workloads of the shard-local mixed-precision AdamW step.

Each workload is one data-parallel rank's share of a model whose flat
parameter vector has psi elements, split over nd ranks.  The model's tensor
list follows the GPT-2-like layout that the ZeRO paper's experiments vary by
hidden size and depth ("ZeRO: Memory Optimizations Toward Training Trillion
Parameter Models", paper summary page, section on the experimental setup):
token and position embeddings, then per layer two layer norms, the fused QKV
projection, the output projection and the two MLP matrices (weights and
biases), then a final layer norm; the LM head is tied to the token embedding.
That gives 12*h*h + 13*h parameters per layer.

Only shapes, dtypes, seeds and hyper-parameters are stated here.
"""
import math
from dataclasses import dataclass, field
from functools import cached_property
from typing import List, Optional, Tuple

import numpy as np

VOCAB = 50257
N_POS = 1024


@dataclass(frozen=True)
class AdamW:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    max_grad_norm: float = 0.0  # <= 0 disables clipping
    inv_loss_scale: float = 1.0


def gpt_param_list(hidden: int, layers: int, vocab: int = VOCAB,
                   n_pos: int = N_POS) -> List[Tuple[str, Tuple[int, ...]]]:
    """(name, shape) of every parameter tensor, in flattening order."""
    h = hidden
    out = [("wte", (vocab, h)), ("wpe", (n_pos, h))]
    for i in range(layers):
        p = f"h{i}."
        out += [
            (p + "ln1.w", (h,)), (p + "ln1.b", (h,)),
            (p + "qkv.w", (3 * h, h)), (p + "qkv.b", (3 * h,)),
            (p + "proj.w", (h, h)), (p + "proj.b", (h,)),
            (p + "ln2.w", (h,)), (p + "ln2.b", (h,)),
            (p + "fc1.w", (4 * h, h)), (p + "fc1.b", (4 * h,)),
            (p + "fc2.w", (h, 4 * h)), (p + "fc2.b", (h,)),
        ]
    out += [("lnf.w", (h,)), ("lnf.b", (h,))]
    return out


def tiny_param_sizes(psi: int = 1 << 20, n_tensors: int = 8, seed: int = 0) -> List[int]:
    """Ragged sizes of the small workload: n_tensors-1 distinct seeded cut
    points drawn without replacement from [1, psi)."""
    rng = np.random.default_rng(seed)
    cuts = sorted(int(c) for c in rng.choice(np.arange(1, psi), n_tensors - 1, replace=False))
    edges = [0] + cuts + [psi]
    return [edges[i + 1] - edges[i] for i in range(n_tensors)]


@dataclass(frozen=True)
class Config:
    idx: int
    name: str
    tensors: Tuple[Tuple[str, Tuple[int, ...]], ...]
    nd: int
    rank: int
    dtype: str                  # 16-bit grad and param storage: "f16" or "bf16"
    grad_sigma: float           # std-dev of the unscaled grads
    loss_scale: float           # grads are stored multiplied by this
    steps: int
    hp: AdamW
    master_sigma: float = 0.02
    bucket_elems: Optional[int] = None    # constant fused-buffer size, in elements
    grads_as_list: bool = True  # grads arrive per tensor (then flattened) or as the shard
    param_list_fp32: bool = False  # master initialised from a list of fp32 tensors
    inject: bool = False        # one step of the run carries inf/nan grads
    host_generated: bool = False  # small enough to draw every input on the host

    @cached_property
    def numels(self) -> List[int]:
        return [math.prod(s) for _, s in self.tensors]

    @property
    def psi(self) -> int:
        return sum(self.numels)

    def master_seed(self) -> int:
        return 1000 + self.idx

    def grad_seed(self, step: int) -> int:
        return 2000 + 100 * self.idx + step

    def inject_seed(self) -> int:
        return 3000 + self.idx


def _tiny() -> Config:
    sizes = tiny_param_sizes()
    return Config(
        idx=1, name="tiny", tensors=tuple((f"t{i}", (s,)) for i, s in enumerate(sizes)),
        nd=4, rank=0, dtype="f16", grad_sigma=1e-3, loss_scale=1024.0, steps=10,
        hp=AdamW(inv_loss_scale=1.0 / 1024.0), bucket_elems=65537,
        param_list_fp32=True, host_generated=True)


def _gpt2_1p5b() -> Config:
    return Config(
        idx=2, name="gpt2-1.5b", tensors=tuple(gpt_param_list(1600, 48)),
        nd=1, rank=0, dtype="f16", grad_sigma=1e-3, loss_scale=65536.0, steps=10,
        hp=AdamW(max_grad_norm=1.0, inv_loss_scale=1.0 / 65536.0),
        bucket_elems=500_000_000)


def _gpt_7p5b() -> Config:
    return Config(
        idx=3, name="gpt-7.5b", tensors=tuple(gpt_param_list(4096, 36)),
        nd=8, rank=3, dtype="bf16", grad_sigma=1e-3, loss_scale=1.0, steps=10,
        hp=AdamW(), bucket_elems=500_000_000)


def _gpt_13b() -> Config:
    return Config(
        idx=4, name="gpt-13b", tensors=tuple(gpt_param_list(5120, 40)),
        nd=1, rank=0, dtype="bf16", grad_sigma=1e-4, loss_scale=1.0, steps=5,
        hp=AdamW(), grads_as_list=False)


def _gpt_100b_shard() -> Config:
    return Config(
        idx=5, name="gpt-100b-nd400-r399", tensors=tuple(gpt_param_list(8192, 124)),
        nd=400, rank=399, dtype="f16", grad_sigma=1e-3, loss_scale=65536.0, steps=4,
        hp=AdamW(max_grad_norm=1.0, inv_loss_scale=1.0 / 65536.0), inject=True)


WORKLOADS = {c.idx: c for c in (_tiny(), _gpt2_1p5b(), _gpt_7p5b(), _gpt_13b(), _gpt_100b_shard())}
