"""Brute-force reference for tiny inputs: exact rational arithmetic.

TEST INFRASTRUCTURE ONLY.  Used to pin the fp64 oracle: every quantity is an
exact ``fractions.Fraction`` of the stored inputs; square roots are taken with
``decimal`` at 60 significant digits.  16-bit values are decoded by numpy
(binary16) and torch (bfloat16), independently of the oracle's own decoder.

Same update as the oracle (Adam with bias correction and decoupled weight
decay, clip by global norm, skip on overflow), written from the definitions.
"""
from decimal import Decimal, getcontext
from fractions import Fraction
from typing import List, Sequence, Tuple

import numpy as np

getcontext().prec = 60


def decode16(bits: Sequence[int], dtype: str) -> List[float]:
    b = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return [float(x) for x in b.view(np.float16)]
    import torch
    t = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    return [float(x) for x in t]


def fsqrt(x: Fraction) -> Fraction:
    if x == 0:
        return Fraction(0)
    return Fraction((Decimal(x.numerator) / Decimal(x.denominator)).sqrt())


def sq_norm(bits, dtype: str, inv_scale: float) -> Fraction:
    inv = Fraction(inv_scale)
    return sum((Fraction(x) * inv) ** 2 for x in decode16(bits, dtype))


def adamw(hp, sq: Fraction, t: int, bits, dtype: str, master, m, v) -> Tuple[list, list, list]:
    """One step at step number t (already advanced).  Returns exact new
    (param, m, v) as Fractions (sqrt rounded to 60 digits)."""
    b1, b2 = Fraction(hp.beta1), Fraction(hp.beta2)
    lr, wd, eps = Fraction(hp.lr), Fraction(hp.weight_decay), Fraction(hp.eps)
    coef = Fraction(1)
    if hp.max_grad_norm > 0 and sq > 0:
        norm = fsqrt(sq)
        c = Fraction(hp.max_grad_norm)
        if c < norm:
            coef = c / norm
    bc1 = 1 - b1 ** t
    bc2 = 1 - b2 ** t
    inv = Fraction(hp.inv_loss_scale)
    P, M, V = [], [], []
    for x, p0, m0, v0 in zip(decode16(bits, dtype), master, m, v):
        g = Fraction(x) * inv * coef
        m1 = b1 * Fraction(float(m0)) + (1 - b1) * g
        v1 = b2 * Fraction(float(v0)) + (1 - b2) * g * g
        p = Fraction(float(p0))
        p1 = p - lr * wd * p - lr * (m1 / bc1) / (fsqrt(v1 / bc2) + eps)
        P.append(p1)
        M.append(m1)
        V.append(v1)
    return P, M, V
