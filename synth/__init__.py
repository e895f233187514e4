"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

This package only *describes* inputs (tensor shapes, dtypes, seeds,
hyper-parameters) and *draws* them (seeded normal samples rounded to the
16-bit storage type).  It holds none of the arithmetic of the method itself:
partitioning, bucketing, statistics and the optimizer step live in the HIP
library and, independently, in the oracle.
"""
from .configs import WORKLOADS, Config, AdamW, gpt_param_list, tiny_param_sizes  # noqa: F401
from . import gen  # noqa: F401
