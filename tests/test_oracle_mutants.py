"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle.c to a temporary directory, applies one plausible
mistake (a dropped term, a wrong sign, index or operand), builds it with gcc
on the CPU and runs the pin suite against it.  Every mutant must fail at
least one pin.  The product code is not involved.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "partition_drops_remainder": ("start += small + (r < extra ? 1 : 0);", "start += small;"),
    "accounting_floor_not_ceil": ("psi / nd + (psi % nd ? 1 : 0)", "psi / nd"),
    "accounting_stage2_grads_unsharded": ("if (stage >= 2) grads = 2 * largest;", ""),
    "accounting_stage3_params_unsharded": ("if (stage >= 3) params = 2 * largest;", ""),
    "f16_subnormal_exponent": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "bf16_bias": ("ldexp((double)(128 + f), e - 134)", "ldexp((double)(128 + f), e - 135)"),
    "rounding_truncates": ("return nearbyint(a / q) * q;", "return floor(a / q) * q;"),
    "bf16_overflow_threshold": ("ldexp(255.0, 120)", "ldexp(255.0, 119)"),
    "overflow_misses_inf": ("if (!isfinite(x))", "if (isnan(x))"),
    "stats_not_unscaled": ("double u = x * inv_scale;", "double u = x;"),
    "stats_drops_compensation": ("neumaier_add(&s, &c, pc[t]);", ""),
    "skip_advances_counter": ("s->t = s->skip ? t_prev : t_prev + 1;", "s->t = t_prev + 1;"),
    "clip_uses_squared_norm": ("s->coef = hp->max_grad_norm / norm;",
                               "s->coef = hp->max_grad_norm / sq_norm;"),
    "bias_correction_off_by_one": ("s->bc2 = 1.0 - pow(hp->beta2, (double)s->t);",
                                   "s->bc2 = 1.0 - pow(hp->beta2, (double)(s->t + 1));"),
    "bias_correction1_uses_beta2": ("s->bc1 = 1.0 - pow(hp->beta1, (double)s->t);",
                                    "s->bc1 = 1.0 - pow(hp->beta2, (double)s->t);"),
    "momentum_uses_beta2": ("(1.0 - s->beta1) * g;", "(1.0 - s->beta2) * g;"),
    "variance_not_squared": ("(1.0 - s->beta2) * g * g;", "(1.0 - s->beta2) * g;"),
    "eps_inside_sqrt": ("(sqrt(v_hat) + s->eps)", "sqrt(v_hat + s->eps)"),
    "decay_not_lr_scaled": ("p - s->lr * s->weight_decay * p", "p - s->weight_decay * p"),
    "update_wrong_sign": ("- s->lr * m_hat /", "+ s->lr * m_hat /"),
    "grad_not_unscaled": ("graw * s->inv_scale * s->coef", "graw * s->coef"),
    "grad_not_clipped": ("graw * s->inv_scale * s->coef", "graw * s->inv_scale"),
    "skip_ignored": ("    if (s->skip)\n        return;\n#pragma omp parallel for",
                     "#pragma omp parallel for"),
    "param_from_old_master": ("        master[i] = (float)pn;\n", ""),
    "loss_scale_keeps_count_on_overflow": ("        s->good_steps = 0;\n        s->overflows += 1;",
                                           "        s->overflows += 1;"),
    "loss_scale_grows_one_step_late": ("if (s->good_steps == c->growth_interval)",
                                       "if (s->good_steps > c->growth_interval)"),
    "loss_scale_ignores_floor": ("s->scale = reduced > c->min_scale ? reduced : c->min_scale;",
                                 "s->scale = reduced;"),
}


def _run(name, tmpdir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    c = os.path.join(tmpdir, f"{name}.c")
    so = os.path.join(tmpdir, f"{name}.so")
    open(c, "w").write(mutated)
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                           "-std=c11", "-w", "-o", so, c, "-lm"])
    env = dict(os.environ, ORACLE_LIB=so, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda n: _run(n, str(tmp_path)), sorted(MUTANTS)))
    survivors = [n for n, rc in results if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
    assert all(rc == 1 for _, rc in results), results  # 1 = tests failed (not a crash)
