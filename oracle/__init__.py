"""Oracle for the shard-local mixed-precision AdamW step of ZeRO-DP.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the library or its binding.
It shares no code with the HIP path.

The arithmetic lives in ``oracle.c`` (plain fp64 loops, built with gcc); the
bucket plan and the flatten are written here in plain Python / torch-CPU.

Sources (web pages on ZeRO):
  [P2] "ZeRO: Memory Optimizations Toward Training Trillion Parameter Models"
       (paper summary page): memory accounting, ZeRO-DP stages, ZeRO-R CB.
  [P4] "ZeRO" (AI-library tutorial page): 16 bytes/param with AdamW and the
       per-stage memory equations.
"""
import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

U64 = ctypes.c_uint64
U32 = ctypes.c_uint32
DBL = ctypes.c_double
VP = ctypes.c_void_p


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc: fp64, no FMA contraction, no fast-math."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                               "-fno-fast-math", "-std=c11", "-Wall", "-Wextra", "-o", tmp,
                               _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _HP(ctypes.Structure):
    _fields_ = [("lr", DBL), ("beta1", DBL), ("beta2", DBL), ("eps", DBL),
                ("weight_decay", DBL), ("max_grad_norm", DBL), ("inv_loss_scale", DBL)]


class Scalars(ctypes.Structure):
    _fields_ = [("t", U64), ("skip", U32), ("pad", U32), ("coef", DBL), ("inv_scale", DBL),
                ("bc1", DBL), ("bc2", DBL), ("lr", DBL), ("beta1", DBL), ("beta2", DBL),
                ("eps", DBL), ("weight_decay", DBL)]


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB")  # a planted-mistake build, for mutation tests
        if not path:
            if not os.path.exists(_LIB):
                build()
            path = _LIB
        L = ctypes.CDLL(path)
        L.orc_partition.argtypes = [U64, U32, U32, ctypes.POINTER(U64), ctypes.POINTER(U64)]
        L.orc_mem_bytes.argtypes = [U32, U64, U32, U32, ctypes.POINTER(U64)]
        L.orc_f16_value.argtypes = [ctypes.c_uint16]
        L.orc_f16_value.restype = DBL
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_value.restype = DBL
        L.orc_f16_bits.argtypes = [ctypes.c_float]
        L.orc_f16_bits.restype = ctypes.c_uint16
        L.orc_bf16_bits.argtypes = [ctypes.c_float]
        L.orc_bf16_bits.restype = ctypes.c_uint16
        L.orc_value16_array.argtypes = [VP, ctypes.c_int, VP, U64]
        L.orc_bits16_array.argtypes = [VP, ctypes.c_int, VP, U64]
        L.orc_grad_stats.argtypes = [VP, ctypes.c_int, U64, DBL, ctypes.POINTER(DBL),
                                     ctypes.POINTER(U32)]
        L.orc_step_scalars.argtypes = [ctypes.POINTER(_HP), ctypes.c_int, DBL, U32, U64,
                                       ctypes.POINTER(Scalars)]
        L.orc_adamw.argtypes = [ctypes.POINTER(Scalars), VP, ctypes.c_int, VP, VP, VP, VP,
                                ctypes.c_int, U64]
        L.orc_adamw_f64.argtypes = [ctypes.POINTER(Scalars), VP, ctypes.c_int, VP, VP, VP,
                                    VP, VP, VP, U64]
        L.orc_loss_scale_init.argtypes = [ctypes.POINTER(Scaler), ctypes.POINTER(ScaleState)]
        L.orc_loss_scale_update.argtypes = [ctypes.POINTER(Scaler), U32,
                                            ctypes.POINTER(ScaleState)]
        L.orc_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(VP)


def _is_bf16(dtype: str) -> int:
    if dtype not in ("f16", "bf16"):
        raise ValueError(dtype)
    return 1 if dtype == "bf16" else 0


def num_threads() -> int:
    return lib().orc_num_threads()


# ------------------------------------------------------------------ planner
def partition(psi: int, nd: int, rank: int) -> Tuple[int, int]:
    """[P2] ZeRO-DP Stage 1: rank's contiguous part of the flat psi elements."""
    b, e = U64(), U64()
    if lib().orc_partition(psi, nd, rank, ctypes.byref(b), ctypes.byref(e)):
        raise ValueError("invalid partition arguments")
    return b.value, e.value


def mem_bytes(stage: int, psi: int, nd: int, k: int = 12) -> int:
    """[P2] memory accounting and ZeRO-DP table; [P4] ZeRO-1/2/3 equations."""
    out = U64()
    if lib().orc_mem_bytes(stage, psi, nd, k, ctypes.byref(out)):
        raise ValueError("invalid accounting arguments")
    return out.value


@dataclass(frozen=True)
class Segment:
    bucket: int
    tensor: int
    src_off: int
    dst_off: int
    len: int


def bucket_plan(numels: Sequence[int], bucket_elems: int, lo: int, hi: int) -> List[Segment]:
    """[P2] ZeRO-R, CB: the tensors are laid end to end in list order and the
    flat stream is cut into windows of a constant number of elements
    (a tensor may straddle two windows; the last window may be short).
    Returns every non-empty piece of (tensor interval) x (window) x [lo, hi),
    in flat order; dst_off counts from lo."""
    if bucket_elems <= 0 or lo > hi or hi > sum(numels):
        raise ValueError("invalid plan arguments")
    segs = []
    start = 0
    for ti, k in enumerate(numels):
        t_lo, t_hi = start, start + k
        start = t_hi
        a, b = max(t_lo, lo), min(t_hi, hi)
        while a < b:
            bucket = a // bucket_elems
            cut = min(b, (bucket + 1) * bucket_elems)
            segs.append(Segment(bucket, ti, a - t_lo, a - lo, cut - a))
            a = cut
    return segs


def flatten(tensors: Sequence, lo: int, hi: int) -> np.ndarray:
    """The flat stream of the list (in list order), elements [lo, hi)."""
    import torch
    ts = [t if isinstance(t, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(t))
          for t in tensors]
    return torch.cat([t.reshape(-1) for t in ts])[lo:hi].numpy()


# --------------------------------------------------------------- numerics
def value16(bits: np.ndarray, dtype: str) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.size, dtype=np.float64)
    lib().orc_value16_array(_ptr(bits), _is_bf16(dtype), _ptr(out), bits.size)
    return out


def bits16(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, dtype=np.uint16)
    lib().orc_bits16_array(_ptr(x), _is_bf16(dtype), _ptr(out), x.size)
    return out


def grad_stats(g_bits: np.ndarray, dtype: str, inv_scale: float) -> Tuple[float, int]:
    """(squared L2 norm of the unscaled grads, overflow flag)."""
    g_bits = np.ascontiguousarray(g_bits, dtype=np.uint16)
    sq, ov = DBL(), U32()
    lib().orc_grad_stats(_ptr(g_bits), _is_bf16(dtype), g_bits.size, inv_scale,
                         ctypes.byref(sq), ctypes.byref(ov))
    return sq.value, ov.value


def step_scalars(hp, have_stats: bool, sq_norm: float, overflow: int, t_prev: int) -> Scalars:
    h = _HP(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.max_grad_norm,
            hp.inv_loss_scale)
    s = Scalars()
    lib().orc_step_scalars(ctypes.byref(h), int(have_stats), sq_norm, overflow, t_prev,
                           ctypes.byref(s))
    return s


class Scaler(ctypes.Structure):
    _fields_ = [("init_scale", DBL), ("growth_factor", DBL), ("backoff_factor", DBL),
                ("growth_interval", U64), ("min_scale", DBL), ("max_scale", DBL)]


class ScaleState(ctypes.Structure):
    _fields_ = [("scale", DBL), ("inv_scale", DBL), ("good_steps", U64), ("overflows", U64)]


def loss_scale_sequence(cfg: Scaler, overflows: Sequence[int]) -> List[Tuple[float, float, int, int]]:
    """(scale, inv_scale, good_steps, overflows) after each step of a run whose
    per-step overflow flags are given, starting from cfg.init_scale."""
    st = ScaleState()
    lib().orc_loss_scale_init(ctypes.byref(cfg), ctypes.byref(st))
    out = []
    for ov in overflows:
        lib().orc_loss_scale_update(ctypes.byref(cfg), int(bool(ov)), ctypes.byref(st))
        out.append((st.scale, st.inv_scale, st.good_steps, st.overflows))
    return out


def adamw_(s: Scalars, g_bits: np.ndarray, gdtype: str, master: np.ndarray, m: np.ndarray,
           v: np.ndarray, p_bits: np.ndarray, pdtype: str) -> None:
    """In-place AdamW on contiguous fp32 master/m/v; writes 16-bit params."""
    n = g_bits.size
    for a, dt in ((g_bits, np.uint16), (master, np.float32), (m, np.float32),
                  (v, np.float32), (p_bits, np.uint16)):
        if a.dtype != dt or not a.flags.c_contiguous or a.size != n:
            raise ValueError("adamw_: arrays must be contiguous and of equal length")
    lib().orc_adamw(ctypes.byref(s), _ptr(g_bits), _is_bf16(gdtype), _ptr(master), _ptr(m),
                    _ptr(v), _ptr(p_bits), _is_bf16(pdtype), n)


def adamw_f64(s: Scalars, g_bits: np.ndarray, gdtype: str, master: np.ndarray, m: np.ndarray,
              v: np.ndarray):
    """Unrounded fp64 results (p', m', v') of one AdamW step."""
    g_bits = np.ascontiguousarray(g_bits, dtype=np.uint16)
    master = np.ascontiguousarray(master, dtype=np.float32)
    m = np.ascontiguousarray(m, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    n = g_bits.size
    po, mo, vo = (np.empty(n, dtype=np.float64) for _ in range(3))
    lib().orc_adamw_f64(ctypes.byref(s), _ptr(g_bits), _is_bf16(gdtype), _ptr(master), _ptr(m),
                        _ptr(v), _ptr(po), _ptr(mo), _ptr(vo), n)
    return po, mo, vo
