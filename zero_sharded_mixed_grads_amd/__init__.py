"""Python binding of libzero_mi355x: the shard-local mixed-precision AdamW
step of ZeRO-DP for AMD MI355X.

Argument marshalling only: every function forwards to the C entry point of
the same name in ``libzero_mi355x.so`` (declared in ``include/zero.h``).
Tensors are accepted where the C call takes a device pointer (their
``data_ptr()`` is passed); the stream defaults to torch's current stream.
Nothing here computes any part of the step, and there is no fallback: if the
library is missing, importing a device call raises.
"""
import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import torch  # loads the HIP runtime that the library then binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzero_mi355x.so")

ZERO_OK, ZERO_EINVAL, ZERO_ENOSPC, ZERO_EALIGN, ZERO_EDEVICE, ZERO_EIO = range(6)
ZERO_F32, ZERO_F16, ZERO_BF16 = range(3)

_DTYPES = {"f32": ZERO_F32, "f16": ZERO_F16, "bf16": ZERO_BF16,
           torch.float32: ZERO_F32, torch.float16: ZERO_F16, torch.bfloat16: ZERO_BF16}

U64, U32, DBL, VP = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double, ctypes.c_void_p


class ZeroError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(detail)
        self.status = status


class Segment(ctypes.Structure):
    _fields_ = [("bucket", U64), ("tensor", U64), ("src_off", U64), ("dst_off", U64),
                ("len", U64)]


class AdamW(ctypes.Structure):
    _fields_ = [("lr", DBL), ("beta1", DBL), ("beta2", DBL), ("eps", DBL),
                ("weight_decay", DBL), ("max_grad_norm", DBL), ("inv_loss_scale", DBL)]


class GradStats(ctypes.Structure):  # zero_grad_stats_t, device resident
    _fields_ = [("sq_norm", DBL), ("overflow", U32), ("pad", U32)]


class AdamState(ctypes.Structure):  # zero_adam_state_t, device resident
    _fields_ = [("step", U64), ("skip", U32), ("pad0", U32), ("coef", DBL),
                ("inv_scale", DBL), ("bc1", DBL), ("bc2", DBL), ("inv_bc1", DBL),
                ("inv_bc2", DBL)]


class LossScaler(ctypes.Structure):  # zero_loss_scaler, host parameters
    _fields_ = [("init_scale", DBL), ("growth_factor", DBL), ("backoff_factor", DBL),
                ("growth_interval", U64), ("min_scale", DBL), ("max_scale", DBL)]


class LossScale(ctypes.Structure):  # zero_loss_scale_t, device resident
    _fields_ = [("scale", DBL), ("inv_scale", DBL), ("good_steps", U64), ("overflows", U64)]


class CkptHeader(ctypes.Structure):  # zero_ckpt_header
    _fields_ = [("magic", ctypes.c_char * 8), ("version", U32), ("nd", U32), ("rank", U32),
                ("pad", U32), ("psi", U64), ("begin", U64), ("end", U64), ("step", U64),
                ("flags", U64)]


assert ctypes.sizeof(GradStats) == 16 and ctypes.sizeof(AdamState) == 64
assert ctypes.sizeof(CkptHeader) == 64
assert ctypes.sizeof(LossScaler) == 48 and ctypes.sizeof(LossScale) == 32

EXPORTS = ("zero_status_str", "zero_last_error", "zero_partition", "zero_mem_bytes",
           "zero_bucket_plan", "zero_bucket_flatten", "zero_grad_stats_workspace",
           "zero_grad_stats", "zero_bucket_flatten_stats_workspace", "zero_bucket_flatten_stats",
           "zero_grad_stats_noalloc", "zero_grad_stats_tensors", "zero_adam_step_tensors",
           "zero_adam_step", "zero_offload_staging_bytes", "zero_offload_adam_step",
           "zero_ckpt_save", "zero_ckpt_read_header", "zero_ckpt_load",
           "zero_loss_scale_init", "zero_loss_scale_update", "zero_state_layout")

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def load(path: str):
    """Loads a build of the library at `path` and declares its signatures."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(path)
    L.zero_status_str.argtypes = [ctypes.c_int]
    L.zero_status_str.restype = ctypes.c_char_p
    L.zero_last_error.argtypes = []
    L.zero_last_error.restype = ctypes.c_char_p
    L.zero_partition.argtypes = [U64, U32, U32, ctypes.POINTER(U64), ctypes.POINTER(U64)]
    L.zero_mem_bytes.argtypes = [U32, U64, U32, U32, ctypes.POINTER(U64)]
    L.zero_bucket_plan.argtypes = [ctypes.POINTER(U64), U32, U64, U64, U64,
                                   ctypes.POINTER(Segment), U64, ctypes.POINTER(U64)]
    L.zero_bucket_flatten.argtypes = [ctypes.POINTER(VP), ctypes.POINTER(U64), U32,
                                      ctypes.c_int, U64, U64, VP, VP]
    L.zero_grad_stats_workspace.argtypes = [U64, ctypes.POINTER(ctypes.c_size_t)]
    L.zero_grad_stats.argtypes = [VP, ctypes.c_int, U64, DBL, VP, VP, ctypes.c_size_t, VP,
                                  VP]
    L.zero_grad_stats_noalloc.argtypes = [VP, ctypes.c_int, U64, DBL, VP, VP, VP]
    L.zero_grad_stats_tensors.argtypes = [ctypes.POINTER(VP), ctypes.POINTER(U64), U32,
                                          ctypes.c_int, U64, U64, DBL, VP, VP, ctypes.c_size_t,
                                          VP, VP]
    L.zero_adam_step_tensors.argtypes = [ctypes.POINTER(AdamW), ctypes.POINTER(VP),
                                         ctypes.POINTER(U64), U32, ctypes.c_int, U64, U64, VP,
                                         VP, VP, VP, ctypes.c_int, VP, VP, VP, VP]
    L.zero_bucket_flatten_stats_workspace.argtypes = [ctypes.POINTER(U64), U32, U64, U64,
                                                      ctypes.POINTER(ctypes.c_size_t)]
    L.zero_bucket_flatten_stats.argtypes = [ctypes.POINTER(VP), ctypes.POINTER(U64), U32,
                                            ctypes.c_int, U64, U64, VP, DBL, VP, VP,
                                            ctypes.c_size_t, VP, VP]
    L.zero_adam_step.argtypes = [ctypes.POINTER(AdamW), VP, ctypes.c_int, VP, VP, VP, VP,
                                 ctypes.c_int, U64, VP, VP, VP, VP]
    L.zero_loss_scale_init.argtypes = [ctypes.POINTER(LossScaler), VP, VP]
    L.zero_state_layout.argtypes = [U64, U64, ctypes.POINTER(U64)]
    L.zero_loss_scale_update.argtypes = [ctypes.POINTER(LossScaler), VP, VP, VP]
    L.zero_offload_staging_bytes.argtypes = [U64, ctypes.POINTER(ctypes.c_size_t)]
    L.zero_offload_adam_step.argtypes = [ctypes.POINTER(AdamW), VP, ctypes.c_int, VP, VP,
                                         VP, VP, ctypes.c_int, U64, VP, VP, VP, VP,
                                         ctypes.c_size_t, VP]
    L.zero_ckpt_save.argtypes = [ctypes.c_char_p, U64, U32, U32, VP, VP, VP, VP, VP, VP]
    L.zero_ckpt_read_header.argtypes = [ctypes.c_char_p, ctypes.POINTER(CkptHeader)]
    L.zero_ckpt_load.argtypes = [ctypes.POINTER(ctypes.c_char_p), U32, U64, U32, U32, VP, VP,
                                 VP, VP, VP, VP]
    for name in EXPORTS[2:]:
        getattr(L, name).restype = ctypes.c_int
    return L


def _check(status: int):
    if status != ZERO_OK:
        raise ZeroError(status, lib().zero_last_error().decode())


def _ptr(x, host: bool = False) -> Optional[int]:
    """The address of a buffer argument: None, an integer address (passed as
    it is), or a contiguous tensor on the device (host=False) or in host
    memory (host=True).  A tensor on the wrong side or with gaps is refused
    here, since the library cannot tell and the kernels would read the wrong
    memory."""
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        if x.is_cuda == host:
            want = "host" if host else "device"
            raise ValueError(f"expected a {want} tensor, got one on {x.device}")
        if not x.is_contiguous():
            raise ValueError("tensor arguments must be contiguous")
        return x.data_ptr()
    return int(x)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dtype(dt) -> int:
    return _DTYPES[dt] if dt in _DTYPES else int(dt)


def status_str(status: int) -> str:
    return lib().zero_status_str(status).decode()


# ------------------------------------------------------------------ planner
def zero_partition(psi: int, nd: int, rank: int) -> Tuple[int, int]:
    b, e = U64(), U64()
    _check(lib().zero_partition(psi, nd, rank, ctypes.byref(b), ctypes.byref(e)))
    return b.value, e.value


def zero_mem_bytes(stage: int, psi: int, nd: int, k: int = 12) -> int:
    out = U64()
    _check(lib().zero_mem_bytes(stage, psi, nd, k, ctypes.byref(out)))
    return out.value


def zero_bucket_plan(numel: Sequence[int], bucket_elems: int, range_begin: int,
                     range_end: int, cap: Optional[int] = None) -> List[Tuple[int, ...]]:
    """Segments (bucket, tensor, src_off, dst_off, len) of the range."""
    arr = (U64 * len(numel))(*numel)
    n = U64()
    if cap is None:  # ask for the count first
        st = lib().zero_bucket_plan(arr, len(numel), bucket_elems, range_begin, range_end,
                                    None, 0, ctypes.byref(n))
        if st not in (ZERO_OK, ZERO_ENOSPC):
            _check(st)
        cap = n.value
    segs = (Segment * max(cap, 1))()
    _check(lib().zero_bucket_plan(arr, len(numel), bucket_elems, range_begin, range_end,
                                  segs, cap, ctypes.byref(n)))
    return [(s.bucket, s.tensor, s.src_off, s.dst_off, s.len) for s in segs[:n.value]]


def zero_state_layout(n: int, pool_bytes: int) -> List[int]:
    """Byte offsets of grad, master, exp_avg, exp_avg_sq and param inside one
    device pool, spread evenly over it."""
    out = (U64 * 5)()
    _check(lib().zero_state_layout(n, pool_bytes, out))
    return list(out)


# ------------------------------------------------------------- device calls
def tensor_table(tensors: Sequence, numel: Optional[Sequence[int]] = None):
    """The (pointer array, element-count array) pair that the gather calls
    take, marshalled once.  tensors: device tensors or device pointers (None
    for tensors outside the range); numel defaults to each tensor's numel().
    Passing the pair to the gathers as `tensors` and `numel` skips building
    the two arrays again on every call, which costs about 0.1 ms per
    thousand tensors."""
    if isinstance(tensors, ctypes.Array) and isinstance(numel, ctypes.Array):
        return tensors, numel
    if numel is None:
        numel = [t.numel() for t in tensors]
    if len(numel) != len(tensors):
        raise ValueError(f"{len(tensors)} tensors but {len(numel)} element counts")
    ptrs = (VP * len(tensors))(*[_ptr(t) for t in tensors])
    nums = (U64 * len(numel))(*numel)
    return ptrs, nums


def zero_bucket_flatten(tensors: Sequence, numel: Optional[Sequence[int]], dtype,
                        range_begin: int, count: int, dst, stream=None) -> None:
    """tensors: device tensors or device pointers (None allowed for tensors
    outside the range); numel defaults to each tensor's numel().  Both may
    also be the arrays of tensor_table()."""
    ptrs, nums = tensor_table(tensors, numel)
    _check(lib().zero_bucket_flatten(ptrs, nums, len(ptrs), _dtype(dtype), range_begin,
                                     count, _ptr(dst), _stream(stream)))


def zero_grad_stats_workspace(n: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().zero_grad_stats_workspace(n, ctypes.byref(out)))
    return out.value


def zero_grad_stats(grad, gdtype, n: int, inv_loss_scale: float, workspace, ws_bytes: int,
                    d_stats, stream=None, d_scale=None) -> None:
    """d_scale: optional device zero_loss_scale_t whose inv_scale replaces
    inv_loss_scale (read on the device)."""
    _check(lib().zero_grad_stats(_ptr(grad), _dtype(gdtype), n, inv_loss_scale, _ptr(d_scale),
                                 _ptr(workspace), ws_bytes, _ptr(d_stats), _stream(stream)))


def zero_grad_stats_noalloc(grad, gdtype, n: int, inv_loss_scale: float, d_stats, stream=None,
                            d_scale=None) -> None:
    """zero_grad_stats with the library's own per-device scratch instead of a
    caller workspace (calls on one device must not overlap)."""
    _check(lib().zero_grad_stats_noalloc(_ptr(grad), _dtype(gdtype), n, inv_loss_scale,
                                         _ptr(d_scale), _ptr(d_stats), _stream(stream)))


def zero_bucket_flatten_stats_workspace(numel: Sequence[int], range_begin: int,
                                        count: int) -> int:
    nums = numel if isinstance(numel, ctypes.Array) else (U64 * len(numel))(*numel)
    out = ctypes.c_size_t()
    _check(lib().zero_bucket_flatten_stats_workspace(nums, len(numel), range_begin, count,
                                                     ctypes.byref(out)))
    return out.value


def zero_bucket_flatten_stats(tensors: Sequence, numel: Optional[Sequence[int]], gdtype,
                              range_begin: int, count: int, dst, inv_loss_scale: float,
                              workspace, ws_bytes: int, d_stats, stream=None,
                              d_scale=None) -> None:
    """tensors and numel as for zero_bucket_flatten."""
    ptrs, nums = tensor_table(tensors, numel)
    _check(lib().zero_bucket_flatten_stats(ptrs, nums, len(ptrs), _dtype(gdtype), range_begin,
                                           count, _ptr(dst), inv_loss_scale, _ptr(d_scale),
                                           _ptr(workspace), ws_bytes, _ptr(d_stats),
                                           _stream(stream)))


def zero_adam_step(hp: AdamW, grad, gdtype, master, exp_avg, exp_avg_sq, param_out, pdtype,
                   n: int, d_stats, d_state, stream=None, d_scale=None) -> None:
    _check(lib().zero_adam_step(ctypes.byref(hp), _ptr(grad), _dtype(gdtype), _ptr(master),
                                _ptr(exp_avg), _ptr(exp_avg_sq), _ptr(param_out), _dtype(pdtype),
                                n, _ptr(d_stats), _ptr(d_scale), _ptr(d_state),
                                _stream(stream)))


def zero_grad_stats_tensors(tensors: Sequence, numel: Optional[Sequence[int]], gdtype,
                            range_begin: int, count: int, inv_loss_scale: float, workspace,
                            ws_bytes: int, d_stats, stream=None, d_scale=None) -> None:
    """tensors and numel as for zero_bucket_flatten; the gradients are read in
    place (workspace from zero_bucket_flatten_stats_workspace)."""
    ptrs, nums = tensor_table(tensors, numel)
    _check(lib().zero_grad_stats_tensors(ptrs, nums, len(ptrs), _dtype(gdtype), range_begin,
                                         count, inv_loss_scale, _ptr(d_scale), _ptr(workspace),
                                         ws_bytes, _ptr(d_stats), _stream(stream)))


def zero_adam_step_tensors(hp: AdamW, tensors: Sequence, numel: Optional[Sequence[int]], gdtype,
                           range_begin: int, count: int, master, exp_avg, exp_avg_sq, param_out,
                           pdtype, d_stats, d_state, stream=None, d_scale=None) -> None:
    """zero_adam_step with the gradients read in place from the tensors."""
    ptrs, nums = tensor_table(tensors, numel)
    _check(lib().zero_adam_step_tensors(ctypes.byref(hp), ptrs, nums, len(ptrs), _dtype(gdtype),
                                        range_begin, count, _ptr(master), _ptr(exp_avg),
                                        _ptr(exp_avg_sq), _ptr(param_out), _dtype(pdtype),
                                        _ptr(d_stats), _ptr(d_scale), _ptr(d_state),
                                        _stream(stream)))


def zero_loss_scale_init(cfg: LossScaler, d_scale, stream=None) -> None:
    _check(lib().zero_loss_scale_init(ctypes.byref(cfg), _ptr(d_scale), _stream(stream)))


def zero_loss_scale_update(cfg: LossScaler, d_stats, d_scale, stream=None) -> None:
    _check(lib().zero_loss_scale_update(ctypes.byref(cfg), _ptr(d_stats), _ptr(d_scale),
                                        _stream(stream)))


# ------------------------------------------ optimizer state in host memory
def zero_offload_staging_bytes(chunk_elems: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().zero_offload_staging_bytes(chunk_elems, ctypes.byref(out)))
    return out.value


def zero_offload_adam_step(hp: AdamW, grad, gdtype, master_host, exp_avg_host, exp_avg_sq_host,
                           param_out, pdtype, n: int, d_stats, d_state, staging,
                           staging_bytes: int, stream=None, d_scale=None) -> None:
    """master/exp_avg/exp_avg_sq: host tensors (or addresses); staging: pinned
    host memory; grad, param_out, d_stats, d_state: device."""
    _check(lib().zero_offload_adam_step(ctypes.byref(hp), _ptr(grad), _dtype(gdtype),
                                        _ptr(master_host, host=True),
                                        _ptr(exp_avg_host, host=True),
                                        _ptr(exp_avg_sq_host, host=True), _ptr(param_out),
                                        _dtype(pdtype), n, _ptr(d_stats), _ptr(d_scale),
                                        _ptr(d_state), _ptr(staging, host=True), staging_bytes,
                                        _stream(stream)))


# ---------------------------------------------------- sharded checkpoints
def zero_ckpt_save(path: str, psi: int, nd: int, rank: int, master, exp_avg, exp_avg_sq,
                   d_state, stream=None, d_scale=None) -> None:
    _check(lib().zero_ckpt_save(os.fsencode(path), psi, nd, rank, _ptr(master), _ptr(exp_avg),
                                _ptr(exp_avg_sq), _ptr(d_state), _ptr(d_scale),
                                _stream(stream)))


def zero_ckpt_read_header(path: str) -> CkptHeader:
    h = CkptHeader()
    _check(lib().zero_ckpt_read_header(os.fsencode(path), ctypes.byref(h)))
    return h


def zero_ckpt_load(paths: Sequence[str], psi: int, nd: int, rank: int, master, exp_avg,
                   exp_avg_sq, d_state, stream=None, d_scale=None) -> None:
    arr = (ctypes.c_char_p * len(paths))(*[os.fsencode(p) for p in paths])
    _check(lib().zero_ckpt_load(arr, len(paths), psi, nd, rank, _ptr(master), _ptr(exp_avg),
                                _ptr(exp_avg_sq), _ptr(d_state), _ptr(d_scale),
                                _stream(stream)))


# ----------------------------------------------- device struct conveniences
def new_grad_stats(device) -> torch.Tensor:
    """A zeroed device buffer for one zero_grad_stats_t."""
    return torch.zeros(ctypes.sizeof(GradStats), dtype=torch.uint8, device=device)


def new_adam_state(device) -> torch.Tensor:
    """A zeroed device buffer for one zero_adam_state_t (step 0)."""
    return torch.zeros(ctypes.sizeof(AdamState), dtype=torch.uint8, device=device)


def new_loss_scale(device) -> torch.Tensor:
    """A device buffer for one zero_loss_scale_t (set it with zero_loss_scale_init)."""
    return torch.zeros(ctypes.sizeof(LossScale), dtype=torch.uint8, device=device)


def read_loss_scale(buf: torch.Tensor) -> LossScale:
    """Synchronising copy of a device zero_loss_scale_t."""
    return LossScale.from_buffer_copy(bytes(buf.cpu().numpy()))


def loss_scaler(init_scale=2.0 ** 16, growth_factor=2.0, backoff_factor=0.5,
                growth_interval=2000, min_scale=1.0, max_scale=float("inf")) -> LossScaler:
    return LossScaler(init_scale, growth_factor, backoff_factor, growth_interval, min_scale,
                      max_scale)


def new_workspace(n: int, device) -> torch.Tensor:
    return torch.empty(max(zero_grad_stats_workspace(n), 16), dtype=torch.uint8, device=device)


def read_grad_stats(buf: torch.Tensor) -> GradStats:
    """Synchronising copy of a device zero_grad_stats_t."""
    return GradStats.from_buffer_copy(bytes(buf.cpu().numpy()))


def read_adam_state(buf: torch.Tensor) -> AdamState:
    """Synchronising copy of a device zero_adam_state_t."""
    return AdamState.from_buffer_copy(bytes(buf.cpu().numpy()))


def adamw(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=0.0,
          inv_loss_scale=1.0) -> AdamW:
    return AdamW(lr, beta1, beta2, eps, weight_decay, max_grad_norm, inv_loss_scale)
