"""ctypes binding of the Muon C ABI (``include/muon.h``).

Argument marshalling only: tensors become device pointers, leading dimensions
and dtype codes; every step of the computation runs in the HIP library.  The
library must be built (``newton_schulz_matrix_step_amd._build.build()``); if it
is missing, loading raises instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

# the in-tree build; MUON_LIBRARY names another build of the same library to load instead
LIB_PATH = os.environ.get("MUON_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                          "libmuon_mi355x.so")
ABI_VERSION = 6   # the MUON_ABI_VERSION of the header this binding mirrors

MUON_OK = 0
MUON_ERR_INVALID_ARG = 1
MUON_ERR_DTYPE = 2
MUON_ERR_NO_DEVICE = 3
MUON_ERR_OOM = 4
MUON_ERR_HIP = 5

MUON_BF16 = 0
MUON_F32 = 1
MUON_COMPUTE_BF16 = 0
MUON_COMPUTE_FP32 = 1

MUON_INIT_PROFILE = 0x1
MUON_INIT_FAIL_ALLOC = 0x2
MUON_INIT_DEBUG = 0x4

# kernel roles (muon_role), named as in muon_kernel_stats
ROLE_NAMES = ("momentum_norm", "norm_finalize", "ns_gram", "ns_poly", "ns_axpy", "ns_axpy_update",
              "direct_update", "fill_zero", "adamw", "norm_rescale")


def profile_roles(names) -> int:
    """MUON_INIT_PROFILE_ROLES for the named roles: init flag bits that limit a
    profiling handle's events to those roles."""
    mask = 0
    for nm in names:
        mask |= 1 << ROLE_NAMES.index(nm)
    return (mask & 0x3FF) << 16

EXPORTED_SYMBOLS = (
    "muon_abi_version",
    "muon_init",
    "muon_step",
    "muon_step_noalloc",
    "muon_adamw_step",
    "muon_orthogonalize",
    "muon_read_norms",
    "muon_kernel_stats_read",
    "muon_kernel_stats_reset",
    "muon_workspace_bytes",
    "muon_destroy",
    "muon_status_str",
    "muon_last_error",
)


class muon_matrix(ctypes.Structure):
    _fields_ = [
        ("param", ctypes.c_void_p),
        ("grad", ctypes.c_void_p),
        ("momentum", ctypes.c_void_p),
        ("update_out", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("ld_param", ctypes.c_int64),
        ("ld_grad", ctypes.c_int64),
        ("ld_mom", ctypes.c_int64),
        ("ld_update", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("block_rows", ctypes.c_int32),
        ("block_cols", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class muon_adamw_tensor(ctypes.Structure):
    _fields_ = [
        ("param", ctypes.c_void_p),
        ("grad", ctypes.c_void_p),
        ("exp_avg", ctypes.c_void_p),
        ("exp_avg_sq", ctypes.c_void_p),
        ("numel", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class muon_adamw_hparams(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float),
        ("beta1", ctypes.c_float),
        ("beta2", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("weight_decay", ctypes.c_float),
        ("step", ctypes.c_int32),
    ]


class muon_hparams(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float),
        ("beta", ctypes.c_float),
        ("weight_decay", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("a", ctypes.c_float),
        ("b", ctypes.c_float),
        ("c", ctypes.c_float),
        ("nesterov", ctypes.c_int32),
        ("ns_steps", ctypes.c_int32),
        ("compute", ctypes.c_int32),
        ("coeffs", ctypes.POINTER(ctypes.c_float)),
    ]


class muon_kernel_stats(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


class MuonError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_str(status)}: {msg}" if msg else status_str(status))
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"Muon HIP library not built: {path} is missing "
                          "(run newton_schulz_matrix_step_amd._build.build())")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.muon_abi_version.restype = ctypes.c_int
    lib.muon_abi_version.argtypes = []
    if lib.muon_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} implements ABI version {lib.muon_abi_version()}, the binding expects "
                          f"{ABI_VERSION}: rebuild the library")
    lib.muon_init.restype = ctypes.c_int
    lib.muon_init.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.c_uint32]
    lib.muon_step.restype = ctypes.c_int
    lib.muon_step.argtypes = [vp, ctypes.POINTER(muon_matrix), i32, ctypes.POINTER(muon_hparams), vp]
    lib.muon_step_noalloc.restype = ctypes.c_int
    lib.muon_step_noalloc.argtypes = [vp, ctypes.POINTER(muon_matrix), i32, ctypes.POINTER(muon_hparams), vp]
    lib.muon_adamw_step.restype = ctypes.c_int
    lib.muon_adamw_step.argtypes = [vp, ctypes.POINTER(muon_adamw_tensor), i32, ctypes.POINTER(muon_adamw_hparams), vp]
    lib.muon_orthogonalize.restype = ctypes.c_int
    lib.muon_orthogonalize.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, ctypes.POINTER(muon_hparams), vp]
    lib.muon_read_norms.restype = ctypes.c_int
    lib.muon_read_norms.argtypes = [vp, ctypes.POINTER(ctypes.c_float), i32, vp]
    lib.muon_kernel_stats_read.restype = i32
    lib.muon_kernel_stats_read.argtypes = [vp, ctypes.POINTER(muon_kernel_stats), i32]
    lib.muon_kernel_stats_reset.restype = None
    lib.muon_kernel_stats_reset.argtypes = [vp]
    lib.muon_workspace_bytes.restype = i64
    lib.muon_workspace_bytes.argtypes = [vp]
    lib.muon_destroy.restype = ctypes.c_int
    lib.muon_destroy.argtypes = [vp]
    lib.muon_status_str.restype = ctypes.c_char_p
    lib.muon_status_str.argtypes = [ctypes.c_int]
    lib.muon_last_error.restype = ctypes.c_char_p
    lib.muon_last_error.argtypes = [vp]
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().muon_status_str(int(status)).decode()


def _check(handle, status: int) -> None:
    if status != MUON_OK:
        msg = load().muon_last_error(handle).decode() if handle else ""
        raise MuonError(status, msg)


@dataclass
class Hparams:
    lr: float = 0.02
    beta: float = 0.95
    weight_decay: float = 0.0
    eps: float = 1e-7
    a: float = 3.4445
    b: float = -4.7750
    c: float = 2.0315
    nesterov: bool = False
    ns_steps: int = 5
    compute: str = "bf16"      # "bf16" or "fp32"
    coeffs: Optional[Sequence[Sequence[float]]] = None   # per-iteration (a_k, b_k, c_k)

    def to_c(self) -> muon_hparams:
        comp = {"bf16": MUON_COMPUTE_BF16, "fp32": MUON_COMPUTE_FP32}.get(self.compute, -1)
        hp = muon_hparams(self.lr, self.beta, self.weight_decay, self.eps, self.a, self.b, self.c,
                          int(bool(self.nesterov)), int(self.ns_steps), comp, None)
        if self.coeffs is not None:
            flat = [float(v) for t in self.coeffs for v in t]
            if len(flat) != 3 * len(self.coeffs) or len(self.coeffs) < self.ns_steps:
                raise ValueError("coeffs: one (a, b, c) triple per iteration")
            arr = (ctypes.c_float * len(flat))(*flat)
            hp.coeffs = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
            hp._coeffs_keepalive = arr   # the array lives as long as the struct
        return hp


@dataclass
class AdamWHparams:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    step: int = 1              # 1-based step count of this update

    def to_c(self) -> muon_adamw_hparams:
        return muon_adamw_hparams(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay, int(self.step))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MUON_BF16
    if t.dtype == torch.float32:
        return MUON_F32
    return -1


def _ld(t) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("matrices must be 2-D with unit column stride")
    return int(t.stride(0))


def _stream_ptr(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def muon_abi_version() -> int:
    return int(load().muon_abi_version())


def muon_init(device: int = 0, flags: int = 0) -> int:
    h = ctypes.c_void_p()
    st = load().muon_init(ctypes.byref(h), int(device), int(flags))
    _check(None, st)
    return h.value


def _check_device_tensors(what: str, tensors, device=None):
    """Every tensor a CUDA (HIP) tensor on one device; returns that device."""
    for t in tensors:
        if not getattr(t, "is_cuda", False):
            raise ValueError(f"{what}: tensors must be on the GPU (got one on {t.device})")
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError(f"{what}: tensors on {device} and {t.device}")
    return device


def make_matrix(param, grad, momentum, update_out=None, block=(0, 0)) -> muon_matrix:
    """Describe one weight's tensors (device tensors on one device, unit column
    stride); ``block`` = (block_rows, block_cols) cuts it into separately
    orthogonalised blocks (0 = the whole dimension).  The C ABI sees only
    pointers and sizes, so shapes and dtypes are checked here: grad,
    momentum and update_out have param's shape, momentum and update_out are
    float32, param and grad share a dtype."""
    import torch
    ts = [param, grad, momentum] + ([update_out] if update_out is not None else [])
    for t in ts:
        if t.dim() != 2:
            raise ValueError("muon_step: param, grad, momentum and update_out must be 2-D")
    shape = tuple(param.shape)
    for nm, t in (("grad", grad), ("momentum", momentum), ("update_out", update_out)):
        if t is not None and tuple(t.shape) != shape:
            raise ValueError(f"muon_step: {nm} has shape {tuple(t.shape)}, param {shape}")
    if momentum.dtype != torch.float32:
        raise ValueError(f"muon_step: momentum must be float32, got {momentum.dtype}")
    if update_out is not None and update_out.dtype != torch.float32:
        raise ValueError(f"muon_step: update_out must be float32, got {update_out.dtype}")
    _check_device_tensors("muon_step", ts)
    return muon_matrix(
        param.data_ptr(), grad.data_ptr(), momentum.data_ptr(),
        update_out.data_ptr() if update_out is not None else None,
        int(param.shape[0]), int(param.shape[1]),
        _ld(param), _ld(grad), _ld(momentum), _ld(update_out) if update_out is not None else 0,
        _dtype_code(param) if _dtype_code(param) == _dtype_code(grad) else -1,
        int(block[0]), int(block[1]), 0)


def _matrices(params: Sequence, grads: Sequence, moms: Sequence, update_outs: Optional[Sequence] = None,
              blocks: Optional[Sequence] = None):
    """The muon_matrix array of one call."""
    n = len(params)
    if len(grads) != n or len(moms) != n or (update_outs is not None and len(update_outs) != n) or \
            (blocks is not None and len(blocks) != n):
        raise ValueError("params, grads, moms (and update_outs, blocks) must have the same length")
    arr = (muon_matrix * max(n, 1))()
    for i in range(n):
        arr[i] = make_matrix(params[i], grads[i], moms[i], update_outs[i] if update_outs is not None else None,
                             blocks[i] if blocks is not None else (0, 0))
    return arr, n


def muon_step(handle: int, params: Sequence, grads: Sequence, moms: Sequence, hp: Hparams,
              update_outs: Optional[Sequence] = None, stream=None, blocks: Optional[Sequence] = None) -> None:
    """One Muon step over every (param, grad, momentum) triple, on ``stream``;
    ``blocks[i]`` = (block_rows, block_cols) of matrix i, or None for all (0, 0)."""
    arr, n = _matrices(params, grads, moms, update_outs, blocks)
    c_hp = hp.to_c()
    st = load().muon_step(handle, arr, n, ctypes.byref(c_hp), _stream_ptr(stream))
    _check(handle, st)


def muon_step_noalloc(handle: int, params: Sequence, grads: Sequence, moms: Sequence, hp: Hparams,
                      update_outs: Optional[Sequence] = None, stream=None, blocks: Optional[Sequence] = None) -> None:
    """muon_step without any device allocation: the library's static
    per-GPU scratch holds every buffer beyond the caller's tensors."""
    arr, n = _matrices(params, grads, moms, update_outs, blocks)
    c_hp = hp.to_c()
    st = load().muon_step_noalloc(handle, arr, n, ctypes.byref(c_hp), _stream_ptr(stream))
    _check(handle, st)


def make_adamw_tensor(param, grad, exp_avg, exp_avg_sq) -> muon_adamw_tensor:
    """Describe one AdamW tensor (contiguous device tensors of equal size, on one device)."""
    for t in (param, grad, exp_avg, exp_avg_sq):
        if not t.is_contiguous():
            raise ValueError("AdamW tensors must be contiguous")
    n = int(param.numel())
    if any(int(t.numel()) != n for t in (grad, exp_avg, exp_avg_sq)):
        raise ValueError("param, grad, exp_avg and exp_avg_sq must have the same number of elements")
    import torch
    if exp_avg.dtype != torch.float32 or exp_avg_sq.dtype != torch.float32:
        raise ValueError("exp_avg and exp_avg_sq are float32")
    _check_device_tensors("muon_adamw_step", (param, grad, exp_avg, exp_avg_sq))
    return muon_adamw_tensor(param.data_ptr(), grad.data_ptr(), exp_avg.data_ptr(), exp_avg_sq.data_ptr(), n,
                             _dtype_code(param) if _dtype_code(param) == _dtype_code(grad) else -1, 0)


def muon_adamw_step(handle: int, params: Sequence, grads: Sequence, exp_avgs: Sequence, exp_avg_sqs: Sequence,
                    hp: AdamWHparams, stream=None) -> None:
    """One AdamW step over every (param, grad, exp_avg, exp_avg_sq) set, on ``stream``."""
    n = len(params)
    if len(grads) != n or len(exp_avgs) != n or len(exp_avg_sqs) != n:
        raise ValueError("params, grads, exp_avgs and exp_avg_sqs must have the same length")
    arr = (muon_adamw_tensor * max(n, 1))()
    for i in range(n):
        arr[i] = make_adamw_tensor(params[i], grads[i], exp_avgs[i], exp_avg_sqs[i])
    c_hp = hp.to_c()
    _check(handle, load().muon_adamw_step(handle, arr, n, ctypes.byref(c_hp), _stream_ptr(stream)))


def muon_adamw_step_raw(handle: int, arr, n: int, hp: muon_adamw_hparams, stream_ptr: int) -> int:
    """Call with prepared ctypes arguments (the benchmark's inner loop); returns the status."""
    return load().muon_adamw_step(handle, arr, n, ctypes.byref(hp), stream_ptr)


def muon_step_raw(handle: int, arr, n: int, hp: muon_hparams, stream_ptr: int) -> int:
    """Call with prepared ctypes arguments (the benchmark's inner loop); returns the status."""
    return load().muon_step(handle, arr, n, ctypes.byref(hp), stream_ptr)


def muon_orthogonalize(handle: int, inp, out, hp: Hparams, stream=None) -> None:
    """out (float32, inp's shape, same device) = Newton-Schulz(inp)."""
    import torch
    if inp.dim() != 2 or tuple(out.shape) != tuple(inp.shape):
        raise ValueError(f"muon_orthogonalize: out has shape {tuple(out.shape)}, input {tuple(inp.shape)} (2-D)")
    if out.dtype != torch.float32:
        raise ValueError(f"muon_orthogonalize: out must be float32, got {out.dtype}")
    _check_device_tensors("muon_orthogonalize", (inp, out))
    c_hp = hp.to_c()
    st = load().muon_orthogonalize(handle, inp.data_ptr(), out.data_ptr(), int(inp.shape[0]), int(inp.shape[1]),
                                   _ld(inp), _ld(out), _dtype_code(inp), ctypes.byref(c_hp), _stream_ptr(stream))
    _check(handle, st)


def muon_read_norms(handle: int, n: int, stream=None) -> List[float]:
    buf = (ctypes.c_float * max(n, 1))()
    _check(handle, load().muon_read_norms(handle, buf, int(n), _stream_ptr(stream)))
    return [float(buf[i]) for i in range(n)]


def muon_kernel_stats_read(handle: int) -> dict:
    buf = (muon_kernel_stats * 16)()
    k = load().muon_kernel_stats_read(handle, buf, 16)
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(k)}


def muon_kernel_stats_reset(handle: int) -> None:
    load().muon_kernel_stats_reset(handle)


def muon_workspace_bytes(handle: int) -> int:
    return int(load().muon_workspace_bytes(handle))


def muon_destroy(handle: int) -> None:
    _check(None, load().muon_destroy(handle))


def muon_status_str(status: int) -> str:
    return status_str(status)


def muon_last_error(handle: int) -> str:
    return load().muon_last_error(handle).decode()
