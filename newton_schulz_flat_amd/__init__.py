"""MI355X (gfx950) Muon optimizer step over flat buffers.

A thin ctypes binding of ``libmuon_step.so`` (C ABI in ``include/muon_step.h``).
It only marshals arguments: every step of the computation runs in the
library's HIP kernels.  PyTorch provides device memory and the current
stream.  If the library is missing, every entry point raises: there is no
fallback.

Entry points (same names as the C ABI):

``muon_step``           momentum, Nesterov input, Newton-Schulz, decay + apply
``muon_step_noalloc``   ``muon_step`` without workspace or device allocation
``muon_step_grouped``   the same with per-matrix optimizer groups read from a
                        device table (graph-capturable) and an optional
                        bfloat16 copy of float32 weights
``muon_momentum``       momentum update and orthogonalization input only
``muon_orthogonalize``  Newton-Schulz orthogonalization (with shape scale) only
``muon_apply``          decoupled decay and update, scattered into slices
``muon_workspace_bytes``      workspace for one wave
``muon_workspace_min_bytes``  smallest workspace (the matrices then run in waves)

Descriptors are objects with ``offset, rows, cols`` and optionally
``param_offset`` (default ``offset``), ``shard_stride`` (0), ``n_shards`` (1)
and ``group`` (0), or tuples in that field order.
"""

from __future__ import annotations

import ctypes
import os
from typing import Iterable, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmuon_step.so")

MUON_OK = 0
MUON_DTYPE_F32 = 0
MUON_DTYPE_BF16 = 1
MUON_GEMM_BF16_MFMA = 0
MUON_GEMM_F32 = 1
_MODES = {"bf16": MUON_GEMM_BF16_MFMA, "f32": MUON_GEMM_F32}

#: C names of every exported entry point (mirrors include/muon_step.h).
EXPORTS = ("muon_workspace_bytes", "muon_workspace_min_bytes", "muon_step", "muon_step_grouped",
           "muon_step_noalloc", "muon_momentum", "muon_orthogonalize", "muon_apply",
           "muon_profile_begin", "muon_profile_end", "muon_status_string", "muon_last_error")


class MatrixDescC(ctypes.Structure):
    """``muon_matrix_desc_t``."""

    _fields_ = [("offset", ctypes.c_int64), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("param_offset", ctypes.c_int64), ("shard_stride", ctypes.c_int64),
                ("n_shards", ctypes.c_int32), ("group", ctypes.c_int32)]


class KernelTimeC(ctypes.Structure):
    """``muon_kernel_time_t``."""

    _fields_ = [("name", ctypes.c_char * 48), ("total_ms", ctypes.c_double),
                ("launches", ctypes.c_int64)]


class MuonError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, status: int, name: str, message: str):
        super().__init__(f"{name}: {message}")
        self.status = status
        self.name = name


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m newton_schulz_flat_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(path)
    p, i64, i32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                            ctypes.c_size_t)
    dp = ctypes.POINTER(MatrixDescC)
    lib.muon_workspace_bytes.argtypes = [dp, i64, i32, ctypes.POINTER(sz)]
    lib.muon_workspace_min_bytes.argtypes = [dp, i64, i32, ctypes.POINTER(sz)]
    lib.muon_step.argtypes = [p, i32, i64, p, p, i64, dp, i64, f32, f32, f32, i32, i32, i32, p,
                              sz, p]
    lib.muon_step_grouped.argtypes = [p, i32, i64, p, p, p, i64, dp, i64, p, ctypes.c_int32, i32,
                                      i32, p, sz, p]
    lib.muon_step_noalloc.argtypes = [p, i32, i64, p, p, i64, dp, i64, f32, f32, f32, i32, i32,
                                      i32, p]
    lib.muon_momentum.argtypes = [p, p, p, i64, dp, i64, f32, i32, p]
    lib.muon_orthogonalize.argtypes = [p, p, i64, dp, i64, i32, i32, p, sz, p]
    lib.muon_apply.argtypes = [p, i32, i64, p, i64, dp, i64, f32, f32, p]
    lib.muon_profile_begin.argtypes = []
    lib.muon_profile_end.argtypes = [ctypes.POINTER(KernelTimeC), i32, ctypes.POINTER(i32)]
    lib.muon_status_string.argtypes = [i32]
    lib.muon_status_string.restype = ctypes.c_char_p
    lib.muon_last_error.argtypes = []
    lib.muon_last_error.restype = ctypes.c_char_p
    for name in ("muon_workspace_bytes", "muon_workspace_min_bytes", "muon_step",
                 "muon_step_grouped", "muon_step_noalloc", "muon_momentum", "muon_orthogonalize",
                 "muon_apply", "muon_profile_begin", "muon_profile_end"):
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def check(status: int) -> None:
    """Raise MuonError for a non-zero status."""
    if status != MUON_OK:
        lib = load_library()
        raise MuonError(status, lib.muon_status_string(status).decode(),
                        lib.muon_last_error().decode())


def descs_array(descs: Iterable) -> ctypes.Array:
    """Descriptors as a ``muon_matrix_desc_t`` array."""
    items = list(descs)
    arr = (MatrixDescC * max(1, len(items)))()
    for k, d in enumerate(items):
        if isinstance(d, (tuple, list)):
            vals = list(d) + [None] * (7 - len(d))
            off, rows, cols, poff, stride, shards, group = vals[:7]
        else:
            off, rows, cols = d.offset, d.rows, d.cols
            poff = getattr(d, "param_offset", None)
            stride = getattr(d, "shard_stride", None)
            shards = getattr(d, "n_shards", None)
            group = getattr(d, "group", None)
        arr[k] = MatrixDescC(int(off), int(rows), int(cols), int(off if poff is None else poff),
                             int(stride or 0), int(1 if shards is None else shards),
                             int(group or 0))
    return arr


def _count(descs) -> int:
    return len(descs) if isinstance(descs, Sequence) else len(list(descs))


def _mode(mode: str) -> int:
    try:
        return _MODES[mode]
    except KeyError:
        raise ValueError(f"mode must be one of {sorted(_MODES)}, got {mode!r}") from None


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _require(t, name, dtypes):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def muon_workspace_bytes(descs, mode: str = "bf16") -> int:
    """Workspace bytes with which the descriptors run in one wave."""
    lib = load_library()
    arr = descs_array(descs)
    out = ctypes.c_size_t(0)
    check(lib.muon_workspace_bytes(arr, _count(descs), _mode(mode), ctypes.byref(out)))
    return out.value


def muon_workspace_min_bytes(descs, mode: str = "bf16") -> int:
    """Smallest workspace that runs the descriptors (in waves, one matrix or more each)."""
    lib = load_library()
    arr = descs_array(descs)
    out = ctypes.c_size_t(0)
    check(lib.muon_workspace_min_bytes(arr, _count(descs), _mode(mode), ctypes.byref(out)))
    return out.value


#: Default workspaces, one per (device, stream): calls sharing a workspace must
#: be ordered on one stream.  Each is allocated on the stream it serves, so the
#: caching allocator hands a replaced (smaller) one out again only in that
#: stream's order.
_workspaces: dict = {}


def workspace_for(descs, mode: str, device):
    """A cached uint8 workspace of at least the one-wave size, for the current
    stream of ``device``.  Not usable under graph capture (the graph would keep
    a pointer that a later, larger set frees): pass an explicit workspace there."""
    import torch
    dev = torch.device(device)
    if torch.cuda.is_current_stream_capturing():
        raise RuntimeError("pass an explicit workspace to calls made under graph capture")
    stream = torch.cuda.current_stream(dev)
    need = muon_workspace_bytes(descs, mode)
    key = (dev, stream.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        _workspaces.pop(key, None)
        with torch.cuda.stream(stream):
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def muon_step(params, grads, momentum, descs, lr: float, weight_decay: float, beta: float,
              nesterov: bool = True, ns_steps: int = 5, mode: str = "bf16", workspace=None):
    """One Muon step in place on ``params`` (f32 or bf16) and ``momentum`` (f32).

    ``workspace``: a uint8 GPU tensor (default: a cached one per device and
    stream, of the one-wave size).  A workspace smaller than
    ``muon_workspace_bytes`` but at least ``muon_workspace_min_bytes`` runs the
    matrices in waves that fit it, with identical results."""
    import torch
    _require(params, "params", (torch.float32, torch.bfloat16))
    _require(grads, "grads", (torch.float32,))
    _require(momentum, "momentum", (torch.float32,))
    if workspace is None:
        workspace = workspace_for(descs, mode, grads.device)
    lib = load_library()
    dt = MUON_DTYPE_BF16 if params.dtype == torch.bfloat16 else MUON_DTYPE_F32
    check(lib.muon_step(params.data_ptr(), dt, params.numel(), grads.data_ptr(),
                        momentum.data_ptr(), grads.numel(), descs_array(descs), _count(descs),
                        lr, weight_decay, beta, int(bool(nesterov)), int(ns_steps), _mode(mode),
                        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                        _stream(grads)))


def muon_step_noalloc(params, grads, momentum, descs, lr: float, weight_decay: float,
                      beta: float, nesterov: bool = True, ns_steps: int = 5, mode: str = "bf16"):
    """``muon_step`` without a workspace and without any device allocation:
    the library's fixed per-GPU scratch array holds every intermediate.  Calls
    that overlap on one GPU race (they share the array)."""
    import torch
    _require(params, "params", (torch.float32, torch.bfloat16))
    _require(grads, "grads", (torch.float32,))
    _require(momentum, "momentum", (torch.float32,))
    lib = load_library()
    dt = MUON_DTYPE_BF16 if params.dtype == torch.bfloat16 else MUON_DTYPE_F32
    check(lib.muon_step_noalloc(params.data_ptr(), dt, params.numel(), grads.data_ptr(),
                                momentum.data_ptr(), grads.numel(), descs_array(descs),
                                _count(descs), lr, weight_decay, beta, int(bool(nesterov)),
                                int(ns_steps), _mode(mode), _stream(grads)))


def group_table(groups, device):
    """A device table of optimizer groups for ``muon_step_grouped``: rows of
    ``(lr, weight_decay, beta, nesterov)``, stored as ``muon_group_t`` (three
    float32 and one int32) in an int32 tensor of shape (len(groups), 4)."""
    import numpy as np
    import torch
    rows = np.zeros((len(groups), 4), dtype=np.int32)
    for k, (lr, wd, beta, nesterov) in enumerate(groups):
        rows[k, :3] = np.array([lr, wd, beta], dtype=np.float32).view(np.int32)
        rows[k, 3] = int(bool(nesterov))
    return torch.from_numpy(rows).to(device)


def muon_step_grouped(params, grads, momentum, descs, groups, ns_steps: int = 5,
                      mode: str = "bf16", model_copy=None, workspace=None):
    """One Muon step with per-matrix optimizer groups: descriptor ``group`` k
    uses row k of ``groups`` (a ``group_table`` on the GPU, read when the
    kernels run).  ``model_copy`` (bf16, shaped like float32 ``params``)
    receives the updated weights rounded to bfloat16."""
    import torch
    _require(params, "params", (torch.float32, torch.bfloat16))
    _require(grads, "grads", (torch.float32,))
    _require(momentum, "momentum", (torch.float32,))
    _require(groups, "groups", (torch.int32,))
    if groups.dim() != 2 or groups.shape[1] != 4:
        raise ValueError("groups must be a group_table of shape (n_groups, 4)")
    copy_ptr = None
    if model_copy is not None:
        _require(model_copy, "model_copy", (torch.bfloat16,))
        if model_copy.numel() != params.numel():
            raise ValueError("model_copy must have as many elements as params")
        copy_ptr = model_copy.data_ptr()
    if workspace is None:
        workspace = workspace_for(descs, mode, grads.device)
    lib = load_library()
    dt = MUON_DTYPE_BF16 if params.dtype == torch.bfloat16 else MUON_DTYPE_F32
    check(lib.muon_step_grouped(params.data_ptr(), dt, params.numel(), copy_ptr, grads.data_ptr(),
                                momentum.data_ptr(), grads.numel(), descs_array(descs),
                                _count(descs), groups.data_ptr(), groups.shape[0], int(ns_steps),
                                _mode(mode), workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), _stream(grads)))


def muon_momentum(grads, momentum, u_out, descs, beta: float, nesterov: bool = True):
    """Momentum update (in place) and orthogonalization input written to ``u_out``."""
    import torch
    for t, nm in ((grads, "grads"), (momentum, "momentum"), (u_out, "u_out")):
        _require(t, nm, (torch.float32,))
    lib = load_library()
    check(lib.muon_momentum(grads.data_ptr(), momentum.data_ptr(), u_out.data_ptr(),
                            grads.numel(), descs_array(descs), _count(descs), beta,
                            int(bool(nesterov)), _stream(grads)))


def muon_orthogonalize(u, o_out, descs, ns_steps: int = 5, mode: str = "bf16", workspace=None):
    """``o_out = sqrt(max(1, rows/cols)) * NS(u)`` for every descriptor."""
    import torch
    _require(u, "u", (torch.float32,))
    _require(o_out, "o_out", (torch.float32,))
    if workspace is None:
        workspace = workspace_for(descs, mode, u.device)
    lib = load_library()
    check(lib.muon_orthogonalize(u.data_ptr(), o_out.data_ptr(), u.numel(), descs_array(descs),
                                 _count(descs), int(ns_steps), _mode(mode), workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), _stream(u)))


def muon_apply(params, updates, descs, lr: float, weight_decay: float):
    """``W <- W (1 - lr wd) - lr O`` scattered into ``params`` slices."""
    import torch
    _require(params, "params", (torch.float32, torch.bfloat16))
    _require(updates, "updates", (torch.float32,))
    lib = load_library()
    dt = MUON_DTYPE_BF16 if params.dtype == torch.bfloat16 else MUON_DTYPE_F32
    check(lib.muon_apply(params.data_ptr(), dt, params.numel(), updates.data_ptr(),
                         updates.numel(), descs_array(descs), _count(descs), lr, weight_decay,
                         _stream(updates)))


def muon_profile_begin() -> None:
    """Start timing every kernel launch with HIP events on its stream."""
    check(load_library().muon_profile_begin())


def muon_profile_end() -> dict:
    """Stop timing; returns {kernel name: (total_ms, launches)}."""
    lib = load_library()
    rows = (KernelTimeC * 64)()
    count = ctypes.c_int(0)
    check(lib.muon_profile_end(rows, 64, ctypes.byref(count)))
    return {rows[k].name.decode(): (rows[k].total_ms, rows[k].launches)
            for k in range(min(count.value, 64))}
