"""LayerNorm / RMSNorm backward for AMD MI355X (gfx950): Python binding.

Thin ctypes marshalling over the C ABI in ``include/norm_bwd.h`` (library
``rmsnorm_backward_amd/_lib/libnorm_bwd.so``). Every step of the backward pass
runs in the library's HIP kernels on the tensors' GPU; this module only checks
tensor metadata, allocates outputs and the workspace with ``torch.empty``
(PyTorch supplies device memory and the current stream), and forwards raw
pointers. There is no CPU fallback: without the built library, or with tensors
that are not on a GPU, the calls raise.

The functions carry the C names:

* ``norm_bwd_layernorm(x, dy, gamma, mean, rstd, eps)`` -> (dx, dgamma, dbeta)
* ``norm_bwd_rmsnorm(x, dy, gamma, rstd, eps)`` -> (dx, dgamma, dbeta or None)
* ``norm_fwd_layernorm(x, gamma, beta, eps)`` -> (y, mean, rstd),
  ``norm_fwd_rmsnorm(x, gamma, eps)`` -> (y, rstd): the forward pass that
  produces the statistics the backward consumes
* ``norm_bwd_ex(kind, x, dy, gamma, mean, rstd, eps, ...)``: row-strided 2-D
  views, an explicit group count, accumulation into given dgamma/dbeta
* ``norm_bwd_ex_static(...)``: the same with the workspace in the library's
  static scratch (no workspace argument), for callers that cannot allocate
* ``norm_bwd_wgrad(kind, x, dy, mean, rstd)`` -> (dgamma, dbeta or None): the
  weight gradients alone (column walk, no workspace)
* ``norm_bwd_workspace_bytes``, ``norm_bwd_make_plan``, ``norm_bwd_execute``,
  ``norm_bwd_execute_partials``, ``norm_bwd_reduce_partials``,
  ``norm_bwd_probe_copy``, ``norm_bwd_probe_triad``, ``norm_bwd_status_string``,
  ``norm_bwd_last_error``.

Every tensor handed to the library is checked first: on x's GPU, contiguous
unless a row stride is taken, and of the dtype and element count the kernels
assume. The library only sees raw pointers, so this is what keeps a kernel
inside the tensors. ``rmsnorm_backward_amd.autograd`` wraps the forward and
backward as torch.autograd Functions and nn.Modules.
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libnorm_bwd.so")

# Codes from include/norm_bwd.h
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
F32, F16, BF16 = 0, 1, 2
LAYERNORM, RMSNORM = 0, 1
_DTYPE_CODE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
_CODE_DTYPE = {v: k for k, v in _DTYPE_CODE.items()}
_KIND_CODE = {"layernorm": LAYERNORM, "rmsnorm": RMSNORM, LAYERNORM: LAYERNORM, RMSNORM: RMSNORM}


class NormBwdError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class NormBwdPlan(ctypes.Structure):
    """Mirror of norm_bwd_plan_t."""
    _fields_ = [
        ("kind", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
        ("with_dbeta", ctypes.c_int32), ("vec", ctypes.c_int32),
        ("M", ctypes.c_int64), ("N", ctypes.c_int64),
        ("groups", ctypes.c_int64), ("rows_per_group", ctypes.c_int64),
        ("chunks", ctypes.c_int32), ("waves_per_row", ctypes.c_int32),
        ("rows_in_flight", ctypes.c_int32), ("threads", ctypes.c_int32),
        ("grid", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
        ("rows_per_wave", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}

    def copy(self) -> "NormBwdPlan":
        c = NormBwdPlan()
        ctypes.memmove(ctypes.byref(c), ctypes.byref(self), ctypes.sizeof(self))
        return c


ACCUMULATE = 1
# bytes of the static scratch of norm_bwd_ex_static (NORM_BWD_STATIC_SCRATCH_BYTES)
STATIC_SCRATCH_BYTES = 32 << 20


class NormBwdArgs(ctypes.Structure):
    """Mirror of norm_bwd_args_t (the argument block of norm_bwd_ex)."""
    _fields_ = [
        ("kind", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
        ("wgrad_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("groups", ctypes.c_int64),
        ("x", ctypes.c_void_p), ("ldx", ctypes.c_int64),
        ("dy", ctypes.c_void_p), ("lddy", ctypes.c_int64),
        ("gamma", ctypes.c_void_p), ("mean", ctypes.c_void_p), ("rstd", ctypes.c_void_p),
        ("dx", ctypes.c_void_p), ("lddx", ctypes.c_int64),
        ("dgamma", ctypes.c_void_p), ("dbeta", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p), ("eps", ctypes.c_float), ("reserved", ctypes.c_int32),
    ]


_lock = threading.Lock()
_lib = None


def library_path() -> str:
    return LIB_PATH


def _declare(lib, strict: bool = True) -> None:
    """Set the argument and result types of the library's entry points.
    strict=False leaves out the entry points a build does not export (an
    older build, loaded to compare with)."""
    vp, i32, i64, sz, fp = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                            ctypes.c_size_t, ctypes.c_float)
    P = ctypes.POINTER(NormBwdPlan)
    sigs = {
        "norm_bwd_layernorm": [vp, vp, vp, vp, vp, i64, i64, i32, i32, fp, vp, vp, vp, vp, sz, vp],
        "norm_bwd_rmsnorm": [vp, vp, vp, vp, i64, i64, i32, i32, fp, vp, vp, vp, vp, sz, vp],
        "norm_bwd_workspace_bytes": [i32, i64, i64, i32, i32],
        "norm_bwd_make_plan": [i32, i64, i64, i32, i32, i64, P],
        "norm_bwd_execute": [P, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp],
        "norm_bwd_execute_partials": [P, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "norm_bwd_reduce_partials": [i64, i64, i32, vp, sz, vp, vp, vp],
        "norm_bwd_status_string": [i32],
        "norm_bwd_last_error": [],
        "norm_bwd_probe_copy": [vp, vp, sz, vp],
        "norm_bwd_probe_triad": [vp, vp, vp, sz, i32, i32, vp],
        "norm_bwd_probe_triad_policy": [vp, vp, vp, sz, i32, i32, i32, vp],
        "norm_fwd_layernorm": [vp, vp, vp, i64, i64, i32, fp, vp, vp, vp, vp],
        "norm_fwd_rmsnorm": [vp, vp, i64, i64, i32, fp, vp, vp, vp],
        "norm_bwd_ex": [ctypes.POINTER(NormBwdArgs)],
        "norm_bwd_ex_static": [ctypes.POINTER(NormBwdArgs)],
        "norm_bwd_wgrad": [i32, vp, vp, vp, vp, i64, i64, i32, i32, vp, vp, ctypes.c_uint, vp],
    }
    restypes = {"norm_bwd_workspace_bytes": ctypes.c_size_t,
                "norm_bwd_status_string": ctypes.c_char_p,
                "norm_bwd_last_error": ctypes.c_char_p}
    for name, args in sigs.items():
        f = getattr(lib, name, None)
        if f is None:
            if strict:
                raise RuntimeError(f"the library does not export {name}")
            continue
        f.argtypes = args
        f.restype = restypes.get(name, ctypes.c_int)


def load_library():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -m rmsnorm_backward_amd._build "
                "or __graft_entry__.build()). There is no CPU fallback.")
        lib = ctypes.CDLL(LIB_PATH)
        _declare(lib)
        _lib = lib
        return lib


def load_library_at(path: str):
    """Another build of the library at `path`, loaded beside this one (its
    own symbols and kernels), for timing two builds on the same buffers.
    Entry points that build does not export stay undeclared."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} does not exist")
    lib = ctypes.CDLL(os.path.abspath(path))
    _declare(lib, strict=False)
    return lib


def norm_bwd_status_string(status: int) -> str:
    return load_library().norm_bwd_status_string(status).decode()


def norm_bwd_last_error() -> str:
    return load_library().norm_bwd_last_error().decode()


def _check(status: int):
    if status != OK:
        raise NormBwdError(status, norm_bwd_last_error() or norm_bwd_status_string(status))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device) -> ctypes.c_void_p:
    """The stream to launch on: torch's current stream of the tensors' device
    by default. A torch stream of another device is refused (its kernels
    would touch this device's memory from there); a raw handle (int) is the
    caller's responsibility."""
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if hasattr(stream, "cuda_stream"):
        sdev = getattr(stream, "device", None)
        if sdev is not None and torch.device(sdev) != torch.device(device):
            raise ValueError(f"stream is on {sdev}, the tensors on {device}")
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _gpu_any(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device}); there is no CPU path")


def _gpu(t: torch.Tensor, name: str):
    _gpu_any(t, name)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _tensor(t: torch.Tensor, name: str, dev: torch.device, dtype: Optional[torch.dtype] = None,
            numel: Optional[int] = None, contiguous: bool = True):
    """Check a tensor the library reads or writes through a raw pointer: on
    x's GPU, contiguous (unless the entry point takes a row stride), and of
    the dtype and element count the kernels assume, so no kernel can read or
    write past it."""
    (_gpu if contiguous else _gpu_any)(t, name)
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, x on {dev}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements (got {t.numel()})")


def _addr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _rows(x: torch.Tensor):
    if x.dim() < 1:
        raise ValueError("x must have at least one dimension (features last)")
    N = x.shape[-1]
    M = 1
    for d in x.shape[:-1]:
        M *= d
    return M, N


def _code(dtype: torch.dtype, what: str) -> int:
    try:
        return _DTYPE_CODE[dtype]
    except KeyError:
        raise ValueError(f"{what} dtype {dtype} not supported (float32, float16, bfloat16)")


def norm_bwd_workspace_bytes(kind, M: int, N: int, io_dtype, with_dbeta: bool) -> int:
    code = io_dtype if isinstance(io_dtype, int) else _code(io_dtype, "io")
    n = load_library().norm_bwd_workspace_bytes(_KIND_CODE[kind], M, N, code, int(bool(with_dbeta)))
    if n == ctypes.c_size_t(-1).value:
        raise NormBwdError(ERR_INVALID_ARG, "invalid arguments for norm_bwd_workspace_bytes")
    return n


def _auto_workspace(kind, M, N, io, with_dbeta) -> int:
    """Workspace for an automatic plan of either statistics mode (fused or
    wide-row path). An invalid shape raises with the plan call's status."""
    n = load_library().norm_bwd_workspace_bytes(_KIND_CODE[kind], M, N, io, int(bool(with_dbeta)))
    if n == ctypes.c_size_t(-1).value:
        norm_bwd_make_plan(kind, M, N, io, with_dbeta)      # raises the precise status
        raise NormBwdError(ERR_INVALID_ARG, "invalid arguments for norm_bwd_workspace_bytes")
    return n


def norm_bwd_make_plan(kind, M: int, N: int, io_dtype, with_dbeta: bool,
                       groups: int = 0) -> NormBwdPlan:
    code = io_dtype if isinstance(io_dtype, int) else _code(io_dtype, "io")
    plan = NormBwdPlan()
    _check(load_library().norm_bwd_make_plan(_KIND_CODE[kind], M, N, code,
                                              int(bool(with_dbeta)), groups, ctypes.byref(plan)))
    return plan


def _backward(kind, x, dy, gamma, mean, rstd, eps, wgrad_dtype, dx, dgamma, dbeta,
              with_dbeta, workspace, stream, plan: Optional[NormBwdPlan]):
    lib = load_library()
    _gpu(x, "x")
    dev = x.device
    # rstd None (LayerNorm: mean and rstd None) selects the recompute mode
    recompute = rstd is None
    if kind == LAYERNORM and (mean is None) != recompute:
        raise ValueError("LayerNorm takes both mean and rstd, or neither (recompute)")
    if recompute and plan is not None:
        raise ValueError("an explicit plan needs the saved statistics")
    M, N = _rows(x)
    io = _code(x.dtype, "x")
    if plan is not None and (plan.M, plan.N, plan.io_dtype) != (M, N, io):
        raise ValueError(f"the plan is for {plan.M}x{plan.N} of dtype code {plan.io_dtype}, "
                         f"x is {M}x{N} of dtype code {io}")
    if not isinstance(dy, torch.Tensor) or dy.shape != x.shape:
        raise ValueError("dy must have x's shape")
    _tensor(dy, "dy", dev, x.dtype)
    _tensor(gamma, "gamma", dev, x.dtype, N)
    for t, n in ((rstd, "rstd"), (mean if kind == LAYERNORM else None, "mean")):
        if t is not None:
            _tensor(t, n, dev, torch.float32, M)
    # dgamma/dbeta are written in wgrad_dtype: by default that of a given dgamma
    wgrad_dtype = wgrad_dtype or (dgamma.dtype if dgamma is not None else torch.float32)
    wcode = _code(wgrad_dtype, "wgrad")
    if dx is None:
        dx = torch.empty_like(x)
    if dgamma is None:
        dgamma = torch.empty(N, dtype=wgrad_dtype, device=dev)
    if with_dbeta and dbeta is None:
        dbeta = torch.empty(N, dtype=wgrad_dtype, device=dev)
    _tensor(dx, "dx", dev, x.dtype, M * N)
    _tensor(dgamma, "dgamma", dev, wgrad_dtype, N)
    if dbeta is not None:
        _tensor(dbeta, "dbeta", dev, wgrad_dtype, N)
    if workspace is not None:
        _tensor(workspace, "workspace", dev)
    s = _stream(stream, dev)
    with torch.cuda.device(dev):
        if plan is None:
            need = _auto_workspace(kind, M, N, io, dbeta is not None)
            if workspace is None:
                workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
            wsb = workspace.numel() * workspace.element_size()
            if kind == LAYERNORM:
                st = lib.norm_bwd_layernorm(_ptr(x), _ptr(dy), _ptr(gamma), _ptr(mean), _ptr(rstd),
                                            M, N, io, wcode, float(eps), _ptr(dx), _ptr(dgamma),
                                            _ptr(dbeta), _ptr(workspace), wsb, s)
            else:
                st = lib.norm_bwd_rmsnorm(_ptr(x), _ptr(dy), _ptr(gamma), _ptr(rstd), M, N, io,
                                          wcode, float(eps), _ptr(dx), _ptr(dgamma), _ptr(dbeta),
                                          _ptr(workspace), wsb, s)
        else:
            if workspace is None:
                workspace = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
            wsb = workspace.numel() * workspace.element_size()
            st = lib.norm_bwd_execute(ctypes.byref(plan), _ptr(x), _ptr(dy), _ptr(gamma),
                                      _ptr(mean) if kind == LAYERNORM else None, _ptr(rstd),
                                      wcode, _ptr(dx), _ptr(dgamma), _ptr(dbeta),
                                      _ptr(workspace), wsb, s)
    _check(st)
    return dx, dgamma, dbeta


def norm_bwd_layernorm(x: torch.Tensor, dy: torch.Tensor, gamma: torch.Tensor,
                       mean: Optional[torch.Tensor], rstd: Optional[torch.Tensor],
                       eps: float = 1e-5, *,
                       wgrad_dtype: Optional[torch.dtype] = None, dx=None, dgamma=None,
                       dbeta=None, with_dbeta: bool = True, workspace=None, stream=None
                       ) -> Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """LayerNorm backward on the GPU: returns (dx, dgamma, dbeta). mean = rstd =
    None recomputes the statistics from x with eps."""
    return _backward(LAYERNORM, x, dy, gamma, mean, rstd, eps, wgrad_dtype, dx, dgamma, dbeta,
                     with_dbeta or dbeta is not None, workspace, stream, None)


def norm_bwd_rmsnorm(x: torch.Tensor, dy: torch.Tensor, gamma: torch.Tensor,
                     rstd: Optional[torch.Tensor], eps: float = 1e-6, *,
                     wgrad_dtype: Optional[torch.dtype] = None, dx=None, dgamma=None,
                     dbeta=None, with_dbeta: bool = False, workspace=None, stream=None
                     ) -> Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """RMSNorm backward on the GPU: returns (dx, dgamma, dbeta or None). rstd =
    None recomputes it from x with eps."""
    return _backward(RMSNORM, x, dy, gamma, None, rstd, eps, wgrad_dtype, dx, dgamma, dbeta,
                     with_dbeta or dbeta is not None, workspace, stream, None)


def _rows2d(t: torch.Tensor, name: str):
    """(rows, cols, row stride) of a 2-D view with unit column stride."""
    _gpu_any(t, name)
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a 2-D view with unit column stride")
    return t.shape[0], t.shape[1], (t.stride(0) if t.shape[0] > 1 else t.shape[1])


def norm_bwd_ex(kind: str, x: torch.Tensor, dy: torch.Tensor, gamma: torch.Tensor,
                mean: Optional[torch.Tensor] = None, rstd: Optional[torch.Tensor] = None,
                eps: float = 1e-5, *, wgrad_dtype: Optional[torch.dtype] = None, dx=None,
                dgamma=None, dbeta=None, with_dbeta: Optional[bool] = None,
                accumulate: bool = False, groups: int = 0, workspace=None, stream=None):
    """Extended backward (norm_bwd_ex): x, dy (and dx) may be row-strided 2-D
    views; accumulate=True adds into the given dgamma/dbeta. Returns
    (dx, dgamma, dbeta)."""
    return _ex(False, kind, x, dy, gamma, mean, rstd, eps, wgrad_dtype, dx, dgamma, dbeta,
               with_dbeta, accumulate, groups, workspace, stream)


def norm_bwd_ex_static(kind: str, x: torch.Tensor, dy: torch.Tensor, gamma: torch.Tensor,
                       mean: Optional[torch.Tensor] = None, rstd: Optional[torch.Tensor] = None,
                       eps: float = 1e-5, *, wgrad_dtype: Optional[torch.dtype] = None, dx=None,
                       dgamma=None, dbeta=None, with_dbeta: Optional[bool] = None,
                       accumulate: bool = False, groups: int = 0, stream=None):
    """norm_bwd_ex_static: norm_bwd_ex with the workspace in the library's
    static scratch (no workspace argument; the library allocates nothing).
    Outputs not given are allocated here with torch.empty; a caller that must
    not allocate passes dx, dgamma (and dbeta). Returns (dx, dgamma, dbeta)."""
    return _ex(True, kind, x, dy, gamma, mean, rstd, eps, wgrad_dtype, dx, dgamma, dbeta,
               with_dbeta, accumulate, groups, None, stream)


def _ex(static, kind, x, dy, gamma, mean, rstd, eps, wgrad_dtype, dx, dgamma, dbeta, with_dbeta,
        accumulate, groups, workspace, stream):
    lib = load_library()
    code = kind = _KIND_CODE[kind]
    M, N, ldx = _rows2d(x, "x")
    dev = x.device
    M2, N2, lddy = _rows2d(dy, "dy")
    if (M2, N2) != (M, N):
        raise ValueError("dy must match x")
    _tensor(dy, "dy", dev, x.dtype, contiguous=False)
    _tensor(gamma, "gamma", dev, x.dtype, N)
    if kind == RMSNORM:
        mean = None
    for t, n in ((mean, "mean"), (rstd, "rstd")):
        if t is not None:
            _tensor(t, n, dev, torch.float32, M)
    if with_dbeta is None:
        with_dbeta = dbeta is not None or (kind == LAYERNORM and not accumulate)
    if accumulate and (dgamma is None or (with_dbeta and dbeta is None)):
        raise ValueError("accumulate=True needs the dgamma (and dbeta) to add into")
    wgrad_dtype = wgrad_dtype or (dgamma.dtype if dgamma is not None else torch.float32)
    if dx is None:
        dx = torch.empty((M, N), dtype=x.dtype, device=dev)
    M3, N3, lddx = _rows2d(dx, "dx")
    if (M3, N3) != (M, N):
        raise ValueError("dx must be [M, N]")
    _tensor(dx, "dx", dev, x.dtype, contiguous=False)
    if dgamma is None:
        dgamma = torch.empty(N, dtype=wgrad_dtype, device=dev)
    if with_dbeta and dbeta is None:
        dbeta = torch.empty(N, dtype=wgrad_dtype, device=dev)
    for t, n in ((dgamma, "dgamma"), (dbeta, "dbeta")):
        if t is not None:
            _tensor(t, n, dev, wgrad_dtype, N)
    io = _code(x.dtype, "x")
    if not static:
        if workspace is None:
            need = (norm_bwd_make_plan(kind, M, N, io, dbeta is not None, groups).workspace_bytes
                    if groups else _auto_workspace(kind, M, N, io, dbeta is not None))
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        _tensor(workspace, "workspace", dev)
    a = NormBwdArgs()
    a.kind, a.io_dtype, a.wgrad_dtype = code, io, _code(wgrad_dtype, "wgrad")
    a.flags = ACCUMULATE if accumulate else 0
    a.M, a.N, a.groups = M, N, groups
    a.x, a.ldx = _addr(x), ldx
    a.dy, a.lddy = _addr(dy), lddy
    a.gamma, a.mean, a.rstd = _addr(gamma), _addr(mean), _addr(rstd)
    a.dx, a.lddx = _addr(dx), lddx
    a.dgamma, a.dbeta = _addr(dgamma), _addr(dbeta)
    if not static:
        a.workspace = _addr(workspace)
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    a.stream = _stream(stream, dev).value
    a.eps = float(eps)
    with torch.cuda.device(dev):
        st = (lib.norm_bwd_ex_static if static else lib.norm_bwd_ex)(ctypes.byref(a))
    _check(st)
    return dx, dgamma, dbeta


def norm_bwd_wgrad(kind, x: torch.Tensor, dy: torch.Tensor, mean: Optional[torch.Tensor],
                   rstd: torch.Tensor, *, wgrad_dtype: Optional[torch.dtype] = None,
                   dgamma=None, dbeta=None, with_dbeta: Optional[bool] = None,
                   accumulate: bool = False, stream=None):
    """dgamma (and dbeta) alone by the column walk (no dx, no workspace)."""
    lib = load_library()
    code = kind = _KIND_CODE[kind]
    _gpu(x, "x")
    dev = x.device
    M, N = _rows(x)
    if not isinstance(dy, torch.Tensor) or dy.shape != x.shape:
        raise ValueError("dy must have x's shape")
    _tensor(dy, "dy", dev, x.dtype)
    if kind == LAYERNORM:
        _tensor(mean, "mean", dev, torch.float32, M)
    else:
        mean = None
    _tensor(rstd, "rstd", dev, torch.float32, M)
    if with_dbeta is None:
        with_dbeta = dbeta is not None or (kind == LAYERNORM and not accumulate)
    if accumulate and (dgamma is None or (with_dbeta and dbeta is None)):
        raise ValueError("accumulate=True needs the dgamma (and dbeta) to add into")
    wgrad_dtype = wgrad_dtype or (dgamma.dtype if dgamma is not None else torch.float32)
    if dgamma is None:
        dgamma = torch.empty(N, dtype=wgrad_dtype, device=dev)
    if with_dbeta and dbeta is None:
        dbeta = torch.empty(N, dtype=wgrad_dtype, device=dev)
    for t, n in ((dgamma, "dgamma"), (dbeta, "dbeta")):
        if t is not None:
            _tensor(t, n, dev, wgrad_dtype, N)
    s = _stream(stream, dev)
    with torch.cuda.device(dev):
        st = lib.norm_bwd_wgrad(code, _ptr(x), _ptr(dy), _ptr(mean), _ptr(rstd), M, N,
                                _code(x.dtype, "x"), _code(wgrad_dtype, "wgrad"), _ptr(dgamma),
                                _ptr(dbeta), ACCUMULATE if accumulate else 0, s)
    _check(st)
    return dgamma, dbeta


def norm_bwd_execute(plan: NormBwdPlan, x, dy, gamma, mean, rstd, *, wgrad_dtype=None,
                     dx=None, dgamma=None, dbeta=None, workspace=None, stream=None):
    """Run an explicit plan (kernel A then kernel B)."""
    kind = plan.kind
    return _backward(kind, x, dy, gamma, mean, rstd, 0.0, wgrad_dtype, dx, dgamma, dbeta,
                     bool(plan.with_dbeta), workspace, stream, plan)


def norm_bwd_execute_partials(plan: NormBwdPlan, x, dy, gamma, mean, rstd, dx, workspace,
                              stream=None):
    """Kernel A alone (dx and the per-group partials in `workspace`)."""
    lib = load_library()
    _gpu(x, "x")
    dev = x.device
    dt = _CODE_DTYPE.get(plan.io_dtype)
    if dt is None:
        raise ValueError(f"plan.io_dtype {plan.io_dtype} unknown")
    M, N = plan.M, plan.N
    for t, n in ((x, "x"), (dy, "dy"), (dx, "dx")):
        _tensor(t, n, dev, dt, M * N)
    _tensor(gamma, "gamma", dev, dt, N)
    _tensor(rstd, "rstd", dev, torch.float32, M)
    if plan.kind == LAYERNORM:
        _tensor(mean, "mean", dev, torch.float32, M)
    _tensor(workspace, "workspace", dev)
    s = _stream(stream, dev)
    with torch.cuda.device(x.device):
        st = lib.norm_bwd_execute_partials(
            ctypes.byref(plan), _ptr(x), _ptr(dy), _ptr(gamma),
            _ptr(mean) if plan.kind == LAYERNORM else None, _ptr(rstd), _ptr(dx),
            _ptr(workspace), workspace.numel() * workspace.element_size(), s)
    _check(st)


def norm_bwd_reduce_partials(groups: int, N: int, workspace: torch.Tensor,
                             dgamma: torch.Tensor, dbeta: Optional[torch.Tensor] = None,
                             stream=None):
    """Kernel B alone: fixed-order sum of the per-group partials."""
    lib = load_library()
    _gpu(dgamma, "dgamma")
    dev = dgamma.device
    _tensor(dgamma, "dgamma", dev, None, N)
    if dbeta is not None:
        _tensor(dbeta, "dbeta", dev, dgamma.dtype, N)
    _tensor(workspace, "workspace", dev)
    s = _stream(stream, dev)
    with torch.cuda.device(dgamma.device):
        st = lib.norm_bwd_reduce_partials(groups, N, _code(dgamma.dtype, "dgamma"), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          _ptr(dgamma), _ptr(dbeta), s)
    _check(st)


def _forward(kind, x, gamma, beta, eps, y, mean, rstd, want_mean, want_rstd, stream):
    lib = load_library()
    _gpu(x, "x")
    dev = x.device
    M, N = _rows(x)
    io = _code(x.dtype, "x")
    _tensor(gamma, "gamma", dev, x.dtype, N)
    if beta is not None:
        _tensor(beta, "beta", dev, x.dtype, N)
    if y is None:
        y = torch.empty_like(x)
    if want_mean and mean is None:
        mean = torch.empty(M, dtype=torch.float32, device=dev)
    if want_rstd and rstd is None:
        rstd = torch.empty(M, dtype=torch.float32, device=dev)
    _tensor(y, "y", dev, x.dtype, M * N)
    for t, n in ((mean, "mean"), (rstd, "rstd")):
        if t is not None:
            _tensor(t, n, dev, torch.float32, M)
    s = _stream(stream, dev)
    with torch.cuda.device(dev):
        if kind == LAYERNORM:
            st = lib.norm_fwd_layernorm(_ptr(x), _ptr(gamma), _ptr(beta), M, N, io, float(eps),
                                        _ptr(y), _ptr(mean), _ptr(rstd), s)
        else:
            st = lib.norm_fwd_rmsnorm(_ptr(x), _ptr(gamma), M, N, io, float(eps), _ptr(y),
                                      _ptr(rstd), s)
    _check(st)
    return y, mean, rstd


def norm_fwd_layernorm(x: torch.Tensor, gamma: torch.Tensor, beta: Optional[torch.Tensor] = None,
                       eps: float = 1e-5, *, y=None, mean=None, rstd=None, want_stats: bool = True,
                       stream=None):
    """LayerNorm forward on the GPU: returns (y, mean, rstd) with fp32 statistics."""
    return _forward(LAYERNORM, x, gamma, beta, eps, y, mean, rstd, want_stats, want_stats, stream)


def norm_fwd_rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6, *, y=None,
                     rstd=None, want_stats: bool = True, stream=None):
    """RMSNorm forward on the GPU: returns (y, rstd) with fp32 rstd."""
    y, _, rstd = _forward(RMSNORM, x, gamma, None, eps, y, None, rstd, False, want_stats, stream)
    return y, rstd


def norm_bwd_probe_copy(src: torch.Tensor, dst: torch.Tensor, stream=None):
    """Plain streaming copy kernel (bandwidth and counter calibration)."""
    lib = load_library()
    _gpu(src, "src")
    _tensor(dst, "dst", src.device)
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst smaller than src")
    s = _stream(stream, src.device)
    with torch.cuda.device(src.device):
        _check(lib.norm_bwd_probe_copy(_ptr(src), _ptr(dst), n, s))


def norm_bwd_probe_triad(a: torch.Tensor, b: torch.Tensor, c: torch.Tensor, grid: int = 0,
                         unroll: int = 4, stream=None):
    """Streaming ceiling probe: c = a + b (32-bit words), 16-byte non-temporal
    accesses; moves 3 * a's bytes."""
    lib = load_library()
    _gpu(a, "a")
    _tensor(b, "b", a.device)
    _tensor(c, "c", a.device)
    n = a.numel() * a.element_size()
    if b.numel() * b.element_size() < n or c.numel() * c.element_size() < n:
        raise ValueError("b and c must hold at least a's bytes")
    s = _stream(stream, a.device)
    with torch.cuda.device(a.device):
        _check(lib.norm_bwd_probe_triad(_ptr(a), _ptr(b), _ptr(c), n, grid, unroll, s))


# Cache-policy bits of the gfx950 vector memory instructions, for
# norm_bwd_probe_triad_policy: any OR of them is a policy.
POLICY_SC0, POLICY_NT, POLICY_SC1 = 1, 2, 16
POLICIES = (0, 1, 2, 3, 16, 17, 18, 19)


def norm_bwd_probe_triad_policy(a: torch.Tensor, b: torch.Tensor, c: torch.Tensor,
                                unroll: int = 1, load_policy: int = POLICY_NT,
                                store_policy: int = POLICY_NT, stream=None):
    """The triad in one pass with 16-byte buffer accesses under the given
    load and store cache policies; moves 3 * a's bytes (a multiple of
    4096 * unroll)."""
    lib = load_library()
    _gpu(a, "a")
    _tensor(b, "b", a.device)
    _tensor(c, "c", a.device)
    n = a.numel() * a.element_size()
    if b.numel() * b.element_size() < n or c.numel() * c.element_size() < n:
        raise ValueError("b and c must hold at least a's bytes")
    s = _stream(stream, a.device)
    with torch.cuda.device(a.device):
        _check(lib.norm_bwd_probe_triad_policy(_ptr(a), _ptr(b), _ptr(c), n, unroll,
                                               load_policy, store_policy, s))


__all__ = [
    "norm_bwd_layernorm", "norm_bwd_rmsnorm", "norm_bwd_workspace_bytes", "norm_bwd_make_plan",
    "norm_bwd_execute", "norm_bwd_execute_partials", "norm_bwd_reduce_partials",
    "norm_bwd_probe_copy", "norm_bwd_probe_triad", "norm_bwd_probe_triad_policy",
    "POLICIES", "POLICY_SC0", "POLICY_NT", "POLICY_SC1",
    "norm_bwd_status_string", "norm_bwd_last_error", "NormBwdPlan",
    "norm_fwd_layernorm", "norm_fwd_rmsnorm", "norm_bwd_ex", "norm_bwd_ex_static",
    "NormBwdArgs", "ACCUMULATE", "STATIC_SCRATCH_BYTES",
    "norm_bwd_wgrad",
    "NormBwdError", "load_library", "library_path",
]
