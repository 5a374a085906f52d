"""ctypes binding of libnsortho.so (argument marshalling only).

PyTorch supplies device memory (``data_ptr``) and the current HIP stream;
every step of the computation runs in the library's HIP kernels.  The
library is loaded on first use and a missing library is an error: there is
no fallback.

torch is imported before the library is loaded so that the library binds to
the same HIP runtime instance as torch (both name it ``libamdhip64.so.7``).
"""

from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple, Union

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libnsortho.so")

NS_OK = 0
NS_ERR_NONFINITE = 5
# Status word bits (the device int32 passed as `status`).
STATUS_AT_INPUT = 1 << 8
STATUS_AT_STATE = 1 << 9
STATUS_AT_ITERATE = 1 << 10
STATUS_AT_OUTPUT = 1 << 11
STATUS_AT_SPLIT = 1 << 12
STATUS_GUARD_RESTART = 1 << 16
NS_BF16, NS_FP16, NS_FP32 = 0, 1, 2
NS_STANDARD, NS_GRAM = 0, 1
NS_MAX_STEPS = 16

TUNED_ABC = (3.4445, -4.7750, 2.0315)

_DTYPE_CODE = {torch.bfloat16: NS_BF16, torch.float16: NS_FP16,
               torch.float32: NS_FP32}
_INTERNAL_CODE = {None: -1, "auto": -1, "fp16": NS_FP16, "bf16": NS_BF16,
                  "fp32": NS_FP32}
_MODE_CODE = {"standard": NS_STANDARD, "gram": NS_GRAM}


class NSError(RuntimeError):
    """A libnsortho call returned a non-zero status."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class Trace(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)),
                ("kinds", ctypes.POINTER(ctypes.c_int32)),
                ("flops", ctypes.POINTER(ctypes.c_double)),
                ("bytes", ctypes.POINTER(ctypes.c_double)),
                ("capacity", ctypes.c_int32),
                ("count", ctypes.c_int32),
                ("kind_mask", ctypes.c_uint32)]


class Options(ctypes.Structure):
    _fields_ = [("restart_mask", ctypes.c_uint32),
                ("eps", ctypes.c_float),
                ("internal", ctypes.c_int32),
                ("d_status", ctypes.c_void_p),
                ("trace", ctypes.POINTER(Trace)),
                ("tile", ctypes.c_int32),
                ("guard_threshold", ctypes.c_float)]


class Matrix(ctypes.Structure):
    """ns_matrix: one member of a grouped call."""
    _fields_ = [("data", ctypes.c_void_p),
                ("ld", ctypes.c_int64),
                ("transposed", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


KERNEL_KINDS = ("norm", "stage", "gram", "sym", "update", "threshold",
                "momentum")


_LIB = None

_SIGNATURES = {
    "ns_options_default": (None, [ctypes.POINTER(Options)]),
    "ns_workspace_size": (ctypes.c_size_t,
                          [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                           ctypes.c_int, ctypes.c_int,
                           ctypes.POINTER(Options)]),
    "ns_orthogonalize": (ctypes.c_int,
                         [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                          ctypes.c_int64, ctypes.c_int, ctypes.c_int32,
                          ctypes.POINTER(ctypes.c_float),
                          ctypes.POINTER(ctypes.c_float),
                          ctypes.POINTER(ctypes.c_float), ctypes.c_int,
                          ctypes.POINTER(Options), ctypes.c_void_p,
                          ctypes.c_size_t, ctypes.c_void_p]),
    "ns_orthogonalize_batched": (ctypes.c_int,
                                 [ctypes.c_void_p, ctypes.c_int64,
                                  ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_int, ctypes.c_int32,
                                  ctypes.POINTER(ctypes.c_float),
                                  ctypes.POINTER(ctypes.c_float),
                                  ctypes.POINTER(ctypes.c_float),
                                  ctypes.c_int, ctypes.POINTER(Options),
                                  ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p]),
    "ns_soft_threshold_workspace_size": (ctypes.c_size_t,
                                         [ctypes.c_int64, ctypes.c_int]),
    "ns_soft_threshold_split": (ctypes.c_int,
                                [ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                 ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p]),
    "ns_plan_kernels": (ctypes.c_int64,
                        [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                         ctypes.c_int, ctypes.c_int, ctypes.c_int32,
                         ctypes.POINTER(Options), ctypes.c_char_p,
                         ctypes.c_size_t]),
    "ns_plan_kernels_grouped": (ctypes.c_int64,
                                [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_int32,
                                 ctypes.POINTER(Options), ctypes.c_char_p,
                                 ctypes.c_size_t]),
    "ns_muon_workspace_size": (ctypes.c_size_t,
                               [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                ctypes.c_int, ctypes.c_int,
                                ctypes.POINTER(Options)]),
    "ns_muon_step": (ctypes.c_int,
                     [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                      ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                      ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                      ctypes.c_float, ctypes.c_float, ctypes.c_int32,
                      ctypes.c_int32, ctypes.POINTER(ctypes.c_float),
                      ctypes.POINTER(ctypes.c_float),
                      ctypes.POINTER(ctypes.c_float), ctypes.c_int,
                      ctypes.POINTER(Options), ctypes.c_void_p,
                      ctypes.c_size_t, ctypes.c_void_p]),
    "ns_grouped_workspace_size": (ctypes.c_size_t,
                                  [ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(Options)]),
    "ns_orthogonalize_grouped": (ctypes.c_int,
                                 [ctypes.POINTER(Matrix), ctypes.c_int64,
                                  ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_int, ctypes.c_int32,
                                  ctypes.POINTER(ctypes.c_float),
                                  ctypes.POINTER(ctypes.c_float),
                                  ctypes.POINTER(ctypes.c_float),
                                  ctypes.c_int, ctypes.POINTER(Options),
                                  ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p]),
    "ns_static_scratch_bytes": (ctypes.c_size_t, []),
    "ns_orthogonalize_static": (ctypes.c_int,
                                [ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_int, ctypes.c_int32,
                                 ctypes.POINTER(ctypes.c_float),
                                 ctypes.POINTER(ctypes.c_float),
                                 ctypes.POINTER(ctypes.c_float),
                                 ctypes.c_int, ctypes.POINTER(Options),
                                 ctypes.c_void_p]),
    "ns_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ns_version": (ctypes.c_int32, []),
}


def _check_single_hip_runtime() -> None:
    try:
        with open("/proc/self/maps") as f:
            maps = f.read()
    except OSError:
        return
    paths = {line.split()[-1] for line in maps.splitlines()
             if "libamdhip64" in line and "/" in line}
    if len(paths) > 1:
        raise RuntimeError("two HIP runtimes are loaded in this process: "
                           + ", ".join(sorted(paths)))


def lib() -> ctypes.CDLL:
    """Load libnsortho.so (once) and declare its signatures."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run "
                "`python -m newton_schulz_matrix_amd.build` first")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _check_single_hip_runtime()
        _LIB = handle
    return _LIB


def status_string(status: int) -> str:
    return lib().ns_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != NS_OK:
        raise NSError(status, what)


def dtype_code(dtype: torch.dtype) -> int:
    try:
        return _DTYPE_CODE[dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {dtype}; use bf16, fp16 or fp32")


def make_options(restart_mask: int = 1 << 4, eps: float = 1e-7,
                 internal: Optional[str] = None,
                 status: Optional[torch.Tensor] = None,
                 trace: Optional[Trace] = None, tile: int = 0,
                 guard: float = 0.0) -> Options:
    opt = Options()
    lib().ns_options_default(ctypes.byref(opt))
    opt.tile = int(tile)
    opt.guard_threshold = float(guard)
    opt.restart_mask = int(restart_mask)
    opt.eps = float(eps)
    opt.internal = _INTERNAL_CODE[internal]
    if status is not None:
        if status.dtype != torch.int32 or not status.is_cuda:
            raise TypeError("status must be a device int32 tensor")
        opt.d_status = status.data_ptr()
    if trace is not None:
        opt.trace = ctypes.pointer(trace)
    return opt


def _coefficients(abc, steps: int):
    """(a, b, c) as three ctypes float arrays of length ``steps``."""
    rows = list(abc) if not isinstance(abc[0], (int, float)) else [abc] * steps
    if len(rows) != steps:
        raise ValueError("abc must be one triple or `steps` triples")
    arr = ctypes.c_float * steps
    return (arr(*[float(r[0]) for r in rows]), arr(*[float(r[1]) for r in rows]),
            arr(*[float(r[2]) for r in rows]))


def _stream_handle(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def status_code(word: int) -> int:
    """The ns_status held in a status word's low byte (NS_STATUS_CODE)."""
    return int(word) & 0xFF


def _workspace(nbytes: int, device: torch.device,
               workspace: Optional[torch.Tensor]) -> Tuple[int, int, torch.Tensor]:
    """A 256-byte aligned device buffer of at least nbytes (from torch)."""
    if workspace is None:
        workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    elif not workspace.is_cuda or workspace.device != device:
        raise ValueError(f"workspace must be a device tensor on {device}")
    elif not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    ptr = workspace.data_ptr()
    pad = (-ptr) % 256
    avail = workspace.numel() * workspace.element_size() - pad
    return ptr + pad, avail, workspace


def workspace_size(rows: int, cols: int, batch: int = 1,
                   dtype: torch.dtype = torch.bfloat16,
                   mode: str = "standard", restart_mask: int = 1 << 4,
                   internal: Optional[str] = None, tile: int = 0) -> int:
    opt = make_options(restart_mask, 1e-7, internal, tile=tile)
    return int(lib().ns_workspace_size(rows, cols, batch, dtype_code(dtype),
                                       _MODE_CODE[mode], ctypes.byref(opt)))


def plan_kernels(rows: int, cols: int, batch: int = 1,
                 dtype: torch.dtype = torch.bfloat16, mode: str = "standard",
                 steps: int = 5, restart_mask: int = 1 << 4,
                 internal: Optional[str] = None, tile: int = 0,
                 guard: float = 0.0, grouped: bool = False) -> List[str]:
    """The kernel builds one call would launch (host only, no device).

    ``grouped``: a grouped call of ``batch`` matrices of this shape up to
    orientation (orthogonalize_grouped) instead of a batched one."""
    opt = make_options(restart_mask, 1e-7, internal, tile=tile, guard=guard)
    if grouped:
        fn, args = lib().ns_plan_kernels_grouped, (min(rows, cols), max(rows, cols))
    else:
        fn, args = lib().ns_plan_kernels, (rows, cols)
    name = "ns_plan_kernels_grouped" if grouped else "ns_plan_kernels"
    need = int(fn(*args, batch, dtype_code(dtype), _MODE_CODE[mode], steps,
                  ctypes.byref(opt), None, 0))
    if need < 0:
        raise NSError(1, name)
    buf = ctypes.create_string_buffer(need)
    fn(*args, batch, dtype_code(dtype), _MODE_CODE[mode], steps,
       ctypes.byref(opt), buf, need)
    return buf.value.decode().split()


def _check_matrix(x: torch.Tensor, ndim: int) -> None:
    if not x.is_cuda:
        raise ValueError("expects a device tensor")
    if x.dim() != ndim:
        raise ValueError(f"expects a {ndim}-D tensor")
    if x.stride(-1) != 1:
        raise ValueError("rows must be contiguous (stride(-1) == 1)")


def orthogonalize(x: torch.Tensor, steps: int = 5, abc=TUNED_ABC,
                  mode: str = "standard", restart_mask: int = 1 << 4,
                  eps: float = 1e-7, internal: Optional[str] = None,
                  status: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None,
                  trace: Optional[Trace] = None, tile: int = 0,
                  guard: float = 0.0) -> torch.Tensor:
    """Orthogonalize a 2-D device matrix in place; returns it.

    ``tile`` forces the products' tile edge (128, 192 or 256; 0 = automatic).
    ``guard`` > 0 turns on restarts on demand (Gram form) with that
    threshold (see ns_options.guard_threshold; 100 is the tested value).
    """
    _check_matrix(x, 2)
    rows, cols = x.shape
    ld = x.stride(0) if rows > 1 else cols
    code = dtype_code(x.dtype)
    opt = make_options(restart_mask, eps, internal, status, trace, tile, guard)
    need = int(lib().ns_workspace_size(rows, cols, 1, code, _MODE_CODE[mode],
                                       ctypes.byref(opt)))
    if need == 0:
        raise NSError(1, "ns_workspace_size")
    wptr, wbytes, keep = _workspace(need, x.device, workspace)
    a, b, c = _coefficients(abc, steps)
    st = lib().ns_orthogonalize(ctypes.c_void_p(x.data_ptr()), rows, cols, ld,
                                code, steps, a, b, c, _MODE_CODE[mode],
                                ctypes.byref(opt), ctypes.c_void_p(wptr),
                                wbytes, _stream_handle(x.device))
    _check(st, "ns_orthogonalize")
    return x


def orthogonalize_batched(x: torch.Tensor, steps: int = 5, abc=TUNED_ABC,
                          mode: str = "gram", restart_mask: int = 1 << 4,
                          eps: float = 1e-7, internal: Optional[str] = None,
                          status: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None,
                          trace: Optional[Trace] = None,
                          tile: int = 0, guard: float = 0.0) -> torch.Tensor:
    """Orthogonalize each x[e] of a [E, rows, cols] device tensor in place."""
    _check_matrix(x, 3)
    batch, rows, cols = x.shape
    ld = x.stride(1) if rows > 1 else cols
    bstride = x.stride(0) if batch > 1 else rows * ld
    code = dtype_code(x.dtype)
    opt = make_options(restart_mask, eps, internal, status, trace, tile, guard)
    need = int(lib().ns_workspace_size(rows, cols, batch, code,
                                       _MODE_CODE[mode], ctypes.byref(opt)))
    if need == 0:
        raise NSError(1, "ns_workspace_size")
    wptr, wbytes, keep = _workspace(need, x.device, workspace)
    a, b, c = _coefficients(abc, steps)
    st = lib().ns_orthogonalize_batched(
        ctypes.c_void_p(x.data_ptr()), batch, rows, cols, ld, bstride, code,
        steps, a, b, c, _MODE_CODE[mode], ctypes.byref(opt),
        ctypes.c_void_p(wptr), wbytes, _stream_handle(x.device))
    _check(st, "ns_orthogonalize_batched")
    return x


def orthogonalize_grouped(mats: Sequence[torch.Tensor], steps: int = 5,
                          abc=TUNED_ABC, mode: str = "gram",
                          restart_mask: int = 1 << 4, eps: float = 1e-7,
                          internal: Optional[str] = None,
                          status: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None,
                          trace: Optional[Trace] = None, tile: int = 0,
                          guard: float = 0.0) -> Sequence[torch.Tensor]:
    """Orthogonalize 2-D device matrices of one shape up to orientation (for
    example 768 x 3072 and 3072 x 768) in place, each stage launched once
    for all of them; returns ``mats``."""
    if not mats:
        raise ValueError("expects at least one matrix")
    dtype, device = mats[0].dtype, mats[0].device
    shapes = {(min(x.shape), max(x.shape)) for x in mats}
    if len(shapes) != 1:
        raise ValueError("all matrices must have one shape up to orientation")
    n, m = shapes.pop()
    table = (Matrix * len(mats))()
    for i, x in enumerate(mats):
        _check_matrix(x, 2)
        if x.dtype != dtype or x.device != device:
            raise ValueError("all matrices must share dtype and device")
        rows, cols = x.shape
        table[i].data = x.data_ptr()
        table[i].ld = x.stride(0) if rows > 1 else cols
        table[i].transposed = 1 if rows > cols else 0
        table[i].reserved = 0
    code = dtype_code(dtype)
    opt = make_options(restart_mask, eps, internal, status, trace, tile, guard)
    need = int(lib().ns_grouped_workspace_size(n, m, len(mats), code,
                                               _MODE_CODE[mode],
                                               ctypes.byref(opt)))
    if need == 0:
        raise NSError(1, "ns_grouped_workspace_size")
    wptr, wbytes, keep = _workspace(need, device, workspace)
    a, b, c = _coefficients(abc, steps)
    st = lib().ns_orthogonalize_grouped(
        table, len(mats), n, m, code, steps, a, b, c, _MODE_CODE[mode],
        ctypes.byref(opt), ctypes.c_void_p(wptr), wbytes,
        _stream_handle(device))
    _check(st, "ns_orthogonalize_grouped")
    return mats


def grouped_workspace_size(n: int, m: int, count: int,
                           dtype: torch.dtype = torch.bfloat16,
                           mode: str = "gram", restart_mask: int = 1 << 4,
                           internal: Optional[str] = None,
                           tile: int = 0) -> int:
    opt = make_options(restart_mask, 1e-7, internal, tile=tile)
    return int(lib().ns_grouped_workspace_size(n, m, count, dtype_code(dtype),
                                               _MODE_CODE[mode],
                                               ctypes.byref(opt)))


def orthogonalize_static(x: torch.Tensor, steps: int = 5, abc=TUNED_ABC,
                         mode: str = "gram", restart_mask: int = 1 << 4,
                         eps: float = 1e-7, internal: Optional[str] = None,
                         status: Optional[torch.Tensor] = None,
                         tile: int = 0, guard: float = 0.0) -> torch.Tensor:
    """Orthogonalize a [rows, cols] or [E, rows, cols] device tensor in place
    with the library's own device scratch (no allocation at all)."""
    batched = x.dim() == 3
    _check_matrix(x, 3 if batched else 2)
    batch = x.shape[0] if batched else 1
    rows, cols = x.shape[-2], x.shape[-1]
    ld = x.stride(-2) if rows > 1 else cols
    bstride = x.stride(0) if batched and batch > 1 else rows * ld
    opt = make_options(restart_mask, eps, internal, status, None, tile, guard)
    a, b, c = _coefficients(abc, steps)
    st = lib().ns_orthogonalize_static(
        ctypes.c_void_p(x.data_ptr()), batch, rows, cols, ld, bstride,
        dtype_code(x.dtype), steps, a, b, c, _MODE_CODE[mode],
        ctypes.byref(opt), _stream_handle(x.device))
    _check(st, "ns_orthogonalize_static")
    return x


def muon_step(w: torch.Tensor, g: torch.Tensor, m: torch.Tensor, lr: float,
              momentum: float = 0.95, nesterov: bool = True, steps: int = 5,
              abc=TUNED_ABC, mode: str = "gram", restart_mask: int = 1 << 4,
              eps: float = 1e-7, internal: Optional[str] = None,
              status: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None,
              trace: Optional[Trace] = None, tile: int = 0,
              guard: float = 0.0) -> torch.Tensor:
    """One Muon step, in place: M <- mu M + G; W <- W - lr NS(G + mu M).

    ``w`` and ``g``: [rows, cols] or [E, rows, cols] device tensors of the
    same dtype and strides (rows contiguous); ``m``: fp32 momentum with the
    same shape and strides.  ``nesterov=False`` orthogonalizes M itself.
    Returns ``w``.
    """
    if w.shape != g.shape or w.shape != m.shape:
        raise ValueError("w, g and m must have the same shape")
    if w.dtype != g.dtype or m.dtype != torch.float32:
        raise TypeError("g must have w's dtype and m must be float32")
    if w.stride() != g.stride() or w.stride() != m.stride():
        raise ValueError("w, g and m must have the same strides")
    batched = w.dim() == 3
    _check_matrix(w, 3 if batched else 2)
    if not (g.is_cuda and m.is_cuda):
        raise ValueError("expects device tensors")
    batch = w.shape[0] if batched else 1
    rows, cols = w.shape[-2], w.shape[-1]
    ld = w.stride(-2) if rows > 1 else cols
    bstride = w.stride(0) if batched and batch > 1 else rows * ld
    code = dtype_code(w.dtype)
    opt = make_options(restart_mask, eps, internal, status, trace, tile, guard)
    need = int(lib().ns_muon_workspace_size(rows, cols, batch, code,
                                            _MODE_CODE[mode],
                                            ctypes.byref(opt)))
    if need == 0:
        raise NSError(1, "ns_muon_workspace_size")
    wptr, wbytes, keep = _workspace(need, w.device, workspace)
    a, b, c = _coefficients(abc, steps)
    st = lib().ns_muon_step(
        ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(g.data_ptr()),
        ctypes.c_void_p(m.data_ptr()), batch, rows, cols, ld, bstride, code,
        float(lr), float(momentum), 1 if nesterov else 0, steps, a, b, c,
        _MODE_CODE[mode], ctypes.byref(opt), ctypes.c_void_p(wptr), wbytes,
        _stream_handle(w.device))
    _check(st, "ns_muon_step")
    return w


def muon_workspace_size(rows: int, cols: int, batch: int = 1,
                        dtype: torch.dtype = torch.bfloat16,
                        mode: str = "gram", restart_mask: int = 1 << 4,
                        internal: Optional[str] = None, tile: int = 0) -> int:
    opt = make_options(restart_mask, 1e-7, internal, tile=tile)
    return int(lib().ns_muon_workspace_size(rows, cols, batch,
                                            dtype_code(dtype),
                                            _MODE_CODE[mode],
                                            ctypes.byref(opt)))


def soft_threshold_split(m: torch.Tensor, lam: Optional[float] = None,
                         mult: float = 3.0, outliers: bool = True,
                         out_b: Optional[torch.Tensor] = None,
                         lambda_out: Optional[torch.Tensor] = None,
                         status: Optional[torch.Tensor] = None):
    """ROOT split of a contiguous device tensor: returns (B, O or None).

    ``lambda_out`` (device fp32, one element) receives the threshold;
    ``status`` (device int32) is the status word.  ``out_b`` (optional)
    receives B: a contiguous tensor with m's dtype, device and number of
    elements (it may be m itself).
    """
    if not m.is_cuda or not m.is_contiguous():
        raise ValueError("expects a contiguous device tensor")
    code = dtype_code(m.dtype)
    numel = m.numel()
    if out_b is not None:
        if out_b.dtype != m.dtype or out_b.device != m.device:
            raise ValueError("out_b must have m's dtype and device")
        if out_b.numel() != numel or not out_b.is_contiguous():
            raise ValueError("out_b must be contiguous with m's number of elements")
    b = torch.empty_like(m) if out_b is None else out_b
    o = torch.empty_like(m) if outliers else None
    need = int(lib().ns_soft_threshold_workspace_size(numel, code))
    if need == 0:
        raise NSError(1, "ns_soft_threshold_workspace_size")
    wptr, wbytes, keep = _workspace(need, m.device, None)
    lam_arg = -1.0 if lam is None else float(lam)
    lptr = None
    if lambda_out is not None:
        if lambda_out.dtype != torch.float32 or not lambda_out.is_cuda:
            raise TypeError("lambda_out must be a device fp32 tensor")
        lptr = lambda_out.data_ptr()
    sptr = None
    if status is not None:
        if status.dtype != torch.int32 or not status.is_cuda:
            raise TypeError("status must be a device int32 tensor")
        sptr = status.data_ptr()
    st = lib().ns_soft_threshold_split(
        ctypes.c_void_p(m.data_ptr()), ctypes.c_void_p(b.data_ptr()),
        ctypes.c_void_p(o.data_ptr() if o is not None else None), numel, code,
        lam_arg, float(mult), ctypes.c_void_p(lptr), ctypes.c_void_p(sptr),
        ctypes.c_void_p(wptr), wbytes, _stream_handle(m.device))
    _check(st, "ns_soft_threshold_split")
    return b, o
