"""Delayed-scaling FP8 linear layer for AMD MI355X (gfx950): Python binding.

Thin ctypes binding over ``libfp8dsl.so``, whose C ABI is declared in
``include/fp8dsl.h``.  The functions here have the same names as the C entry
points and only marshal arguments: they take torch tensors for device memory,
pass ``data_ptr()`` and the current HIP stream, and turn status codes into
exceptions.  Every step of the computation runs in the HIP kernels.  There is
no CPU fallback: importing this package fails loudly when the library has not
been built.

The pieces, with the pages that define them:

* :class:`Float8Tensor` -- FP8 codes + cached transpose + scale-inverse
  snapshot ("[PyTorch] Refactor FP8 workspaces in linear modules").
* :class:`DelayedScalingState` -- packed amax histories, current amaxes,
  scales and scale-inverses of T tensors (the fp8_meta of te.Linear and the
  packed amax tensor of "support delayed scaling of weight in float8
  all-gather"), with the DelayedScaling recipe of "CPU Overhead of te.Linear
  FP8 Layers" (history 16, "max").
* ``fp8_cast_transpose_amax``, ``fp8_scale_update``, ``fp8_linear_fwd``,
  ``fp8_linear_dgrad``, ``fp8_linear_wgrad`` -- the C entry points.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "E4M3", "E5M2", "DTYPE_BF16", "DTYPE_FP32", "Fp8Error", "Float8Tensor",
    "DelayedScalingState", "fp8_scale_update", "fp8_cast_transpose_amax", "fp8_linear_fwd",
    "fp8_linear_dgrad", "fp8_linear_wgrad", "fp8_status_string", "fp8_abi_version",
    "fp8_cast_transpose_amax_dbias", "fp8_cast_dbias_workspace_bytes",
    "fp8_produce_cast_transpose_amax", "PRODUCE_MODULATE", "PRODUCE_ADD", "PRODUCE_ADD2",
    "PRODUCE_MODULATE_FINITE",
    "fp8_cast_transpose_dynamic", "fp8_linear_fwd_fp8out",
    "fp8_cast_transpose_amax_dbias_noalloc", "NOALLOC_SCRATCH_BYTES",
    "fp8_cast_transpose_amax_cached", "fp8_reference_copy", "fp8_produce_modulate_backward",
    "fp8_gemm_workspace_bytes", "fp8_cast_transpose_amax_group", "CAST_GROUP_MAX",
    "library_path", "lib",
]

E4M3 = 0
E5M2 = 1
DTYPE_BF16 = 0
DTYPE_FP32 = 1
PRODUCE_MODULATE = 1
PRODUCE_ADD = 2
PRODUCE_ADD2 = 3
PRODUCE_MODULATE_FINITE = 4      # the library's addition: non-finite quotients -> +0
NOALLOC_SCRATCH_BYTES = 4 << 20     # FP8DSL_NOALLOC_SCRATCH_BYTES
CAST_GROUP_MAX = 8                  # FP8DSL_CAST_GROUP_MAX

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libfp8dsl.so")


class Fp8Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {fp8_status_string(status)} ({status})")
        self.status = status


class _Desc(ctypes.Structure):
    """Mirror of fp8_tensor_t."""
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("data_t", ctypes.c_void_p),
        ("scale_inv", ctypes.c_void_p),
        ("fmt", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
    ]


class _GroupItem(ctypes.Structure):
    """Mirror of fp8_cast_group_item_t."""
    _fields_ = [
        ("x", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("ld", ctypes.c_int64),
        ("scale", ctypes.c_void_p),
        ("out", ctypes.POINTER(_Desc)),
        ("amax_cur", ctypes.c_void_p),
    ]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libfp8dsl.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(
                f"{library_path} is missing: build it with "
                "`python -m delayed_scaling_linear_amd.build` (there is no CPU fallback)")
        L = ctypes.CDLL(library_path)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        dp = ctypes.POINTER(_Desc)
        L.fp8_scale_update.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]
        L.fp8_cast_transpose_amax.argtypes = [vp, i32, i64, i64, i64, vp, dp, vp, vp, vp]
        L.fp8_cast_transpose_amax_dbias.argtypes = [vp, i32, i64, i64, i64, vp, dp, vp, vp, vp,
                                                    i64, vp, vp]
        L.fp8_cast_transpose_amax_cached.argtypes = [vp, i32, i64, i64, i64, vp, dp, vp, vp, vp]
        L.fp8_reference_copy.argtypes = [vp, vp, i64, i32, i32, vp]
        L.fp8_cast_transpose_amax_dbias_noalloc.argtypes = [vp, i32, i64, i64, i64, vp, dp, vp,
                                                            vp, vp, vp]
        L.fp8_produce_cast_transpose_amax.argtypes = [i32, vp, i64, vp, i64, vp, i64, vp, i64,
                                                      i64, vp, dp, vp, vp, vp]
        L.fp8_produce_modulate_backward.argtypes = [i32, vp, i64, vp, i64, vp, i64, vp, i64, vp,
                                                    i64, vp, i64, vp, i64, i64, i64, vp]
        L.fp8_cast_transpose_dynamic.argtypes = [vp, i32, i64, i64, i64, i32, vp, dp, vp, vp, vp]
        L.fp8_cast_dbias_workspace_bytes.argtypes = [i64, i64]
        L.fp8_cast_dbias_workspace_bytes.restype = i64
        L.fp8_linear_fwd.argtypes = [dp, dp, vp, vp, vp]
        L.fp8_linear_fwd_fp8out.argtypes = [dp, dp, vp, vp, dp, vp, vp]
        L.fp8_linear_dgrad.argtypes = [dp, dp, vp, vp]
        L.fp8_linear_wgrad.argtypes = [dp, dp, vp, i32, vp]
        L.fp8_cast_transpose_amax_group.argtypes = [i32, ctypes.POINTER(_GroupItem), i32, vp, vp]
        L.fp8_cast_transpose_amax_group.restype = ctypes.c_int
        L.fp8_gemm_workspace_bytes.argtypes = [i64, i64, i64]
        L.fp8_gemm_workspace_bytes.restype = i64
        L.fp8_linear_fwd_ws.argtypes = [dp, dp, vp, vp, vp, i64, vp]
        L.fp8_linear_dgrad_ws.argtypes = [dp, dp, vp, vp, i64, vp]
        L.fp8_linear_wgrad_ws.argtypes = [dp, dp, vp, i32, vp, i64, vp]
        for f in (L.fp8_scale_update, L.fp8_cast_transpose_amax, L.fp8_cast_transpose_amax_dbias,
                  L.fp8_cast_transpose_amax_dbias_noalloc, L.fp8_cast_transpose_amax_cached,
                  L.fp8_reference_copy,
                  L.fp8_produce_cast_transpose_amax, L.fp8_cast_transpose_dynamic,
                  L.fp8_linear_fwd, L.fp8_linear_fwd_fp8out, L.fp8_linear_dgrad,
                  L.fp8_linear_wgrad, L.fp8_linear_fwd_ws, L.fp8_linear_dgrad_ws,
                  L.fp8_linear_wgrad_ws):
            f.restype = ctypes.c_int
        L.fp8_status_string.argtypes = [ctypes.c_int]
        L.fp8_status_string.restype = ctypes.c_char_p
        L.fp8_abi_version.argtypes = []
        L.fp8_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def fp8_status_string(status: int) -> str:
    return lib().fp8_status_string(status).decode()


def fp8_abi_version() -> int:
    return lib().fp8_abi_version()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise Fp8Error(status, what)


def _ptr(t: Optional[torch.Tensor], dtype=None, what: str = "tensor") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def _need_shape(t: Optional[torch.Tensor], shape, what: str) -> None:
    """The C ABI trusts the sizes it is given: a tensor smaller than the call
    assumes would be read or written out of bounds on the device, so every
    extent is checked here before the call."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _need_scalar(t: Optional[torch.Tensor], what: str) -> None:
    if t is not None and t.numel() < 1:
        raise ValueError(f"{what} must have at least one element")


def _row_stride(t: torch.Tensor) -> int:
    """Row stride (elements) of a 2-D source.  torch gives an empty tensor an
    arbitrary stride; no memory is read for it, so its column count is
    passed instead."""
    return t.stride(0) if t.numel() > 0 else t.shape[1]


# torch's raw getter of the current stream handle (the public
# torch.cuda.current_stream() builds a Stream object on every call, which
# costs more host time than the library call itself); the public call is the
# fallback where the raw one does not exist.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_raw_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream(stream) -> int:
    if stream is None:
        if _raw_stream is not None and _raw_device is not None:
            return _raw_stream(_raw_device())
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


@dataclass
class Float8Tensor:
    """FP8 codes [rows, cols] (optional), their transpose [cols, rows]
    (optional) and the scale-inverse [1] in force when they were written."""
    data: Optional[torch.Tensor]
    data_t: Optional[torch.Tensor]
    scale_inv: torch.Tensor
    fmt: int
    rows: int
    cols: int

    @staticmethod
    def empty(rows: int, cols: int, fmt: int, *, data: bool = True, transpose: bool = True,
              device="cuda") -> "Float8Tensor":
        d = torch.empty((rows, cols), dtype=torch.uint8, device=device) if data else None
        dt = torch.empty((cols, rows), dtype=torch.uint8, device=device) if transpose else None
        si = torch.ones(1, dtype=torch.float32, device=device)
        return Float8Tensor(d, dt, si, fmt, rows, cols)

    def desc(self) -> _Desc:
        if self.rows < 0 or self.cols < 0:
            raise ValueError("Float8Tensor: negative size")
        _need_shape(self.data, (self.rows, self.cols), "Float8Tensor.data")
        _need_shape(self.data_t, (self.cols, self.rows), "Float8Tensor.data_t")
        if self.scale_inv is None:
            raise ValueError("Float8Tensor.scale_inv is required")
        _need_scalar(self.scale_inv, "Float8Tensor.scale_inv")
        return _Desc(_ptr(self.data, torch.uint8, "data"), _ptr(self.data_t, torch.uint8, "data_t"),
                     _ptr(self.scale_inv, torch.float32, "scale_inv"), self.fmt, 0, self.rows,
                     self.cols)


class DelayedScalingState:
    """Packed delayed-scaling state of T tensors (device memory, caller-owned).

    amax_history [T, H], amax_cur [T], scale [T], scale_inv [T] (fp32) and
    fmt [T] (uint8).  Initial state: empty history, amax 0, scale 1.
    """

    def __init__(self, fmts, history_len: int = 16, margin: int = 0, device="cuda"):
        T = len(fmts)
        self.T, self.H, self.margin = T, history_len, margin
        self.amax_history = torch.zeros((T, history_len), dtype=torch.float32, device=device)
        self.amax_cur = torch.zeros(T, dtype=torch.float32, device=device)
        self.scale = torch.ones(T, dtype=torch.float32, device=device)
        self.scale_inv = torch.ones(T, dtype=torch.float32, device=device)
        self.fmt = torch.tensor(list(fmts), dtype=torch.uint8, device=device)

    def update(self, stream=None) -> None:
        fp8_scale_update(self.amax_history, self.amax_cur, self.scale, self.scale_inv, self.fmt,
                         margin=self.margin, stream=stream)


def fp8_scale_update(amax_history: torch.Tensor, amax_cur: torch.Tensor, scale: torch.Tensor,
                     scale_inv: torch.Tensor, fmt: torch.Tensor, margin: int = 0, algo: int = 0,
                     stream=None) -> None:
    if amax_history.dim() != 2:
        raise ValueError("amax_history must be [T, H]")
    T, H = amax_history.shape
    for t, n in ((amax_cur, "amax_cur"), (scale, "scale"), (scale_inv, "scale_inv"), (fmt, "fmt")):
        if t.numel() != T:
            raise ValueError(f"{n} must have {T} entries")
    _check(lib().fp8_scale_update(_ptr(amax_history, torch.float32, "amax_history"),
                                  _ptr(amax_cur, torch.float32, "amax_cur"),
                                  _ptr(scale, torch.float32, "scale"),
                                  _ptr(scale_inv, torch.float32, "scale_inv"),
                                  _ptr(fmt, torch.uint8, "fmt"), T, H, margin, algo,
                                  _stream(stream)), "fp8_scale_update")


def fp8_cast_transpose_amax(x: torch.Tensor, scale: torch.Tensor, out: Float8Tensor,
                            amax_cur: Optional[torch.Tensor] = None,
                            noop_flag: Optional[torch.Tensor] = None, stream=None) -> None:
    """Cast x (bf16 or fp32, 2-D, unit stride in the last dim) into `out`.

    `scale` and `amax_cur` are 1-element fp32 device tensors (views into a
    DelayedScalingState are fine)."""
    _need_scalar(scale, "scale")
    _need_scalar(amax_cur, "amax_cur")
    _need_scalar(noop_flag, "noop_flag")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride in the last dimension")
    if x.dtype == torch.bfloat16:
        src = DTYPE_BF16
    elif x.dtype == torch.float32:
        src = DTYPE_FP32
    else:
        raise TypeError("x must be bf16 or fp32")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    d = out.desc()
    _check(lib().fp8_cast_transpose_amax(x.data_ptr(), src, x.shape[0], x.shape[1], _row_stride(x),
                                         _ptr(scale, torch.float32, "scale"), ctypes.byref(d),
                                         _ptr(amax_cur, torch.float32, "amax_cur"),
                                         _ptr(noop_flag, torch.int32, "noop_flag"),
                                         _stream(stream)), "fp8_cast_transpose_amax")


def fp8_cast_transpose_amax_group(items, noop_flag: Optional[torch.Tensor] = None,
                                  stream=None) -> None:
    """Cast several tensors in one launch, each exactly as
    fp8_cast_transpose_amax(x, scale, out, amax_cur) casts it.  `items` is a
    sequence of (x, scale, out, amax_cur) tuples, 1 to CAST_GROUP_MAX of them,
    with one source dtype (bf16 or fp32), one FP8 format and the same outputs
    (codes, transpose or both) throughout."""
    items = list(items)
    if not 1 <= len(items) <= CAST_GROUP_MAX:
        raise ValueError(f"a group holds 1 to {CAST_GROUP_MAX} tensors")
    _need_scalar(noop_flag, "noop_flag")
    dtypes = {x.dtype for x, _, _, _ in items}
    if len(dtypes) != 1 or not dtypes <= {torch.bfloat16, torch.float32}:
        raise TypeError("every source must be bf16, or every source fp32")
    src = DTYPE_BF16 if dtypes == {torch.bfloat16} else DTYPE_FP32
    arr = (_GroupItem * len(items))()
    descs = []
    for k, (x, scale, out, amax_cur) in enumerate(items):
        _need_scalar(scale, "scale")
        _need_scalar(amax_cur, "amax_cur")
        if x.dim() != 2 or x.stride(1) != 1:
            raise ValueError("x must be 2-D with unit stride in the last dimension")
        if not x.is_cuda:
            raise ValueError("x must be a device tensor")
        d = out.desc()
        descs.append(d)
        arr[k] = _GroupItem(x.data_ptr(), x.shape[0], x.shape[1], _row_stride(x),
                            _ptr(scale, torch.float32, "scale"), ctypes.pointer(d),
                            _ptr(amax_cur, torch.float32, "amax_cur"))
    _check(lib().fp8_cast_transpose_amax_group(src, arr, len(items),
                                               _ptr(noop_flag, torch.int32, "noop_flag"),
                                               _stream(stream)),
           "fp8_cast_transpose_amax_group")


def fp8_cast_transpose_amax_cached(x: torch.Tensor, scale: torch.Tensor, out: Float8Tensor,
                                   amax_cur: Optional[torch.Tensor] = None,
                                   noop_flag: Optional[torch.Tensor] = None, stream=None) -> None:
    """fp8_cast_transpose_amax with the source read through the caches
    (ordinary loads instead of non-temporal ones); identical results."""
    _need_scalar(scale, "scale")
    _need_scalar(amax_cur, "amax_cur")
    _need_scalar(noop_flag, "noop_flag")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride in the last dimension")
    if x.dtype == torch.bfloat16:
        src = DTYPE_BF16
    elif x.dtype == torch.float32:
        src = DTYPE_FP32
    else:
        raise TypeError("x must be bf16 or fp32")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    d = out.desc()
    _check(lib().fp8_cast_transpose_amax_cached(
        x.data_ptr(), src, x.shape[0], x.shape[1], _row_stride(x),
        _ptr(scale, torch.float32, "scale"), ctypes.byref(d),
        _ptr(amax_cur, torch.float32, "amax_cur"), _ptr(noop_flag, torch.int32, "noop_flag"),
        _stream(stream)), "fp8_cast_transpose_amax_cached")


def fp8_reference_copy(src: torch.Tensor, dst: torch.Tensor, workgroups: int,
                       nontemporal: bool = False, stream=None) -> None:
    """Measurement reference: copy src into dst (contiguous device tensors of
    the same byte size, a multiple of 16)."""
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("src and dst must have the same byte size")
    _check(lib().fp8_reference_copy(_ptr(src, None, "src"), _ptr(dst, None, "dst"), nb,
                                    workgroups, int(nontemporal), _stream(stream)),
           "fp8_reference_copy")


def fp8_cast_dbias_workspace_bytes(rows: int, cols: int) -> int:
    """Bytes of device workspace fp8_cast_transpose_amax_dbias needs."""
    n = lib().fp8_cast_dbias_workspace_bytes(rows, cols)
    if n < 0:
        raise Fp8Error(n, "fp8_cast_dbias_workspace_bytes")
    return n


def fp8_cast_transpose_amax_dbias(x: torch.Tensor, scale: torch.Tensor, out: Float8Tensor,
                                  amax_cur: Optional[torch.Tensor], dbias: torch.Tensor,
                                  workspace: torch.Tensor,
                                  noop_flag: Optional[torch.Tensor] = None, stream=None) -> None:
    """fp8_cast_transpose_amax plus dbias [cols] (fp32) = column sums of x.
    `workspace` is a device uint8 tensor of at least
    fp8_cast_dbias_workspace_bytes(rows, cols) bytes."""
    _need_scalar(scale, "scale")
    _need_scalar(amax_cur, "amax_cur")
    _need_scalar(noop_flag, "noop_flag")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride in the last dimension")
    if x.dtype == torch.bfloat16:
        src = DTYPE_BF16
    elif x.dtype == torch.float32:
        src = DTYPE_FP32
    else:
        raise TypeError("x must be bf16 or fp32")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    if dbias.numel() != x.shape[1]:
        raise ValueError("dbias must have cols elements")
    d = out.desc()
    _check(lib().fp8_cast_transpose_amax_dbias(
        x.data_ptr(), src, x.shape[0], x.shape[1], _row_stride(x), _ptr(scale, torch.float32, "scale"),
        ctypes.byref(d), _ptr(amax_cur, torch.float32, "amax_cur"),
        _ptr(dbias, torch.float32, "dbias"), _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel(), _ptr(noop_flag, torch.int32, "noop_flag"), _stream(stream)),
        "fp8_cast_transpose_amax_dbias")


def fp8_cast_transpose_amax_dbias_noalloc(x: torch.Tensor, scale: torch.Tensor, out: Float8Tensor,
                                          amax_cur: Optional[torch.Tensor], dbias: torch.Tensor,
                                          noop_flag: Optional[torch.Tensor] = None,
                                          stream=None) -> None:
    """fp8_cast_transpose_amax_dbias with the library's own per-device
    scratch array instead of a workspace: the call allocates nothing.  Calls
    that overlap on one GPU race on that array; sources needing more than
    NOALLOC_SCRATCH_BYTES of column-sum scratch raise (FP8_ERR_SCRATCH)."""
    _need_scalar(scale, "scale")
    _need_scalar(amax_cur, "amax_cur")
    _need_scalar(noop_flag, "noop_flag")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride in the last dimension")
    if x.dtype == torch.bfloat16:
        src = DTYPE_BF16
    elif x.dtype == torch.float32:
        src = DTYPE_FP32
    else:
        raise TypeError("x must be bf16 or fp32")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    if dbias.numel() != x.shape[1]:
        raise ValueError("dbias must have cols elements")
    d = out.desc()
    _check(lib().fp8_cast_transpose_amax_dbias_noalloc(
        x.data_ptr(), src, x.shape[0], x.shape[1], _row_stride(x),
        _ptr(scale, torch.float32, "scale"), ctypes.byref(d),
        _ptr(amax_cur, torch.float32, "amax_cur"), _ptr(dbias, torch.float32, "dbias"),
        _ptr(noop_flag, torch.int32, "noop_flag"), _stream(stream)),
        "fp8_cast_transpose_amax_dbias_noalloc")


def fp8_produce_cast_transpose_amax(op: int, x: torch.Tensor, a: torch.Tensor,
                                    b: Optional[torch.Tensor], y: torch.Tensor,
                                    scale: torch.Tensor, out: Float8Tensor,
                                    amax_cur: Optional[torch.Tensor] = None,
                                    noop_flag: Optional[torch.Tensor] = None, stream=None) -> None:
    """y = op(x, a, b) in bf16 (PRODUCE_MODULATE: a * x / b, unsanitised, so a
    zero divisor gives +-inf and 0/0 NaN; PRODUCE_MODULATE_FINITE, the
    library's addition: the same with non-finite results replaced by +0;
    PRODUCE_ADD: x + a; PRODUCE_ADD2: (x + a) + b, each sum rounded), then y
    cast into `out`.  x, a, b: bf16 2-D device
    tensors of one shape with unit column stride (column slices are fine);
    y: contiguous bf16 of that shape."""
    _need_scalar(scale, "scale")
    _need_scalar(amax_cur, "amax_cur")
    _need_scalar(noop_flag, "noop_flag")
    ins = [x, a] + ([b] if b is not None else [])
    for t in ins + [y]:
        if t.dtype != torch.bfloat16 or t.dim() != 2 or t.stride(1) != 1 or not t.is_cuda:
            raise ValueError("x, a, b, y must be 2-D bf16 device tensors with unit column stride")
        if t.shape != x.shape:
            raise ValueError("x, a, b, y must have one shape")
    if not y.is_contiguous():
        raise ValueError("y must be contiguous")
    d = out.desc()
    _check(lib().fp8_produce_cast_transpose_amax(
        op, x.data_ptr(), _row_stride(x), a.data_ptr(), _row_stride(a),
        None if b is None else b.data_ptr(), 0 if b is None else _row_stride(b), y.data_ptr(),
        x.shape[0], x.shape[1], _ptr(scale, torch.float32, "scale"), ctypes.byref(d),
        _ptr(amax_cur, torch.float32, "amax_cur"), _ptr(noop_flag, torch.int32, "noop_flag"),
        _stream(stream)), "fp8_produce_cast_transpose_amax")


def fp8_produce_modulate_backward(op: int, dy: torch.Tensor, x: torch.Tensor, a: torch.Tensor,
                                  b: torch.Tensor, dx: torch.Tensor, da: torch.Tensor,
                                  db: torch.Tensor, stream=None) -> None:
    """Gradient of the modulation y = a * x / b (op PRODUCE_MODULATE or
    PRODUCE_MODULATE_FINITE) for the output gradient dy: writes dx, da and db.
    All seven: 2-D bf16 device tensors of one shape with unit column stride
    (column slices of wider tensors are fine); the outputs must not overlap
    each other or the inputs."""
    for t in (dy, x, a, b, dx, da, db):
        if t.dtype != torch.bfloat16 or t.dim() != 2 or t.stride(1) != 1 or not t.is_cuda:
            raise ValueError("dy, x, a, b, dx, da, db must be 2-D bf16 device tensors with unit "
                             "column stride")
        if t.shape != dy.shape:
            raise ValueError("dy, x, a, b, dx, da, db must have one shape")
    _check(lib().fp8_produce_modulate_backward(
        op, dy.data_ptr(), _row_stride(dy), x.data_ptr(), _row_stride(x), a.data_ptr(),
        _row_stride(a), b.data_ptr(), _row_stride(b), dx.data_ptr(), _row_stride(dx),
        da.data_ptr(), _row_stride(da), db.data_ptr(), _row_stride(db), dy.shape[0],
        dy.shape[1], _stream(stream)), "fp8_produce_modulate_backward")


def fp8_cast_transpose_dynamic(x: torch.Tensor, scale: torch.Tensor, out: Float8Tensor,
                               amax: torch.Tensor, margin: int = 0,
                               noop_flag: Optional[torch.Tensor] = None, stream=None) -> None:
    """Dynamic scaling: amax of x, scale = fp8_max / (amax * 2^margin) (scale
    keeps its value for a zero or non-finite amax), then the cast into `out`.
    `scale` (in/out) and `amax` (out) are 1-element fp32 device tensors."""
    _need_scalar(scale, "scale")
    if amax is None:
        raise ValueError("amax is required")
    _need_scalar(amax, "amax")
    _need_scalar(noop_flag, "noop_flag")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride in the last dimension")
    if x.dtype == torch.bfloat16:
        src = DTYPE_BF16
    elif x.dtype == torch.float32:
        src = DTYPE_FP32
    else:
        raise TypeError("x must be bf16 or fp32")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    d = out.desc()
    _check(lib().fp8_cast_transpose_dynamic(
        x.data_ptr(), src, x.shape[0], x.shape[1], _row_stride(x), margin,
        _ptr(scale, torch.float32, "scale"), ctypes.byref(d), _ptr(amax, torch.float32, "amax"),
        _ptr(noop_flag, torch.int32, "noop_flag"), _stream(stream)), "fp8_cast_transpose_dynamic")


def fp8_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace bytes of the split form of a product with output [M, N] and
    contraction K on the current device (0: it runs unsplit); the
    `workspace` of fp8_linear_fwd / dgrad / wgrad."""
    n = lib().fp8_gemm_workspace_bytes(M, N, K)
    if n < 0:
        raise Fp8Error(n, "fp8_gemm_workspace_bytes")
    return n


def _ws(workspace: Optional[torch.Tensor]):
    """(pointer, bytes) of an optional uint8 device workspace."""
    if workspace is None:
        return None, 0
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 device tensor")
    return _ptr(workspace, torch.uint8, "workspace"), workspace.numel()


def fp8_linear_fwd(x: Float8Tensor, w: Float8Tensor, bias: Optional[torch.Tensor],
                   y: torch.Tensor, stream=None, workspace: Optional[torch.Tensor] = None) -> None:
    """y [M, N] bf16 = x.data [M, K] . w.data [N, K]^T * sinv + bias.  With a
    `workspace` (uint8 device tensor), fp8_linear_fwd_ws: the product split
    over K where it alone would leave compute units idle."""
    _need_shape(y, (x.rows, w.rows), "y")
    _need_shape(bias, (w.rows,), "bias")
    dx, dw = x.desc(), w.desc()
    args = (ctypes.byref(dx), ctypes.byref(dw), _ptr(bias, torch.bfloat16, "bias"),
            _ptr(y, torch.bfloat16, "y"))
    if workspace is None:
        _check(lib().fp8_linear_fwd(*args, _stream(stream)), "fp8_linear_fwd")
    else:
        _check(lib().fp8_linear_fwd_ws(*args, *_ws(workspace), _stream(stream)),
               "fp8_linear_fwd_ws")


def fp8_linear_fwd_fp8out(x: Float8Tensor, w: Float8Tensor, bias: Optional[torch.Tensor],
                          scale_y: torch.Tensor, y: Float8Tensor, amax_y: Optional[torch.Tensor],
                          stream=None) -> None:
    """y.data [M, N] FP8 codes = the cast (scale_y) of v = x.data . w.data^T *
    sinv + bias in fp32; amax_y folds in max|v|; y.scale_inv = 1 / scale_y.
    y must have no transpose buffer."""
    _need_shape(bias, (w.rows,), "bias")
    _need_scalar(scale_y, "scale_y")
    _need_scalar(amax_y, "amax_y")
    dx, dw, dy = x.desc(), w.desc(), y.desc()
    _check(lib().fp8_linear_fwd_fp8out(ctypes.byref(dx), ctypes.byref(dw),
                                       _ptr(bias, torch.bfloat16, "bias"),
                                       _ptr(scale_y, torch.float32, "scale_y"), ctypes.byref(dy),
                                       _ptr(amax_y, torch.float32, "amax_y"), _stream(stream)),
           "fp8_linear_fwd_fp8out")


def fp8_linear_dgrad(dy: Float8Tensor, w: Float8Tensor, dx: torch.Tensor, stream=None,
                     workspace: Optional[torch.Tensor] = None) -> None:
    """dx [M, K] bf16 = dy.data [M, N] . w.data_t [K, N]^T * sinv (with a
    `workspace`: fp8_linear_dgrad_ws)."""
    _need_shape(dx, (dy.rows, w.cols), "dx")
    d1, d2 = dy.desc(), w.desc()
    args = (ctypes.byref(d1), ctypes.byref(d2), _ptr(dx, torch.bfloat16, "dx"))
    if workspace is None:
        _check(lib().fp8_linear_dgrad(*args, _stream(stream)), "fp8_linear_dgrad")
    else:
        _check(lib().fp8_linear_dgrad_ws(*args, *_ws(workspace), _stream(stream)),
               "fp8_linear_dgrad_ws")


def fp8_linear_wgrad(dy: Float8Tensor, x: Float8Tensor, dw: torch.Tensor, stream=None,
                     workspace: Optional[torch.Tensor] = None) -> None:
    """dw [N, K] (fp32 or bf16) = dy.data_t [N, M] . x.data_t [K, M]^T * sinv
    (with a `workspace`: fp8_linear_wgrad_ws)."""
    if dw.dtype == torch.float32:
        od = DTYPE_FP32
    elif dw.dtype == torch.bfloat16:
        od = DTYPE_BF16
    else:
        raise TypeError("dw must be fp32 or bf16")
    _need_shape(dw, (dy.cols, x.cols), "dw")
    d1, d2 = dy.desc(), x.desc()
    args = (ctypes.byref(d1), ctypes.byref(d2), _ptr(dw, None, "dw"), od)
    if workspace is None:
        _check(lib().fp8_linear_wgrad(*args, _stream(stream)), "fp8_linear_wgrad")
    else:
        _check(lib().fp8_linear_wgrad_ws(*args, *_ws(workspace), _stream(stream)),
               "fp8_linear_wgrad_ws")
