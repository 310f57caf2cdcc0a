"""CPU oracle for the delayed-scaling FP8 linear layer (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` import this package.  The GPU library never imports, links or runs
anything here, and nothing here imports the GPU library: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, built with gcc; OpenMP only over
independent outputs, so results do not depend on the thread count).  This
module only marshals numpy arrays into it.  Each wrapper names the passage
of the pages it follows:

* ``fp8_decode`` / ``fp8_encode`` -- the OCP float8_e4m3fn / float8_e5m2 formats
  of "Accelerating PyTorch Training Workloads with FP8 -- Part 2" (finfo table
  and the worked cast table), with saturating round-to-nearest-even.
* ``cast_transpose_amax`` -- the scaled cast with its cached transpose and
  scale-inverse snapshot ("[PyTorch] Refactor FP8 workspaces in linear
  modules": the FP8 tensor keeps a private scale-inverse and a transpose
  cache) and the per-tensor amax ("support delayed scaling of weight in float8
  all-gather": amax buffers packed per tensor).
* ``dbias`` -- the bias gradient (column sums of the output gradient) that the
  training loop of "CPU Overhead of te.Linear FP8 Layers" needs for its biased
  linears (fp32, exact fp64 sum rounded once).
* ``produce_cast`` -- the toy block's elementwise producers (the modulation,
  a product divided by a quotient of the modulation linear's outputs, with
  nothing sanitised; the residual add; and the residual add of two terms, each
  sum rounded) rounded to bf16 and followed by the cast ("CPU Overhead of
  te.Linear FP8 Layers", TEBlock.forward).
* ``dynamic_cast`` -- dynamic scaling, the comparator the float8 all-gather
  page contrasts delayed scaling with (amax of the tensor itself, then the
  cast with fp8_max / amax).
* ``scale_update`` -- the DelayedScaling recipe (history length 16, algorithm
  "max") of "CPU Overhead of te.Linear FP8 Layers".
* ``gemm_nt`` / ``gemm_nt_sampled`` -- the per-tensor-scaled FP8 product with
  bias of the ``torch._scaled_mm`` example (Part 2 blog).
* ``gemm_nt_fp8out`` -- the same product with an FP8 output and its amax (the
  ``torch._scaled_mm`` example's FP8 out_dtype, which also returns the
  output amax): the fp32 product followed by the cast.

Parity pins for every function are in ``tests/test_oracle_*.py``; there is no
function here without one.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

E4M3 = 0
E5M2 = 1
SRC_BF16 = 0
SRC_FP32 = 1
OUT_BF16 = 0
OUT_FP32 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math"]

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no HIP, no GPU)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm", "-lgomp"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        c = ctypes
        vp, i64, f32p = c.c_void_p, c.c_int64, c.POINTER(c.c_float)
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = c.c_int
        L.orc_fp8_max.argtypes = [c.c_int]
        L.orc_fp8_max.restype = c.c_double
        L.orc_fp8_decode.argtypes = [c.c_uint8, c.c_int]
        L.orc_fp8_decode.restype = c.c_double
        L.orc_fp8_encode.argtypes = [c.c_float, c.c_int]
        L.orc_fp8_encode.restype = c.c_uint8
        L.orc_bf16_to_f32.argtypes = [c.c_uint16]
        L.orc_bf16_to_f32.restype = c.c_float
        L.orc_f64_to_bf16.argtypes = [c.c_double]
        L.orc_f64_to_bf16.restype = c.c_uint16
        L.orc_cast_transpose_amax.argtypes = [vp, c.c_int, i64, i64, i64, c.c_float, c.c_int,
                                              vp, vp, f32p, f32p]
        L.orc_cast_transpose_amax.restype = c.c_int
        L.orc_produce_cast.argtypes = [c.c_int, vp, i64, vp, i64, vp, i64, i64, i64, c.c_float,
                                       c.c_int, vp, vp, vp, f32p, f32p]
        L.orc_produce_cast.restype = c.c_int
        L.orc_modulate_backward.argtypes = [c.c_int, vp, i64, vp, i64, vp, i64, vp, i64, i64,
                                            i64, vp, i64, vp, i64, vp, i64]
        L.orc_modulate_backward.restype = c.c_int
        L.orc_dynamic_cast.argtypes = [vp, c.c_int, i64, i64, i64, c.c_int, c.c_int, f32p, vp, vp,
                                       f32p, f32p]
        L.orc_dynamic_cast.restype = c.c_int
        L.orc_dbias.argtypes = [vp, c.c_int, i64, i64, i64, f32p]
        L.orc_dbias.restype = c.c_int
        L.orc_scale_update.argtypes = [vp, vp, vp, vp, vp, c.c_int, c.c_int, c.c_int, c.c_int]
        L.orc_scale_update.restype = c.c_int
        L.orc_gemm_nt.argtypes = [vp, c.c_int, i64, vp, c.c_int, i64, i64, i64, i64,
                                  c.c_float, c.c_float, vp, c.c_int, vp, i64]
        L.orc_gemm_nt.restype = c.c_int
        L.orc_gemm_nt_sampled.argtypes = [vp, c.c_int, i64, vp, c.c_int, i64, i64, c.c_float,
                                          c.c_float, vp, c.c_int, vp, vp, i64, vp]
        L.orc_gemm_nt_sampled.restype = c.c_int
        L.orc_gemm_nt_fp8out.argtypes = [vp, c.c_int, i64, vp, c.c_int, i64, i64, i64, i64,
                                         c.c_float, c.c_float, vp, c.c_float, c.c_int, vp, i64,
                                         vp, f32p, f32p]
        L.orc_gemm_nt_fp8out.restype = c.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """Threads the oracle's parallel loops use."""
    return lib().orc_num_threads()


# ---------------------------------------------------------------- codec ----

def fp8_max(fmt: int) -> float:
    return lib().orc_fp8_max(fmt)


def fp8_decode(codes, fmt: int) -> np.ndarray:
    """Decode FP8 codes (any uint8 array) to float64 values."""
    codes = np.asarray(codes, dtype=np.uint8)
    L = lib()
    out = np.empty(codes.shape, dtype=np.float64)
    flat, of = codes.reshape(-1), out.reshape(-1)
    for i in range(flat.size):
        of[i] = L.orc_fp8_decode(int(flat[i]), fmt)
    return out


def decode_table(fmt: int) -> np.ndarray:
    """The value of each of the 256 codes, index = code."""
    return fp8_decode(np.arange(256, dtype=np.uint8), fmt)


def fp8_encode(values, fmt: int) -> np.ndarray:
    """Saturating RNE of fp32 values to FP8 codes (scale 1, fp32 source)."""
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float32).reshape(-1))
    q = np.empty(v.size, dtype=np.uint8)
    if v.size:
        rc = lib().orc_cast_transpose_amax(_ptr(v), SRC_FP32, 1, v.size, v.size,
                                           ctypes.c_float(1.0), fmt, _ptr(q), None, None, None)
        assert rc == 0
    return q.reshape(np.shape(values))


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f64_to_bf16_bits(values) -> np.ndarray:
    v = np.asarray(values, dtype=np.float64)
    L = lib()
    out = np.empty(v.shape, dtype=np.uint16)
    flat, of = v.reshape(-1), out.reshape(-1)
    for i in range(flat.size):
        of[i] = L.orc_f64_to_bf16(float(flat[i]))
    return out


# ----------------------------------------------------------------- cast ----

def cast_transpose_amax(x: np.ndarray, scale: float, fmt: int, *, want_q: bool = True,
                        want_qt: bool = True, amax_in: float = 0.0):
    """Scaled saturating cast of a 2-D source (uint16 = bf16 bits, or float32).

    Returns (q [R,C] uint8 or None, qt [C,R] uint8 or None, amax float32,
    scale_inv float32).  ``amax`` is max(amax_in, max|x|) in sign-cleared bit
    order.
    """
    if x.dtype == np.uint16:
        src = SRC_BF16
    elif x.dtype == np.float32:
        src = SRC_FP32
    else:
        raise TypeError("source must be bf16 bits (uint16) or float32")
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    q = np.empty((rows, cols), dtype=np.uint8) if want_q else None
    qt = np.empty((cols, rows), dtype=np.uint8) if want_qt else None
    amax = ctypes.c_float(amax_in)
    sinv = ctypes.c_float(0.0)
    rc = lib().orc_cast_transpose_amax(_ptr(x), src, rows, cols, cols, ctypes.c_float(scale),
                                       fmt, _ptr(q), _ptr(qt), ctypes.byref(amax),
                                       ctypes.byref(sinv))
    if rc != 0:
        raise ValueError("oracle cast rejected its arguments")
    return q, qt, np.float32(amax.value), np.float32(sinv.value)


PROD_MODULATE = 1
PROD_ADD = 2
PROD_ADD2 = 3
PROD_MODULATE_FINITE = 4


def produce_cast(op: int, x: np.ndarray, a: np.ndarray, b: np.ndarray | None, scale: float,
                 fmt: int, *, want_q: bool = True, want_qt: bool = True):
    """y = op(x, a, b) in bf16, then the cast of y.  x, a, b: 2-D uint16 (bf16
    bits) arrays of one shape, any row stride (views are fine).  Returns
    (y [R,C] uint16, q or None, qt or None, amax float32, scale_inv float32)."""
    for t in (x, a) + ((b,) if b is not None else ()):
        if t.dtype != np.uint16 or t.ndim != 2 or t.strides[1] != 2:
            raise TypeError("inputs must be 2-D bf16 bit arrays with unit column stride")
    rows, cols = x.shape
    ld = lambda t: t.strides[0] // 2
    y = np.empty((rows, cols), dtype=np.uint16)
    q = np.empty((rows, cols), dtype=np.uint8) if want_q else None
    qt = np.empty((cols, rows), dtype=np.uint8) if want_qt else None
    amax = ctypes.c_float(0.0)
    sinv = ctypes.c_float(0.0)
    vp = lambda t: None if t is None else ctypes.c_void_p(t.ctypes.data)
    rc = lib().orc_produce_cast(op, vp(x), ld(x), vp(a), ld(a), vp(b), ld(b) if b is not None else 0,
                                rows, cols, ctypes.c_float(scale), fmt, _ptr(y), _ptr(q), _ptr(qt),
                                ctypes.byref(amax), ctypes.byref(sinv))
    if rc != 0:
        raise ValueError("oracle produce_cast rejected its arguments")
    return y, q, qt, np.float32(amax.value), np.float32(sinv.value)


def modulate_backward(op: int, dy: np.ndarray, x: np.ndarray, a: np.ndarray, b: np.ndarray):
    """Gradient of the modulation y = bf16(a * x / b) (op PROD_MODULATE or
    PROD_MODULATE_FINITE) for the output gradient dy, with respect to x, a
    and b.  All inputs: 2-D uint16 (bf16 bits) arrays of one shape, any row
    stride.  Returns (dx, da, db), uint16 [R, C]."""
    for t in (dy, x, a, b):
        if t.dtype != np.uint16 or t.ndim != 2 or t.strides[1] != 2 or t.shape != dy.shape:
            raise TypeError("inputs must be 2-D bf16 bit arrays of one shape, unit column stride")
    rows, cols = dy.shape
    ld = lambda t: t.strides[0] // 2
    outs = [np.empty((rows, cols), dtype=np.uint16) for _ in range(3)]
    vp = lambda t: ctypes.c_void_p(t.ctypes.data)
    rc = lib().orc_modulate_backward(op, vp(dy), ld(dy), vp(x), ld(x), vp(a), ld(a), vp(b), ld(b),
                                     rows, cols, _ptr(outs[0]), cols, _ptr(outs[1]), cols,
                                     _ptr(outs[2]), cols)
    if rc != 0:
        raise ValueError("oracle modulate_backward rejected its arguments")
    return tuple(outs)


def dynamic_cast(x: np.ndarray, fmt: int, *, margin: int = 0, fallback_scale: float = 1.0,
                 want_q: bool = True, want_qt: bool = True):
    """Dynamic scaling of a 2-D source (uint16 = bf16 bits, or float32):
    returns (q or None, qt or None, amax, scale, scale_inv), float32 scalars."""
    if x.dtype == np.uint16:
        src = SRC_BF16
    elif x.dtype == np.float32:
        src = SRC_FP32
    else:
        raise TypeError("source must be bf16 bits (uint16) or float32")
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    q = np.empty((rows, cols), dtype=np.uint8) if want_q else None
    qt = np.empty((cols, rows), dtype=np.uint8) if want_qt else None
    scale = ctypes.c_float(fallback_scale)
    amax = ctypes.c_float(0.0)
    sinv = ctypes.c_float(0.0)
    rc = lib().orc_dynamic_cast(_ptr(x), src, rows, cols, cols, margin, fmt, ctypes.byref(scale),
                                _ptr(q), _ptr(qt), ctypes.byref(amax), ctypes.byref(sinv))
    if rc != 0:
        raise ValueError("oracle dynamic_cast rejected its arguments")
    return q, qt, np.float32(amax.value), np.float32(scale.value), np.float32(sinv.value)


def dbias(x: np.ndarray) -> np.ndarray:
    """Column sums [C] (float32) of a 2-D source (uint16 = bf16 bits, or
    float32): the bias gradient, exact in fp64, rounded once."""
    if x.dtype == np.uint16:
        src = SRC_BF16
    elif x.dtype == np.float32:
        src = SRC_FP32
    else:
        raise TypeError("source must be bf16 bits (uint16) or float32")
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    out = np.empty(cols, dtype=np.float32)
    rc = lib().orc_dbias(_ptr(x), src, rows, cols, cols,
                         out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    if rc != 0:
        raise ValueError("oracle dbias rejected its arguments")
    return out


# --------------------------------------------------------- scale update ----

def scale_update(hist: np.ndarray, amax_cur: np.ndarray, scale: np.ndarray,
                 scale_inv: np.ndarray, fmt: np.ndarray, margin: int = 0, algo: int = 0) -> None:
    """In-place delayed-scaling update of T records (see oracle.c)."""
    T, H = hist.shape
    for a, dt in ((hist, np.float32), (amax_cur, np.float32), (scale, np.float32),
                  (scale_inv, np.float32), (fmt, np.uint8)):
        assert a.dtype == dt and a.flags["C_CONTIGUOUS"]
    assert amax_cur.shape == scale.shape == scale_inv.shape == fmt.shape == (T,)
    rc = lib().orc_scale_update(_ptr(hist), _ptr(amax_cur), _ptr(scale), _ptr(scale_inv),
                                _ptr(fmt), T, H, margin, algo)
    if rc != 0:
        raise ValueError("oracle scale update rejected its arguments")


# ----------------------------------------------------------------- GEMM ----

def gemm_nt(A: np.ndarray, fa: int, B: np.ndarray, fb: int, sinv_a: float, sinv_b: float,
            bias: np.ndarray | None = None, out_kind: int = OUT_BF16) -> np.ndarray:
    """out = round(dec(A) @ dec(B).T * sinv_a * sinv_b + bias); A [M,K], B [N,K] uint8.

    Returns uint16 bf16 bits (OUT_BF16) or float32 (OUT_FP32), shape [M, N].
    """
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.uint16)
        assert bias.shape == (N,)
    out = np.empty((M, N), dtype=np.uint16 if out_kind == OUT_BF16 else np.float32)
    rc = lib().orc_gemm_nt(_ptr(A), fa, K, _ptr(B), fb, K, M, N, K, ctypes.c_float(sinv_a),
                           ctypes.c_float(sinv_b), _ptr(bias), out_kind, _ptr(out), N)
    if rc != 0:
        raise ValueError("oracle GEMM rejected its arguments")
    return out


def gemm_nt_fp8out(A: np.ndarray, fa: int, B: np.ndarray, fb: int, sinv_a: float,
                   sinv_b: float, scale_out: float, fo: int, bias: np.ndarray | None = None,
                   amax_in: float = 0.0):
    """torch._scaled_mm with an FP8 out_dtype: v = fp32(dec(A) @ dec(B).T *
    sinv_a * sinv_b + bias), then the cast of v with scale_out.

    Returns (codes [M, N] uint8, v [M, N] float32, amax float32 = max(amax_in,
    max|v|) over the unscaled v, scale_inv float32 = 1 / scale_out).
    """
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.uint16)
        assert bias.shape == (N,)
    codes = np.empty((M, N), dtype=np.uint8)
    v = np.empty((M, N), dtype=np.float32)
    amax = ctypes.c_float(amax_in)
    sinv = ctypes.c_float(0.0)
    rc = lib().orc_gemm_nt_fp8out(_ptr(A), fa, K, _ptr(B), fb, K, M, N, K,
                                  ctypes.c_float(sinv_a), ctypes.c_float(sinv_b), _ptr(bias),
                                  ctypes.c_float(scale_out), fo, _ptr(codes), N, _ptr(v),
                                  ctypes.byref(amax), ctypes.byref(sinv))
    if rc != 0:
        raise ValueError("oracle GEMM rejected its arguments")
    return codes, v, np.float32(amax.value), np.float32(sinv.value)


def gemm_nt_sampled(A: np.ndarray, fa: int, B: np.ndarray, fb: int, sinv_a: float,
                    sinv_b: float, rows: np.ndarray, cols: np.ndarray,
                    bias: np.ndarray | None = None, out_kind: int = OUT_BF16) -> np.ndarray:
    """The same definition as gemm_nt, evaluated only at (rows[s], cols[s])."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    K = A.shape[1]
    assert B.shape[1] == K
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    assert rows.shape == cols.shape
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < A.shape[0]
                              and cols.min() >= 0 and cols.max() < B.shape[0])
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.uint16)
    out = np.empty(rows.size, dtype=np.uint16 if out_kind == OUT_BF16 else np.float32)
    rc = lib().orc_gemm_nt_sampled(_ptr(A), fa, K, _ptr(B), fb, K, K, ctypes.c_float(sinv_a),
                                   ctypes.c_float(sinv_b), _ptr(bias), out_kind, _ptr(rows),
                                   _ptr(cols), rows.size, _ptr(out))
    if rc != 0:
        raise ValueError("oracle GEMM rejected its arguments")
    return out
