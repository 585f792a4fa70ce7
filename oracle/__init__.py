"""The CPU oracle for C = epilogue(A . B) -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (``tensor_core_gemm_amd``)
never imports it, and it imports nothing from the product: the two share no
code, header, table or constant.  Inputs cross over as raw 16-bit patterns
(numpy ``uint16`` arrays), produced by the seeded generators in
``gemm_workloads``.

The arithmetic lives in ``oracle.c`` (plain C, built with gcc and OpenMP,
``-ffp-contract=off``).  It follows the worked example of the page
"gizml:tile": a zero accumulator (Program.zeros), a fold over k in ascending
order (Program.fold), products and sums in F32 (Tile.dot), an optional
bias row added in F32 (Tile.add, broadcast over rows), an activation
(Tile.relu with Tile.maximum's NaN rule, Tile.gelu, Tile.geluErf,
Tile.sigmoid, Tile.tanh; the transcendental ones from their definitions in
double precision, rounded once to F32), then rounding to the storage type
(Tile.to).  Storage codes are the page's constants: F32 = 0, F16 = 4,
BF16 = 5, FP8 = 9 (operands only; E4M3, read as the OCP format).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

F32, F16, BF16, FP8 = 0, 4, 5, 9
EPI_NONE, EPI_RELU, EPI_GELU, EPI_GELU_ERF, EPI_SIGMOID, EPI_TANH = 0, 1, 2, 3, 4, 5

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_i64 = ctypes.c_int64
_int = ctypes.c_int
_vp = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no GPU code involved)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            lib.oracle_decode.argtypes = [_int, _vp, _vp, _i64]
            lib.oracle_decode.restype = None
            lib.oracle_encode.argtypes = [_int, _vp, _vp, _i64]
            lib.oracle_encode.restype = None
            lib.oracle_max_threads.argtypes = []
            lib.oracle_max_threads.restype = _int
            lib.oracle_gemm.argtypes = [_i64, _i64, _i64, _int, _int, _int, _vp, _i64, _vp, _i64,
                                        _vp, _i64, _vp, _i64, _vp, _int]
            lib.oracle_gemm.restype = _int
            lib.oracle_gemm_sampled.argtypes = [_i64, _i64, _i64, _int, _int, _int, _vp, _i64,
                                                _vp, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _vp,
                                                _vp, _int]
            lib.oracle_gemm_sampled.restype = _int
            lib.oracle_gemm_f64.argtypes = [_i64, _i64, _i64, _int, _i64, _vp, _i64, _vp, _i64,
                                            _vp, _vp, _int]
            lib.oracle_gemm_f64.restype = _int
            _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_vp)


def _bits(x, dtype: int | None = None) -> np.ndarray:
    """Raw patterns as a C-contiguous numpy array: uint16 for F16/BF16,
    uint8 for FP8 (dtype None: whatever width x has, 16 or 8 bits)."""
    if hasattr(x, "detach"):  # a torch tensor of a 16- or 8-bit type
        import torch  # local: the oracle itself needs no torch

        t = x.detach().cpu().contiguous()
        if t.dtype in (torch.float16, torch.bfloat16):
            t = t.view(torch.int16)
        elif t.element_size() == 1:
            t = t.view(torch.uint8)
        x = t.numpy()
    a = np.ascontiguousarray(x)
    width = None if dtype is None else (1 if dtype == FP8 else 2)
    if a.dtype.itemsize == 2 and width in (None, 2):
        return a.view(np.uint16)
    if a.dtype.itemsize == 1 and width in (None, 1):
        return a.view(np.uint8)
    raise TypeError("expected 16-bit patterns (F16, BF16) or bytes (FP8)")


def threads() -> int:
    return int(_load().oracle_max_threads())


def decode(dtype: int, bits) -> np.ndarray:
    b = _bits(bits, dtype)
    out = np.empty(b.shape, np.float32)
    _load().oracle_decode(dtype, _ptr(b), _ptr(out), b.size)
    return out


def encode(dtype: int, values) -> np.ndarray:
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_encode(dtype, _ptr(v), _ptr(out), v.size)
    return out


def _bias(bias, N: int):
    """bias -> (keep-alive array or None, pointer or None)."""
    if bias is None:
        return None, None
    if hasattr(bias, "detach"):
        bias = bias.detach().cpu().float().numpy()
    v = np.ascontiguousarray(bias, np.float32).reshape(-1)
    if v.size != N:
        raise ValueError("bias must hold N values")
    return v, _ptr(v)


def _check(rc: int):
    if rc != 0:
        raise ValueError({-1: "bad argument", -2: "bad dtype", -3: "out of memory"}.get(rc, rc))


# What a strided C holds between batch items (16-bit outputs; fp32: its NaN).
C_SENTINEL16 = 0x7e5a
C_SENTINEL32 = 0x7fc05a5a


def gemm(A, B, M: int, N: int, K: int, in_dtype: int, out_dtype: int, epilogue: int,
         batch: int = 1, stride_a: int | None = None, stride_b: int | None = None,
         want_y: bool = False, n_threads: int = 0, bias=None, stride_c: int | None = None):
    """C = act(A . B + bias) for [batch][M][K] x [batch][K][N] row-major operands
    (epilogue: the activation code; bias: N fp32 values or None).

    Returns C as float32 (out F32) or uint16 patterns (F16/BF16), shape
    [batch, M, N], and, if ``want_y``, the fp32 value before rounding too.
    With ``stride_c``, C is instead the flat array of (batch - 1) * stride_c
    + M * N elements that item b fills from b * stride_c, the rest holding
    C_SENTINEL16 / C_SENTINEL32.
    """
    a, b = _bits(A, in_dtype).reshape(-1), _bits(B, in_dtype).reshape(-1)
    sa = M * K if stride_a is None else stride_a
    sb = K * N if stride_b is None else stride_b
    if batch < 1 or a.size < (batch - 1) * sa + M * K or b.size < (batch - 1) * sb + K * N:
        raise ValueError("operand arrays smaller than the shape and strides need")
    if stride_c is not None and stride_c < M * N:
        raise ValueError("stride_c smaller than one item of C")
    kind = np.float32 if out_dtype == F32 else np.uint16
    if stride_c is None:
        C = np.zeros((batch, M, N), kind)
        sc = M * N
    else:
        sc = stride_c
        C = np.full((batch - 1) * sc + M * N, C_SENTINEL32 if kind is np.float32 else C_SENTINEL16,
                    np.uint32 if kind is np.float32 else np.uint16).view(kind)
    Y = np.zeros((batch, M, N), np.float32) if want_y else None
    keep, bp = _bias(bias, N)
    _check(_load().oracle_gemm(M, N, K, in_dtype, out_dtype, epilogue, bp, batch, _ptr(a), sa,
                               _ptr(b), sb, _ptr(C), sc, _ptr(Y) if Y is not None else None,
                               n_threads))
    return (C, Y) if want_y else C


def gemm_sampled(A, B, M: int, N: int, K: int, in_dtype: int, out_dtype: int, epilogue: int,
                 bi, ii, jj, batch: int = 1, stride_a: int | None = None,
                 stride_b: int | None = None, n_threads: int = 0, bias=None):
    """The oracle for the listed elements C[bi[e], ii[e], jj[e]] only.

    Returns (values in out_dtype storage, fp32 y before rounding).
    """
    a, b = _bits(A, in_dtype).reshape(-1), _bits(B, in_dtype).reshape(-1)
    sa = M * K if stride_a is None else stride_a
    sb = K * N if stride_b is None else stride_b
    bi = np.ascontiguousarray(bi, np.int64)
    ii = np.ascontiguousarray(ii, np.int64)
    jj = np.ascontiguousarray(jj, np.int64)
    if not (bi.shape == ii.shape == jj.shape):
        raise ValueError("index arrays differ in shape")
    if a.size < (batch - 1) * sa + M * K or b.size < (batch - 1) * sb + K * N:
        raise ValueError("operand arrays smaller than the shape and strides need")
    out = np.zeros(ii.shape, np.float32 if out_dtype == F32 else np.uint16)
    Y = np.zeros(ii.shape, np.float32)
    keep, bp = _bias(bias, N)
    _check(_load().oracle_gemm_sampled(M, N, K, in_dtype, out_dtype, epilogue, bp, batch, _ptr(a),
                                       sa, _ptr(b), sb, ii.size, _ptr(bi), _ptr(ii), _ptr(jj),
                                       _ptr(out), _ptr(Y), n_threads))
    return out, Y


def gemm_f64(A, B, M: int, N: int, K: int, in_dtype: int, batch: int = 1,
             stride_a: int | None = None, stride_b: int | None = None, n_threads: int = 0):
    """fp64 twin: (sum in double before any epilogue, sum of |a||b|)."""
    a, b = _bits(A, in_dtype).reshape(-1), _bits(B, in_dtype).reshape(-1)
    sa = M * K if stride_a is None else stride_a
    sb = K * N if stride_b is None else stride_b
    if a.size < (batch - 1) * sa + M * K or b.size < (batch - 1) * sb + K * N:
        raise ValueError("operand arrays smaller than the shape and strides need")
    Y = np.zeros((batch, M, N), np.float64)
    S = np.zeros((batch, M, N), np.float64)
    _check(_load().oracle_gemm_f64(M, N, K, in_dtype, batch, _ptr(a), sa, _ptr(b), sb, _ptr(Y),
                                   _ptr(S), n_threads))
    return Y, S


def to_float(dtype: int, C) -> np.ndarray:
    """Output storage -> float32 values (identity for F32)."""
    C = np.asarray(C)
    return C.astype(np.float32) if dtype == F32 else decode(dtype, C)
