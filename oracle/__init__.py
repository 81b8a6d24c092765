"""CPU oracle for the GEMM / fully-connected hot path (float64, plain loops).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the bench's
CPU-baseline leg are the only callers. The product path never imports this
module, and this module imports nothing from the product package.

The arithmetic lives in ``oracle.c`` (built with gcc and OpenMP, no fast-math);
this file only builds it, loads it and marshals numpy arrays into it. Each
routine returns ``(R, T)``: ``R`` the float64 result, ``T`` the per-element sum
of ``|A[m,k]*B[k,n]|`` that the parity tolerance is scaled by.

Definitions followed (cited in full in ``oracle.c``): page "GEMM 优化详解",
section "GEMM 基础理论 / 数学定义" (C = alpha*A*B + beta*C) and section
"Level 6: Kernel Fusion" (ReLU(X*W + bias)); page "第5章-基础Kernel",
sections 1.1 and 7.1 (the sum over k and the CPU triple loop). The batched form
(page "GEMM 优化详解", section "矩阵大小选择策略": many small products as one
batched GEMM) is that definition applied to each batch item independently.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True, extra_flags=()) -> str:
    """Compile oracle.c into liboracle.so (gcc, OpenMP, strict IEEE double).

    ``extra_flags`` go to gcc as well (the sanitizer test builds a copy with
    AddressSanitizer and UndefinedBehaviorSanitizer this way)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra", *extra_flags,
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, f64, i32 = ctypes.c_int64, ctypes.c_double, ctypes.c_int
    vp = ctypes.c_void_p
    lib.oracle_gemm_f32.argtypes = [i64, i64, i64, f64, vp, i64, vp, i64, i32, f64, vp, i64, vp, vp, i32]
    lib.oracle_gemm_f16.argtypes = lib.oracle_gemm_f32.argtypes
    lib.oracle_gemm_bf16.argtypes = lib.oracle_gemm_f32.argtypes
    lib.oracle_linear.argtypes = [i64, i64, i64, vp, i64, vp, i64, i32, vp, i32, vp, vp, i32]
    lib.oracle_gemm_f32_at.argtypes = [i64, f64, vp, i64, vp, i64, i32, f64, vp, i64, i64, vp, vp, vp, vp, i32]
    lib.oracle_gemm_f16_at.argtypes = lib.oracle_gemm_f32_at.argtypes
    lib.oracle_gemm_bf16_at.argtypes = lib.oracle_gemm_f32_at.argtypes
    lib.oracle_linear_at.argtypes = [i64, vp, i64, vp, i64, i32, vp, i32, i64, vp, vp, vp, vp, i32]
    for f in (lib.oracle_gemm_f32, lib.oracle_gemm_f16, lib.oracle_gemm_bf16, lib.oracle_linear,
              lib.oracle_gemm_f32_at, lib.oracle_gemm_f16_at, lib.oracle_gemm_bf16_at,
              lib.oracle_linear_at):
        f.restype = None
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = f64
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = f64
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i32
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _mat(a, dtype, name):
    """A 2-D row-major view with unit column stride; returns (array, ld)."""
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"{name} must be {np.dtype(dtype).name}, got {a.dtype}")
    if a.ndim != 2:
        raise ValueError(f"{name} must be 2-D")
    if a.shape[1] > 0 and a.strides[1] != a.itemsize:
        a = np.ascontiguousarray(a)
    ld = a.strides[0] // a.itemsize if a.shape[0] > 1 else max(a.shape[1], 1)
    return a, ld


def _threads(nthreads):
    return int(nthreads) if nthreads else 0


def max_threads() -> int:
    return _load().oracle_max_threads()


def half_to_double(bits: int) -> float:
    """Decode one IEEE binary16 bit pattern (the oracle's own decoder)."""
    return _load().oracle_half_to_double(int(bits) & 0xFFFF)


def bf16_to_double(bits: int) -> float:
    """Decode one bfloat16 bit pattern (the oracle's own decoder)."""
    return _load().oracle_bf16_to_double(int(bits) & 0xFFFF)


def gemm(A, B, alpha=1.0, beta=0.0, C=None, nthreads=None, bf16=False, b_trans=False):
    """R = alpha*A*B + beta*C for fp32 A (MxK), B (KxN); C read only if beta != 0.

    A and B may instead be uint16 arrays of 16-bit bit patterns (both of them):
    binary16 by default, bfloat16 with ``bf16=True``. With ``b_trans=True``, B
    is given N-by-K and the product is alpha*A*B^T + beta*C.
    """
    lib = _load()
    half = np.asarray(A).dtype == np.uint16
    dt = np.uint16 if half else np.float32
    A, lda = _mat(A, dt, "A")
    B, ldb = _mat(B, dt, "B")
    M, K = A.shape
    N, K2 = B.shape if b_trans else B.shape[::-1]
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if beta != 0.0:
        C, ldc = _mat(C, np.float32, "C")
        if C.shape != (M, N):
            raise ValueError("C shape")
    else:
        C, ldc = None, max(N, 1)
    R = np.empty((M, N), np.float64)
    T = np.empty((M, N), np.float64)
    if bf16 and not half:
        raise TypeError("bf16=True needs uint16 bit patterns")
    fn = (lib.oracle_gemm_bf16 if bf16 else lib.oracle_gemm_f16) if half else lib.oracle_gemm_f32
    fn(M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb, int(b_trans), float(beta), _ptr(C), ldc,
       _ptr(R), _ptr(T), _threads(nthreads))
    return R, T


def linear(X, W, bias=None, act=1, nthreads=None, w_trans=False):
    """R = act(X*W + bias) for fp32 X (MxK), W (KxN), bias (N) or None.

    With ``w_trans=True``, W is given N-by-K (the layout of a PyTorch Linear
    weight) and the layer is act(X*W^T + bias).
    """
    lib = _load()
    X, ldx = _mat(X, np.float32, "X")
    W, ldw = _mat(W, np.float32, "W")
    M, K = X.shape
    N, K2 = W.shape if w_trans else W.shape[::-1]
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        if bias.shape != (N,):
            raise ValueError("bias shape")
    R = np.empty((M, N), np.float64)
    T = np.empty((M, N), np.float64)
    lib.oracle_linear(M, N, K, _ptr(X), ldx, _ptr(W), ldw, int(w_trans), _ptr(bias), int(act),
                      _ptr(R), _ptr(T), _threads(nthreads))
    return R, T


def gemm_batched(A, B, alpha=1.0, beta=0.0, C=None, nthreads=None, bf16=False, b_trans=False):
    """gemm() of every batch item: R[i] = alpha*A[i]*B[i] + beta*C[i].

    A, B (and C when beta != 0) are 3-D arrays whose first axis is the batch;
    an operand shared by every item may be given with batch stride 0
    (``numpy.broadcast_to``). Returns (R, T) of shape (batch, M, N).
    """
    A, B = np.asarray(A), np.asarray(B)
    if A.ndim != 3 or B.ndim != 3 or A.shape[0] != B.shape[0]:
        raise ValueError("A and B must be 3-D with the same batch size")
    nb, M = A.shape[0], A.shape[1]
    N = B.shape[1] if b_trans else B.shape[2]
    if beta != 0.0:
        C = np.asarray(C)
        if C.shape != (nb, M, N):
            raise ValueError("C shape")
    R = np.empty((nb, M, N), np.float64)
    T = np.empty((nb, M, N), np.float64)
    for i in range(nb):
        R[i], T[i] = gemm(A[i], B[i], alpha, beta, None if beta == 0.0 else C[i], nthreads,
                          bf16=bf16, b_trans=b_trans)
    return R, T


def _idx(rows, cols):
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D and of equal length")
    return rows, cols


def gemm_at(A, B, rows, cols, alpha=1.0, beta=0.0, C=None, nthreads=None, bf16=False,
            b_trans=False):
    """gemm() evaluated only at the positions (rows[p], cols[p])."""
    lib = _load()
    half = np.asarray(A).dtype == np.uint16
    dt = np.uint16 if half else np.float32
    A, lda = _mat(A, dt, "A")
    B, ldb = _mat(B, dt, "B")
    M, K = A.shape
    N, K2 = B.shape if b_trans else B.shape[::-1]
    if K2 != K:
        raise ValueError("inner dimensions differ")
    rows, cols = _idx(rows, cols)
    if rows.size and (rows.min() < 0 or rows.max() >= M or cols.min() < 0 or cols.max() >= N):
        raise IndexError("sample position out of range")
    if beta != 0.0:
        C, ldc = _mat(C, np.float32, "C")
        if C.shape != (M, N):
            raise ValueError("C shape")
    else:
        C, ldc = None, max(N, 1)
    R = np.empty(rows.size, np.float64)
    T = np.empty(rows.size, np.float64)
    if bf16 and not half:
        raise TypeError("bf16=True needs uint16 bit patterns")
    fn = (lib.oracle_gemm_bf16_at if bf16 else lib.oracle_gemm_f16_at) if half else lib.oracle_gemm_f32_at
    fn(K, float(alpha), _ptr(A), lda, _ptr(B), ldb, int(b_trans), float(beta), _ptr(C), ldc,
       rows.size, _ptr(rows), _ptr(cols), _ptr(R), _ptr(T), _threads(nthreads))
    return R, T


def linear_at(X, W, rows, cols, bias=None, act=1, nthreads=None, w_trans=False):
    """linear() evaluated only at the positions (rows[p], cols[p])."""
    lib = _load()
    X, ldx = _mat(X, np.float32, "X")
    W, ldw = _mat(W, np.float32, "W")
    M, K = X.shape
    N, K2 = W.shape if w_trans else W.shape[::-1]
    if K2 != K:
        raise ValueError("inner dimensions differ")
    rows, cols = _idx(rows, cols)
    if rows.size and (rows.min() < 0 or rows.max() >= M or cols.min() < 0 or cols.max() >= N):
        raise IndexError("sample position out of range")
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        if bias.shape != (N,):
            raise ValueError("bias shape")
    R = np.empty(rows.size, np.float64)
    T = np.empty(rows.size, np.float64)
    lib.oracle_linear_at(K, _ptr(X), ldx, _ptr(W), ldw, int(w_trans), _ptr(bias), int(act),
                         rows.size, _ptr(rows), _ptr(cols), _ptr(R), _ptr(T), _threads(nthreads))
    return R, T
