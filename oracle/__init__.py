"""CPU oracle for INT8 mixed-precision linear layers (row-wise scaling).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (``int8_mixed_precision_rowwise_amd``) never imports it and shares no
code with it.

This module is argument marshalling over ``i8mp_oracle.c`` (plain scalar C,
built with ``-O2 -fno-fast-math -ffp-contract=off``).  Arrays are numpy:
bf16 tensors travel as ``uint16`` bit patterns.

What each function computes, with its source, is documented in the C file.
Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` (closed forms, invariants, brute force against an
independent pure-Python rational implementation, numpy integer matmul, and
rocRAND's Philox4x32-10 for the random stream).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

RNE = 0
SR = 1
NT = 0
NN = 1
TN = 2
LAYOUTS = {"NT": NT, "NN": NN, "TN": TN}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _build.LIB_PATH
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
        _build.build()
    lib = ctypes.CDLL(path)
    i64, u64, i32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_int
    p = ctypes.c_void_p
    lib.oracle_philox4x32_10_block.argtypes = [p, p, p]
    lib.oracle_philox4x32_10_block.restype = None
    lib.oracle_philox_stream.argtypes = [u64, u64, i64, p]
    lib.oracle_philox_stream.restype = None
    for name in ("oracle_quantize_rowwise", "oracle_quantize_colwise"):
        f = getattr(lib, name)
        f.argtypes = [p, i64, i64, i64, p, i64, p, i32, u64, u64]
        f.restype = None
    lib.oracle_e4m3_to_float.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_float.restype = ctypes.c_float
    lib.oracle_float_to_e4m3.argtypes = [ctypes.c_float]
    lib.oracle_float_to_e4m3.restype = ctypes.c_uint8
    for name in ("oracle_quantize_rowwise_fp8", "oracle_quantize_colwise_fp8"):
        f = getattr(lib, name)
        f.argtypes = [p, i64, i64, i64, p, i64, p]
        f.restype = None
    lib.oracle_fp8_scaled_mm.argtypes = [i32, i64, i64, i64, p, i64, p, p, i64, p, p, i64, p, p]
    lib.oracle_fp8_scaled_mm.restype = None
    lib.oracle_fp8_scaled_mm_at.argtypes = [i32, i64, p, i64, p, p, i64, p, p, p, i64, p, p, p]
    lib.oracle_fp8_scaled_mm_at.restype = None
    lib.oracle_col_absmax.argtypes = [p, i64, i64, i64, p]
    lib.oracle_col_absmax.restype = None
    lib.oracle_quantize_given_u.argtypes = [p, i64, ctypes.c_float, i32, p, p]
    lib.oracle_quantize_given_u.restype = None
    lib.oracle_mm_i32.argtypes = [i32, i64, i64, i64, p, i64, p, i64, p, i64]
    lib.oracle_mm_i32.restype = i64
    lib.oracle_scaled_mm.argtypes = [i32, i64, i64, i64, p, i64, p, p, i64, p, p, i64]
    lib.oracle_scaled_mm.restype = i64
    lib.oracle_scaled_mm_at.argtypes = [i32, i64, p, i64, p, p, i64, p, p, p, i64, p, p]
    lib.oracle_scaled_mm_at.restype = i64
    lib.oracle_linear_fwd.argtypes = [p, p, p, i64, i64, i64, i32, u64, u64]
    lib.oracle_linear_fwd.restype = i64
    lib.oracle_linear_bwd.argtypes = [p, p, p, p, p, i64, i64, i64, i32, u64, u64]
    lib.oracle_linear_bwd.restype = i64
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _c(a: np.ndarray, dtype) -> np.ndarray:
    assert a.dtype == dtype, (a.dtype, dtype)
    return np.ascontiguousarray(a)


def _rows_ld(a: np.ndarray):
    """(rows, cols, leading dim in elements) of a 2-D array with unit column stride."""
    assert a.ndim == 2 and a.strides[1] == a.itemsize, "need unit stride along columns"
    return a.shape[0], a.shape[1], a.strides[0] // a.itemsize


def philox_block(counter, key) -> np.ndarray:
    """One Philox4x32-10 block: 4 uint32 counter words, 2 uint32 key words."""
    lib = _load()
    c = np.asarray(counter, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib.oracle_philox4x32_10_block(_ptr(c), _ptr(k), _ptr(out))
    return out


def philox_stream(seed: int, offset: int, n_blocks: int) -> np.ndarray:
    """4*n_blocks words; block i has counter (offset+i, 0, 0) and key seed."""
    lib = _load()
    out = np.zeros(4 * n_blocks, dtype=np.uint32)
    lib.oracle_philox_stream(seed & (2**64 - 1), offset & (2**64 - 1), n_blocks, _ptr(out))
    return out


def _quantize(fn, x, axis_len, rounding, seed, offset):
    assert x.dtype == np.uint16
    rows, cols, ldx = _rows_ld(x)
    q = np.zeros((rows, cols), dtype=np.int8)
    s = np.zeros(axis_len(rows, cols), dtype=np.float32)
    fn(_ptr(x), rows, cols, ldx, _ptr(q), cols, _ptr(s), int(rounding), seed & (2**64 - 1),
       offset & (2**64 - 1))
    return q, s


def quantize_rowwise(x: np.ndarray, rounding: int = RNE, seed: int = 0, offset: int = 0):
    """Row-wise dynamic quantization of bf16 bits ``x`` [rows, cols] -> (int8 q, fp32 scale[rows])."""
    return _quantize(_load().oracle_quantize_rowwise, x, lambda r, c: r, rounding, seed, offset)


def quantize_colwise(x: np.ndarray, rounding: int = RNE, seed: int = 0, offset: int = 0):
    """Column-wise dynamic quantization -> (int8 q in x's layout, fp32 scale[cols])."""
    return _quantize(_load().oracle_quantize_colwise, x, lambda r, c: c, rounding, seed, offset)


def col_absmax(x: np.ndarray) -> np.ndarray:
    """fp32 [cols]: the maximum |x| of each column of bf16 bits ``x`` (0 without rows)."""
    assert x.dtype == np.uint16
    rows, cols, ldx = _rows_ld(x)
    out = np.zeros(cols, dtype=np.float32)
    _load().oracle_col_absmax(_ptr(x), rows, cols, ldx, _ptr(out))
    return out


def quantize_given_u(x: np.ndarray, s: float, rounding: int, u: np.ndarray | None = None):
    """The rounding step alone: codes of bf16 bits ``x`` under scale ``s`` with
    caller-supplied uniforms ``u`` (float32, same length; unused under RNE)."""
    lib = _load()
    x = _c(x.ravel(), np.uint16)
    if u is not None:
        u = _c(u.ravel(), np.float32)
        assert u.size == x.size
    q = np.zeros(x.size, dtype=np.int8)
    lib.oracle_quantize_given_u(_ptr(x), x.size, float(s), int(rounding), _ptr(u), _ptr(q))
    return q


def _mnk(layout: int, A: np.ndarray, B: np.ndarray):
    ra, ca = A.shape
    rb, cb = B.shape
    if layout == NT:
        M, K, N = ra, ca, rb
        assert cb == K
    elif layout == NN:
        M, K, N = ra, ca, cb
        assert rb == K
    else:
        K, M, N = ra, ca, cb
        assert rb == K
    return M, N, K


def mm_i32(layout: int, A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """int32 C[M,N] = sum_k A(m,k) B(k,n) for the layout (NT: A@B.T, NN: A@B, TN: A.T@B)."""
    lib = _load()
    assert A.dtype == np.int8 and B.dtype == np.int8
    M, N, K = _mnk(layout, A, B)
    _, _, lda = _rows_ld(A)
    _, _, ldb = _rows_ld(B)
    C = np.zeros((M, N), dtype=np.int32)
    bad = lib.oracle_mm_i32(layout, M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), N)
    if bad:
        raise OverflowError(f"{bad} outputs exceed int32")
    return C


def scaled_mm(layout: int, A, sa, B, sb) -> np.ndarray:
    """bf16 bits C[M,N] = bf16(((float)acc * sa[m]) * sb[n])."""
    lib = _load()
    M, N, K = _mnk(layout, A, B)
    _, _, lda = _rows_ld(A)
    _, _, ldb = _rows_ld(B)
    sa = _c(sa, np.float32)
    sb = _c(sb, np.float32)
    assert sa.shape == (M,) and sb.shape == (N,)
    C = np.zeros((M, N), dtype=np.uint16)
    bad = lib.oracle_scaled_mm(layout, M, N, K, _ptr(A), lda, _ptr(sa), _ptr(B), ldb, _ptr(sb),
                               _ptr(C), N)
    if bad:
        raise OverflowError(f"{bad} outputs exceed int32")
    return C


def scaled_mm_at(layout: int, A, sa, B, sb, ms, ns):
    """(int32 acc, bf16 bits y) at output positions (ms[i], ns[i])."""
    lib = _load()
    M, N, K = _mnk(layout, A, B)
    _, _, lda = _rows_ld(A)
    _, _, ldb = _rows_ld(B)
    sa = _c(sa, np.float32)
    sb = _c(sb, np.float32)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    assert ms.shape == ns.shape and (ms < M).all() and (ns < N).all()
    acc = np.zeros(ms.shape, dtype=np.int32)
    y = np.zeros(ms.shape, dtype=np.uint16)
    bad = lib.oracle_scaled_mm_at(layout, K, _ptr(A), lda, _ptr(sa), _ptr(B), ldb, _ptr(sb),
                                  _ptr(ms), _ptr(ns), ms.size, _ptr(acc), _ptr(y))
    if bad:
        raise OverflowError(f"{bad} outputs exceed int32")
    return acc, y


def linear_fwd(X, W, rounding=RNE, seed=0, offset=0):
    """Y[M,N] (bf16 bits) = scaled INT8 X @ W.T, both quantized row-wise over K."""
    lib = _load()
    X = _c(X, np.uint16)
    W = _c(W, np.uint16)
    M, K = X.shape
    N, K2 = W.shape
    assert K == K2
    Y = np.zeros((M, N), dtype=np.uint16)
    bad = lib.oracle_linear_fwd(_ptr(X), _ptr(W), _ptr(Y), M, N, K, int(rounding), seed, offset)
    if bad:
        raise OverflowError("int32 overflow or allocation failure")
    return Y


def linear_bwd(dY, X, W, rounding=RNE, seed=0, offset=0, want_dx=True, want_dw=True):
    """(dX[M,K], dW[N,K]) as bf16 bits; either may be skipped (returned as None)."""
    lib = _load()
    dY = _c(dY, np.uint16)
    X = _c(X, np.uint16)
    W = _c(W, np.uint16)
    M, N = dY.shape
    N2, K = W.shape
    assert N == N2 and X.shape == (M, K)
    dX = np.zeros((M, K), dtype=np.uint16) if want_dx else None
    dW = np.zeros((N, K), dtype=np.uint16) if want_dw else None
    bad = lib.oracle_linear_bwd(_ptr(dY), _ptr(X), _ptr(W), _ptr(dX), _ptr(dW), M, N, K,
                                int(rounding), seed, offset)
    if bad:
        raise OverflowError("int32 overflow or allocation failure")
    return dX, dW


# --------------------------------------------------------------------------- FP8 (E4M3)


def e4m3_to_float(codes) -> np.ndarray:
    """float32 values of E4M3 codes (uint8); 0x7F / 0xFF are NaN."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e4m3_to_float(int(v)) for v in c.ravel()], dtype=np.float32).reshape(c.shape)


def float_to_e4m3(values) -> np.ndarray:
    """Nearest E4M3 codes (ties to even, saturating at +-448) of float32 values."""
    lib = _load()
    v = np.asarray(values, dtype=np.float32)
    return np.array([lib.oracle_float_to_e4m3(float(x)) for x in v.ravel()], dtype=np.uint8).reshape(v.shape)


def _quantize_fp8(fn, x, axis_len):
    assert x.dtype == np.uint16
    rows, cols, ldx = _rows_ld(x)
    q = np.zeros((rows, cols), dtype=np.uint8)
    s = np.zeros(axis_len(rows, cols), dtype=np.float32)
    fn(_ptr(x), rows, cols, ldx, _ptr(q), cols, _ptr(s))
    return q, s


def quantize_rowwise_fp8(x: np.ndarray):
    """Row-wise FP8 quantization of bf16 bits ``x`` -> (E4M3 codes uint8, fp32 scale[rows])."""
    return _quantize_fp8(_load().oracle_quantize_rowwise_fp8, x, lambda r, c: r)


def quantize_colwise_fp8(x: np.ndarray):
    """Column-wise FP8 quantization -> (E4M3 codes in x's layout, fp32 scale[cols])."""
    return _quantize_fp8(_load().oracle_quantize_colwise_fp8, x, lambda r, c: c)


def fp8_scaled_mm(layout: int, A, sa, B, sb, want_acc=False):
    """bf16 bits of the FP8 scaled matmul (exact dot products rounded once to
    fp32, then the epilogue); with want_acc also (acc fp32, sum|a*b| fp64)."""
    A = _c(A, np.uint8)
    B = _c(B, np.uint8)
    M, N, K = _mnk(layout, A, B)
    C = np.zeros((M, N), dtype=np.uint16)
    acc = np.zeros((M, N), dtype=np.float32) if want_acc else None
    absdot = np.zeros((M, N), dtype=np.float64) if want_acc else None
    _load().oracle_fp8_scaled_mm(layout, M, N, K, _ptr(A), A.shape[1], _ptr(_c(sa, np.float32)), _ptr(B),
                                 B.shape[1], _ptr(_c(sb, np.float32)), _ptr(C), N, _ptr(acc), _ptr(absdot))
    return (C, acc, absdot) if want_acc else C


def fp8_scaled_mm_at(layout: int, A, sa, B, sb, ms, ns):
    """FP8 scaled matmul at output positions (ms[i], ns[i]) ->
    (bf16 bits, fp32 accumulators, sum |a*b| in fp64)."""
    A = _c(A, np.uint8)
    B = _c(B, np.uint8)
    M, N, K = _mnk(layout, A, B)
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    assert ((ms >= 0) & (ms < M)).all() and ((ns >= 0) & (ns < N)).all()
    y = np.zeros(len(ms), dtype=np.uint16)
    acc = np.zeros(len(ms), dtype=np.float32)
    absdot = np.zeros(len(ms), dtype=np.float64)
    _load().oracle_fp8_scaled_mm_at(layout, K, _ptr(A), A.shape[1], _ptr(_c(sa, np.float32)), _ptr(B),
                                    B.shape[1], _ptr(_c(sb, np.float32)), _ptr(ms), _ptr(ns), len(ms),
                                    _ptr(y), _ptr(acc), _ptr(absdot))
    return y, acc, absdot
