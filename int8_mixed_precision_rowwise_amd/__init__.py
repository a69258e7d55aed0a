"""INT8 mixed-precision linear layers with row-wise scaling, on MI355X (gfx950).

Thin ctypes binding over ``libi8mp.so`` (C ABI in ``include/i8mp.h``).  This
module only marshals torch tensors into device pointers, leading dimensions
and the current HIP stream; every step of the computation runs in the
library's HIP kernels.  There is no CPU or PyTorch fallback: if the library
is missing, importing this package raises.

torch must be imported before the library is loaded so that the process has
one HIP runtime (torch's); ``libi8mp.so`` then binds to it by soname.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

__all__ = [
    "I8mpError", "RNE", "SR", "NT", "NN", "TN", "MAX_CONTRACTION", "lib",
    "quantize_rowwise", "quantize_colwise", "int8_scaled_mm", "int8_mm_i32",
    "philox4x32_10", "linear_fwd", "linear_bwd", "linear_workspace_bytes",
    "colwise_workspace_bytes", "quantize_rowwise_colmax", "quantize_colwise_given_colmax",
    "rowwise_colmax_workspace_bytes", "linear_fwd_colmax", "quantize_rowwise_fp8",
    "quantize_colwise_fp8", "fp8_scaled_mm", "fp8_mm_f32", "linear_fwd_fp8", "linear_bwd_fp8",
    "EXPORTED_SYMBOLS",
]

RNE, SR = 0, 1
NT, NN, TN = 0, 1, 2
_LAYOUTS = {"NT": NT, "NN": NN, "TN": TN, NT: NT, NN: NN, TN: TN}
_ROUNDING = {"rne": RNE, "sr": SR, RNE: RNE, SR: SR}
MAX_CONTRACTION = 133144

EXPORTED_SYMBOLS = (
    "i8mp_status_str", "i8mp_abi_version", "i8mp_quantize_rowwise",
    "i8mp_quantize_colwise_workspace_bytes", "i8mp_quantize_colwise", "i8mp_int8_scaled_mm",
    "i8mp_int8_mm_i32", "i8mp_philox4x32_10", "i8mp_linear_workspace_bytes", "i8mp_linear_fwd",
    "i8mp_linear_bwd", "i8mp_quantize_rowwise_colmax_workspace_bytes",
    "i8mp_quantize_rowwise_colmax", "i8mp_quantize_colwise_given_colmax", "i8mp_linear_fwd_colmax",
    "i8mp_linear_bwd_colmax", "i8mp_quantize_rowwise_fp8", "i8mp_quantize_colwise_fp8",
    "i8mp_fp8_scaled_mm", "i8mp_fp8_mm_f32", "i8mp_linear_fwd_fp8", "i8mp_linear_bwd_fp8",
)


class I8mpError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({lib.i8mp_status_str(status).decode()})")


class _Opts(ctypes.Structure):
    _fields_ = [("round", ctypes.c_int32), ("seed", ctypes.c_uint64), ("offset", ctypes.c_uint64)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(_build.LIB_PATH):
        raise ImportError(
            f"{_build.LIB_PATH} is missing: build it with `python -m "
            "int8_mixed_precision_rowwise_amd.build` (there is no fallback path)")
    L = ctypes.CDLL(_build.LIB_PATH)
    p, i64, i32, u64, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64,
                            ctypes.c_size_t)
    sigs = {
        "i8mp_status_str": ([i32], ctypes.c_char_p),
        "i8mp_abi_version": ([], i32),
        "i8mp_quantize_rowwise": ([p, i64, i64, i64, p, i64, p, i32, u64, u64, p], i32),
        "i8mp_quantize_colwise_workspace_bytes": ([i64, i64], sz),
        "i8mp_quantize_colwise": ([p, i64, i64, i64, p, i64, p, i32, u64, u64, p, sz, p], i32),
        "i8mp_int8_scaled_mm": ([i32, i64, i64, i64, p, i64, p, p, i64, p, p, i64, p], i32),
        "i8mp_int8_mm_i32": ([i32, i64, i64, i64, p, i64, p, i64, p, i64, p], i32),
        "i8mp_philox4x32_10": ([u64, u64, i64, p, p], i32),
        "i8mp_linear_workspace_bytes": ([i64, i64, i64, i32], sz),
        "i8mp_linear_fwd": ([p, p, p, i64, i64, i64, ctypes.POINTER(_Opts), p, sz, p], i32),
        "i8mp_linear_bwd": ([p, p, p, p, p, i64, i64, i64, ctypes.POINTER(_Opts), p, sz, p], i32),
        "i8mp_quantize_rowwise_colmax_workspace_bytes": ([i64, i64], sz),
        "i8mp_quantize_rowwise_colmax": ([p, i64, i64, i64, p, i64, p, p, i32, u64, u64, p, sz, p], i32),
        "i8mp_quantize_colwise_given_colmax": ([p, i64, i64, i64, p, p, i64, p, i32, u64, u64, p], i32),
        "i8mp_linear_fwd_colmax": ([p, p, p, i64, i64, i64, ctypes.POINTER(_Opts), p, p, p, sz, p], i32),
        "i8mp_linear_bwd_colmax": ([p, p, p, p, p, i64, i64, i64, ctypes.POINTER(_Opts), p, p, p, sz, p],
                                   i32),
        "i8mp_quantize_rowwise_fp8": ([p, i64, i64, i64, p, i64, p, p], i32),
        "i8mp_quantize_colwise_fp8": ([p, i64, i64, i64, p, i64, p, p, sz, p], i32),
        "i8mp_fp8_scaled_mm": ([i32, i64, i64, i64, p, i64, p, p, i64, p, p, i64, p], i32),
        "i8mp_fp8_mm_f32": ([i32, i64, i64, i64, p, i64, p, i64, p, i64, p], i32),
        "i8mp_linear_fwd_fp8": ([p, p, p, i64, i64, i64, p, sz, p], i32),
        "i8mp_linear_bwd_fp8": ([p, p, p, p, p, i64, i64, i64, p, sz, p], i32),
    }
    for name, (args, res) in sigs.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    return L


lib = _load()


# --------------------------------------------------------------------------- helpers


def _ptr(t: torch.Tensor | None):
    return None if t is None or t.numel() == 0 else ctypes.c_void_p(t.data_ptr())


def _ld(t: torch.Tensor) -> int:
    assert t.dim() == 2, "2-D tensor expected"
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("columns must be contiguous (stride 1)")
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check(status: int, what: str):
    if status != 0:
        raise I8mpError(status, what)


def _empty_2d(rows: int, cols: int, dtype, device) -> torch.Tensor:
    """[rows, cols] view of storage whose rows are padded to 16 bytes."""
    per = 16 // torch.empty((), dtype=dtype).element_size()
    ld = max(per, (cols + per - 1) // per * per)
    return torch.empty((rows, ld), dtype=dtype, device=device)[:, :cols]


def _bits(t: torch.Tensor, dtype=torch.bfloat16) -> torch.Tensor:
    if t.dtype != dtype:
        raise TypeError(f"{dtype} tensor expected, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    return t


# --------------------------------------------------------------------------- primitives


def quantize_rowwise(x: torch.Tensor, rounding="rne", seed: int = 0, offset: int = 0,
                     q: torch.Tensor | None = None, scale: torch.Tensor | None = None):
    """Row-wise dynamic INT8 quantization of bf16 ``x`` [R, C] -> (int8 q [R, C], fp32 scale [R])."""
    _bits(x)
    R, C = x.shape
    q = _empty_2d(R, C, torch.int8, x.device) if q is None else q
    scale = torch.empty(R, dtype=torch.float32, device=x.device) if scale is None else scale
    with torch.cuda.device(x.device):
        st = lib.i8mp_quantize_rowwise(_ptr(x), R, C, _ld(x), _ptr(q), _ld(q), _ptr(scale),
                                       _ROUNDING[rounding], seed, offset, _stream(x.device))
    _check(st, "i8mp_quantize_rowwise")
    return q, scale


def rowwise_colmax_workspace_bytes(rows: int, cols: int) -> int:
    return lib.i8mp_quantize_rowwise_colmax_workspace_bytes(rows, cols)


def quantize_rowwise_colmax(x: torch.Tensor, rounding="rne", seed: int = 0, offset: int = 0,
                            q: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                            colmax: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None):
    """Row-wise quantization that also returns the column maxima of |x|:
    (int8 q [R, C], fp32 scale [R], fp32 colmax [C])."""
    _bits(x)
    R, C = x.shape
    q = _empty_2d(R, C, torch.int8, x.device) if q is None else q
    scale = torch.empty(R, dtype=torch.float32, device=x.device) if scale is None else scale
    colmax = torch.empty(C, dtype=torch.float32, device=x.device) if colmax is None else colmax
    need = rowwise_colmax_workspace_bytes(R, C)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        st = lib.i8mp_quantize_rowwise_colmax(_ptr(x), R, C, _ld(x), _ptr(q), _ld(q), _ptr(scale),
                                              _ptr(colmax), _ROUNDING[rounding], seed, offset,
                                              _ptr(workspace), workspace.numel(), _stream(x.device))
    _check(st, "i8mp_quantize_rowwise_colmax")
    return q, scale, colmax


def quantize_colwise_given_colmax(x: torch.Tensor, colmax: torch.Tensor, rounding="rne",
                                  seed: int = 0, offset: int = 0, q: torch.Tensor | None = None,
                                  scale: torch.Tensor | None = None):
    """Column-wise quantization with known column maxima (one pass):
    (int8 q [R, C] in x's layout, fp32 scale [C])."""
    _bits(x)
    _bits(colmax, torch.float32)
    R, C = x.shape
    q = _empty_2d(R, C, torch.int8, x.device) if q is None else q
    scale = torch.empty(C, dtype=torch.float32, device=x.device) if scale is None else scale
    with torch.cuda.device(x.device):
        st = lib.i8mp_quantize_colwise_given_colmax(_ptr(x), R, C, _ld(x), _ptr(colmax), _ptr(q),
                                                    _ld(q), _ptr(scale), _ROUNDING[rounding], seed,
                                                    offset, _stream(x.device))
    _check(st, "i8mp_quantize_colwise_given_colmax")
    return q, scale


def colwise_workspace_bytes(rows: int, cols: int) -> int:
    return lib.i8mp_quantize_colwise_workspace_bytes(rows, cols)


def quantize_colwise(x: torch.Tensor, rounding="rne", seed: int = 0, offset: int = 0,
                     q: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None):
    """Column-wise dynamic INT8 quantization -> (int8 q [R, C] in x's layout, fp32 scale [C])."""
    _bits(x)
    R, C = x.shape
    q = _empty_2d(R, C, torch.int8, x.device) if q is None else q
    scale = torch.empty(C, dtype=torch.float32, device=x.device) if scale is None else scale
    need = colwise_workspace_bytes(R, C)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        st = lib.i8mp_quantize_colwise(_ptr(x), R, C, _ld(x), _ptr(q), _ld(q), _ptr(scale),
                                       _ROUNDING[rounding], seed, offset, _ptr(workspace),
                                       workspace.numel(), _stream(x.device))
    _check(st, "i8mp_quantize_colwise")
    return q, scale


def _mnk(layout: int, A: torch.Tensor, B: torch.Tensor):
    if layout == NT:
        M, K = A.shape
        N = B.shape[0]
        ok = B.shape[1] == K
    elif layout == NN:
        M, K = A.shape
        N = B.shape[1]
        ok = B.shape[0] == K
    else:
        K, M = A.shape
        N = B.shape[1]
        ok = B.shape[0] == K
    if not ok:
        raise ValueError(f"operand shapes {tuple(A.shape)} and {tuple(B.shape)} do not match layout")
    return M, N, K


def int8_scaled_mm(layout, A: torch.Tensor, scale_a: torch.Tensor, B: torch.Tensor,
                   scale_b: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 C[M,N] = bf16(((float)(A(m,:) . B(:,n)) * scale_a[m]) * scale_b[n]).

    layout: "NT" (A [M,K], B [N,K]), "NN" (A [M,K], B [K,N]) or "TN" (A [K,M], B [K,N])."""
    layout = _LAYOUTS[layout]
    _bits(A, torch.int8), _bits(B, torch.int8)
    M, N, K = _mnk(layout, A, B)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device) if out is None else out
    with torch.cuda.device(A.device):
        st = lib.i8mp_int8_scaled_mm(layout, M, N, K, _ptr(A), _ld(A), _ptr(scale_a), _ptr(B),
                                     _ld(B), _ptr(scale_b), _ptr(out), _ld(out), _stream(A.device))
    _check(st, "i8mp_int8_scaled_mm")
    return out


def int8_mm_i32(layout, A: torch.Tensor, B: torch.Tensor,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """int32 C[M,N] = A(m,:) . B(:,n) (same layouts as int8_scaled_mm)."""
    layout = _LAYOUTS[layout]
    _bits(A, torch.int8), _bits(B, torch.int8)
    M, N, K = _mnk(layout, A, B)
    out = torch.empty((M, N), dtype=torch.int32, device=A.device) if out is None else out
    with torch.cuda.device(A.device):
        st = lib.i8mp_int8_mm_i32(layout, M, N, K, _ptr(A), _ld(A), _ptr(B), _ld(B), _ptr(out),
                                  _ld(out), _stream(A.device))
    _check(st, "i8mp_int8_mm_i32")
    return out


def philox4x32_10(seed: int, offset: int, n_blocks: int, device="cuda") -> torch.Tensor:
    """uint32 words (returned as int32) [4 * n_blocks] of Philox4x32-10 blocks offset.."""
    out = torch.empty(4 * n_blocks, dtype=torch.int32, device=device)
    with torch.cuda.device(out.device):
        st = lib.i8mp_philox4x32_10(seed, offset, n_blocks, _ptr(out), _stream(out.device))
    _check(st, "i8mp_philox4x32_10")
    return out


# --------------------------------------------------------------------------- linear layer


def linear_workspace_bytes(M: int, N: int, K: int, backward: bool) -> int:
    return lib.i8mp_linear_workspace_bytes(M, N, K, int(backward))


def _opts(rounding, seed, offset):
    return _Opts(_ROUNDING[rounding], seed & (2**64 - 1), offset & (2**64 - 1))


def linear_fwd(X: torch.Tensor, W: torch.Tensor, rounding="rne", seed: int = 0, offset: int = 0,
               out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Y = X @ W.T with both operands quantized row-wise over K (dense bf16 tensors)."""
    _bits(X), _bits(W)
    M, K = X.shape
    N = W.shape[0]
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device) if out is None else out
    need = linear_workspace_bytes(M, N, K, False)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    o = _opts(rounding, seed, offset)
    with torch.cuda.device(X.device):
        st = lib.i8mp_linear_fwd(_ptr(X), _ptr(W), _ptr(Y), M, N, K, ctypes.byref(o),
                                 _ptr(workspace), workspace.numel(), _stream(X.device))
    _check(st, "i8mp_linear_fwd")
    return Y


def linear_fwd_colmax(X: torch.Tensor, W: torch.Tensor, rounding="rne", seed: int = 0,
                      offset: int = 0, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None):
    """linear_fwd that also returns the column maxima of X and W (fp32 [K]
    each) for linear_bwd: (Y, colmax_x, colmax_w)."""
    _bits(X), _bits(W)
    M, K = X.shape
    N = W.shape[0]
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device) if out is None else out
    cx = torch.empty(K, dtype=torch.float32, device=X.device)
    cw = torch.empty(K, dtype=torch.float32, device=X.device)
    need = linear_workspace_bytes(M, N, K, False)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    o = _opts(rounding, seed, offset)
    with torch.cuda.device(X.device):
        st = lib.i8mp_linear_fwd_colmax(_ptr(X), _ptr(W), _ptr(Y), M, N, K, ctypes.byref(o),
                                        _ptr(cx), _ptr(cw), _ptr(workspace), workspace.numel(),
                                        _stream(X.device))
    _check(st, "i8mp_linear_fwd_colmax")
    return Y, cx, cw


def linear_bwd(dY: torch.Tensor, X: torch.Tensor, W: torch.Tensor, rounding="rne", seed: int = 0,
               offset: int = 0, want_dx: bool = True, want_dw: bool = True,
               dX: torch.Tensor | None = None, dW: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, colmax_x: torch.Tensor | None = None,
               colmax_w: torch.Tensor | None = None):
    """(dX = dY @ W, dW = dY.T @ X), each quantized along its own contraction.
    colmax_x / colmax_w: the column maxima from linear_fwd_colmax (optional;
    the results are the same, the column-wise passes then read X / W once)."""
    _bits(dY), _bits(X), _bits(W)
    for c in (colmax_x, colmax_w):
        if c is not None:
            _bits(c, torch.float32)
    M, N = dY.shape
    K = W.shape[1]
    if want_dx and dX is None:
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=dY.device)
    if want_dw and dW is None:
        dW = torch.empty((N, K), dtype=torch.bfloat16, device=dY.device)
    need = linear_workspace_bytes(M, N, K, True)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dY.device)
    o = _opts(rounding, seed, offset)
    with torch.cuda.device(dY.device):
        st = lib.i8mp_linear_bwd_colmax(_ptr(dY), _ptr(X), _ptr(W), _ptr(dX if want_dx else None),
                                        _ptr(dW if want_dw else None), M, N, K, ctypes.byref(o),
                                        _ptr(colmax_x), _ptr(colmax_w), _ptr(workspace),
                                        workspace.numel(), _stream(dY.device))
    _check(st, "i8mp_linear_bwd_colmax")
    return (dX if want_dx else None), (dW if want_dw else None)


# --------------------------------------------------------------------------- FP8 (E4M3) variant


def quantize_rowwise_fp8(x: torch.Tensor, q: torch.Tensor | None = None,
                         scale: torch.Tensor | None = None):
    """Row-wise FP8 quantization of bf16 ``x`` [R, C] -> (E4M3 codes as uint8 [R, C],
    fp32 scale [R]); ``codes.view(torch.float8_e4m3fn)`` gives torch's view of them."""
    _bits(x)
    R, C = x.shape
    q = _empty_2d(R, C, torch.uint8, x.device) if q is None else q
    scale = torch.empty(R, dtype=torch.float32, device=x.device) if scale is None else scale
    with torch.cuda.device(x.device):
        st = lib.i8mp_quantize_rowwise_fp8(_ptr(x), R, C, _ld(x), _ptr(q), _ld(q), _ptr(scale),
                                           _stream(x.device))
    _check(st, "i8mp_quantize_rowwise_fp8")
    return q, scale


def quantize_colwise_fp8(x: torch.Tensor, q: torch.Tensor | None = None,
                         scale: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Column-wise FP8 quantization -> (E4M3 codes uint8 [R, C] in x's layout, fp32 scale [C])."""
    _bits(x)
    R, C = x.shape
    q = _empty_2d(R, C, torch.uint8, x.device) if q is None else q
    scale = torch.empty(C, dtype=torch.float32, device=x.device) if scale is None else scale
    need = colwise_workspace_bytes(R, C)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        st = lib.i8mp_quantize_colwise_fp8(_ptr(x), R, C, _ld(x), _ptr(q), _ld(q), _ptr(scale),
                                           _ptr(workspace), workspace.numel(), _stream(x.device))
    _check(st, "i8mp_quantize_colwise_fp8")
    return q, scale


def fp8_scaled_mm(layout, A: torch.Tensor, scale_a: torch.Tensor, B: torch.Tensor,
                  scale_b: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 C[M,N] from E4M3 codes (uint8): fp32 sums of the exact products, then
    bf16((sum * scale_a[m]) * scale_b[n]).  Layouts as for int8_scaled_mm; K % 16 == 0."""
    layout = _LAYOUTS[layout]
    _bits(A, torch.uint8), _bits(B, torch.uint8)
    M, N, K = _mnk(layout, A, B)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device) if out is None else out
    with torch.cuda.device(A.device):
        st = lib.i8mp_fp8_scaled_mm(layout, M, N, K, _ptr(A), _ld(A), _ptr(scale_a), _ptr(B),
                                    _ld(B), _ptr(scale_b), _ptr(out), _ld(out), _stream(A.device))
    _check(st, "i8mp_fp8_scaled_mm")
    return out


def fp8_mm_f32(layout, A: torch.Tensor, B: torch.Tensor,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """float32 C[M,N]: the matrix core's fp32 sums of E4M3 products (same layouts
    as fp8_scaled_mm, no scales)."""
    layout = _LAYOUTS[layout]
    _bits(A, torch.uint8), _bits(B, torch.uint8)
    M, N, K = _mnk(layout, A, B)
    out = torch.empty((M, N), dtype=torch.float32, device=A.device) if out is None else out
    with torch.cuda.device(A.device):
        st = lib.i8mp_fp8_mm_f32(layout, M, N, K, _ptr(A), _ld(A), _ptr(B), _ld(B), _ptr(out),
                                 _ld(out), _stream(A.device))
    _check(st, "i8mp_fp8_mm_f32")
    return out


def linear_fwd_fp8(X: torch.Tensor, W: torch.Tensor, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None):
    """Y = X @ W.T with both operands quantized row-wise to FP8 (E4M3) over K."""
    _bits(X), _bits(W)
    M, K = X.shape
    N = W.shape[0]
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device) if out is None else out
    need = linear_workspace_bytes(M, N, K, False)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    with torch.cuda.device(X.device):
        st = lib.i8mp_linear_fwd_fp8(_ptr(X), _ptr(W), _ptr(Y), M, N, K, _ptr(workspace),
                                     workspace.numel(), _stream(X.device))
    _check(st, "i8mp_linear_fwd_fp8")
    return Y


def linear_bwd_fp8(dY: torch.Tensor, X: torch.Tensor, W: torch.Tensor, want_dx: bool = True,
                   want_dw: bool = True, workspace: torch.Tensor | None = None):
    """(dX = dY @ W, dW = dY.T @ X) with FP8 (E4M3) operands, each quantized along
    its own contraction."""
    _bits(dY), _bits(X), _bits(W)
    M, N = dY.shape
    K = W.shape[1]
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dY.device) if want_dx else None
    dW = torch.empty((N, K), dtype=torch.bfloat16, device=dY.device) if want_dw else None
    need = linear_workspace_bytes(M, N, K, True)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dY.device)
    with torch.cuda.device(dY.device):
        st = lib.i8mp_linear_bwd_fp8(_ptr(dY), _ptr(X), _ptr(W), _ptr(dX), _ptr(dW), M, N, K,
                                     _ptr(workspace), workspace.numel(), _stream(dY.device))
    _check(st, "i8mp_linear_bwd_fp8")
    return dX, dW
