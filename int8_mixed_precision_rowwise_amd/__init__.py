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
    "linear_fwd_fp8_colmax",
    "quantize_colwise_noalloc", "STATIC_SCRATCH_BYTES", "mfma_rate_probe", "EXPORTED_SYMBOLS",
]

RNE, SR = 0, 1
NT, NN, TN = 0, 1, 2
_LAYOUTS = {"NT": NT, "NN": NN, "TN": TN, NT: NT, NN: NN, TN: TN}
_ROUNDING = {"rne": RNE, "sr": SR, RNE: RNE, SR: SR}
MAX_CONTRACTION = 133144
STATIC_SCRATCH_BYTES = 4 << 20  # the library's per-GPU scratch of i8mp_quantize_colwise_noalloc

EXPORTED_SYMBOLS = (
    "i8mp_status_str", "i8mp_abi_version", "i8mp_quantize_rowwise",
    "i8mp_quantize_colwise_workspace_bytes", "i8mp_quantize_colwise", "i8mp_int8_scaled_mm",
    "i8mp_int8_mm_i32", "i8mp_philox4x32_10", "i8mp_linear_workspace_bytes", "i8mp_linear_fwd",
    "i8mp_linear_bwd", "i8mp_quantize_rowwise_colmax_workspace_bytes",
    "i8mp_quantize_rowwise_colmax", "i8mp_quantize_colwise_given_colmax", "i8mp_linear_fwd_colmax",
    "i8mp_linear_bwd_colmax", "i8mp_quantize_rowwise_fp8", "i8mp_quantize_colwise_fp8",
    "i8mp_fp8_scaled_mm", "i8mp_fp8_mm_f32", "i8mp_linear_fwd_fp8", "i8mp_linear_bwd_fp8",
    "i8mp_linear_fwd_fp8_colmax", "i8mp_linear_bwd_fp8_colmax",
    "i8mp_quantize_colwise_noalloc", "i8mp_mfma_rate_probe",
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
        "i8mp_linear_fwd_fp8_colmax": ([p, p, p, i64, i64, i64, p, p, p, sz, p], i32),
        "i8mp_linear_bwd_fp8_colmax": ([p, p, p, p, p, i64, i64, i64, p, p, p, sz, p], i32),
        "i8mp_quantize_colwise_noalloc": ([p, i64, i64, i64, p, i64, p, i32, u64, u64, p], i32),
        "i8mp_mfma_rate_probe": ([p, i64, i64, p, p], i32),
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


# Argument checks.  The C ABI receives bare pointers and sizes, so every
# tensor's dtype, shape, layout and device is checked here, before the call:
# a mismatch raises (TypeError for a wrong type or dtype, ValueError for a
# wrong shape, layout or device) and nothing is launched.  Type and shape
# checks come first and the device check last, so they hold on any device.


def _tensor(t, name: str, dtype) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: torch.Tensor expected, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: {dtype} tensor expected, got {t.dtype}")
    return t


def _mat(t, name: str, dtype, shape=None, dense: bool = False) -> torch.Tensor:
    """2-D matrix of `dtype`, rows with contiguous columns (a leading
    dimension), of `shape` if given; `dense`: fully contiguous (the linear
    chains take leading dimension = columns)."""
    _tensor(t, name, dtype)
    if t.dim() != 2:
        raise ValueError(f"{name}: 2-D tensor expected, got {t.dim()}-D")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(shape)} expected, got {tuple(t.shape)}")
    if t.numel() > 0:
        if t.shape[1] > 1 and t.stride(1) != 1:
            raise ValueError(f"{name}: columns must be contiguous (stride 1)")
        if t.shape[0] > 1 and t.stride(0) < t.shape[1]:
            raise ValueError(f"{name}: row stride {t.stride(0)} is shorter than a row ({t.shape[1]})")
        if dense and not t.is_contiguous():
            raise ValueError(f"{name}: contiguous tensor expected")
    return t


def _vec(t, name: str, n: int, dtype=torch.float32) -> torch.Tensor:
    """Contiguous 1-D vector of n elements."""
    _tensor(t, name, dtype)
    if t.dim() != 1 or t.numel() != n:
        raise ValueError(f"{name}: 1-D tensor of {n} elements expected, got shape {tuple(t.shape)}")
    if n > 1 and t.stride(0) != 1:
        raise ValueError(f"{name}: contiguous tensor expected")
    return t


def _workspace(t, name: str = "workspace") -> torch.Tensor:
    _tensor(t, name, torch.uint8)
    if t.dim() != 1 or not t.is_contiguous():
        raise ValueError(f"{name}: contiguous 1-D uint8 tensor expected")
    return t


def _device(*ts) -> torch.device:
    """The one GPU that every given tensor lives on."""
    devs = {t.device for t in ts if t is not None}
    if len(devs) != 1:
        raise ValueError(f"tensors on one device expected, got {sorted(str(d) for d in devs)}")
    dev = devs.pop()
    if dev.type != "cuda":
        raise ValueError(f"device tensors expected, got tensors on {dev}")
    return dev


# --------------------------------------------------------------------------- primitives


def quantize_rowwise(x: torch.Tensor, rounding="rne", seed: int = 0, offset: int = 0,
                     q: torch.Tensor | None = None, scale: torch.Tensor | None = None):
    """Row-wise dynamic INT8 quantization of bf16 ``x`` [R, C] -> (int8 q [R, C], fp32 scale [R])."""
    _mat(x, "x", torch.bfloat16)
    R, C = x.shape
    if q is not None:
        _mat(q, "q", torch.int8, (R, C))
    if scale is not None:
        _vec(scale, "scale", R)
    dev = _device(x, q, scale)
    q = _empty_2d(R, C, torch.int8, dev) if q is None else q
    scale = torch.empty(R, dtype=torch.float32, device=dev) if scale is None else scale
    with torch.cuda.device(dev):
        st = lib.i8mp_quantize_rowwise(_ptr(x), R, C, _ld(x), _ptr(q), _ld(q), _ptr(scale),
                                       _ROUNDING[rounding], seed, offset, _stream(dev))
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
    _mat(x, "x", torch.bfloat16)
    R, C = x.shape
    if q is not None:
        _mat(q, "q", torch.int8, (R, C))
    if scale is not None:
        _vec(scale, "scale", R)
    if colmax is not None:
        _vec(colmax, "colmax", C)
    if workspace is not None:
        _workspace(workspace)
    dev = _device(x, q, scale, colmax, workspace)
    q = _empty_2d(R, C, torch.int8, dev) if q is None else q
    scale = torch.empty(R, dtype=torch.float32, device=dev) if scale is None else scale
    colmax = torch.empty(C, dtype=torch.float32, device=dev) if colmax is None else colmax
    need = rowwise_colmax_workspace_bytes(R, C)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = lib.i8mp_quantize_rowwise_colmax(_ptr(x), R, C, _ld(x), _ptr(q), _ld(q), _ptr(scale),
                                              _ptr(colmax), _ROUNDING[rounding], seed, offset,
                                              _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "i8mp_quantize_rowwise_colmax")
    return q, scale, colmax


def quantize_colwise_given_colmax(x: torch.Tensor, colmax: torch.Tensor, rounding="rne",
                                  seed: int = 0, offset: int = 0, q: torch.Tensor | None = None,
                                  scale: torch.Tensor | None = None):
    """Column-wise quantization with known column maxima (one pass):
    (int8 q [R, C] in x's layout, fp32 scale [C])."""
    _mat(x, "x", torch.bfloat16)
    R, C = x.shape
    _vec(colmax, "colmax", C)
    if q is not None:
        _mat(q, "q", torch.int8, (R, C))
    if scale is not None:
        _vec(scale, "scale", C)
    dev = _device(x, colmax, q, scale)
    q = _empty_2d(R, C, torch.int8, dev) if q is None else q
    scale = torch.empty(C, dtype=torch.float32, device=dev) if scale is None else scale
    with torch.cuda.device(dev):
        st = lib.i8mp_quantize_colwise_given_colmax(_ptr(x), R, C, _ld(x), _ptr(colmax), _ptr(q),
                                                    _ld(q), _ptr(scale), _ROUNDING[rounding], seed,
                                                    offset, _stream(dev))
    _check(st, "i8mp_quantize_colwise_given_colmax")
    return q, scale


def colwise_workspace_bytes(rows: int, cols: int) -> int:
    return lib.i8mp_quantize_colwise_workspace_bytes(rows, cols)


def quantize_colwise(x: torch.Tensor, rounding="rne", seed: int = 0, offset: int = 0,
                     q: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None):
    """Column-wise dynamic INT8 quantization -> (int8 q [R, C] in x's layout, fp32 scale [C])."""
    _mat(x, "x", torch.bfloat16)
    R, C = x.shape
    if q is not None:
        _mat(q, "q", torch.int8, (R, C))
    if scale is not None:
        _vec(scale, "scale", C)
    if workspace is not None:
        _workspace(workspace)
    dev = _device(x, q, scale, workspace)
    q = _empty_2d(R, C, torch.int8, dev) if q is None else q
    scale = torch.empty(C, dtype=torch.float32, device=dev) if scale is None else scale
    need = colwise_workspace_bytes(R, C)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = lib.i8mp_quantize_colwise(_ptr(x), R, C, _ld(x), _ptr(q), _ld(q), _ptr(scale),
                                       _ROUNDING[rounding], seed, offset, _ptr(workspace),
                                       workspace.numel(), _stream(dev))
    _check(st, "i8mp_quantize_colwise")
    return q, scale


def quantize_colwise_noalloc(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor,
                             rounding="rne", seed: int = 0, offset: int = 0):
    """quantize_colwise into caller-given q (int8 [R, C]) and scale (fp32 [C])
    with no allocation at all: the library's static per-GPU scratch holds the
    column maxima (STATIC_SCRATCH_BYTES; larger problems raise).  Calls that
    overlap on one GPU share that scratch and race."""
    _mat(x, "x", torch.bfloat16)
    R, C = x.shape
    _mat(q, "q", torch.int8, (R, C))
    _vec(scale, "scale", C)
    dev = _device(x, q, scale)
    with torch.cuda.device(dev):
        st = lib.i8mp_quantize_colwise_noalloc(_ptr(x), R, C, _ld(x), _ptr(q), _ld(q), _ptr(scale),
                                               _ROUNDING[rounding], seed, offset, _stream(dev))
    _check(st, "i8mp_quantize_colwise_noalloc")
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


def _mm_args(layout, A, B, code_dtype, scale_a=None, scale_b=None, out=None, out_dtype=None):
    """Checks of a GEMM's operands (codes of `code_dtype` in `layout`), its
    scales and its output; returns (layout, M, N, K, device)."""
    if layout not in _LAYOUTS:
        raise ValueError(f"layout must be 'NT', 'NN' or 'TN', got {layout!r}")
    layout = _LAYOUTS[layout]
    _mat(A, "A", code_dtype)
    _mat(B, "B", code_dtype)
    M, N, K = _mnk(layout, A, B)
    if out_dtype is torch.bfloat16:
        _vec(scale_a, "scale_a", M)
        _vec(scale_b, "scale_b", N)
    if out is not None:
        _mat(out, "out", out_dtype, (M, N))
    return layout, M, N, K, _device(A, B, scale_a, scale_b, out)


def int8_scaled_mm(layout, A: torch.Tensor, scale_a: torch.Tensor, B: torch.Tensor,
                   scale_b: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 C[M,N] = bf16(((float)(A(m,:) . B(:,n)) * scale_a[m]) * scale_b[n]).

    layout: "NT" (A [M,K], B [N,K]), "NN" (A [M,K], B [K,N]) or "TN" (A [K,M], B [K,N])."""
    layout, M, N, K, dev = _mm_args(layout, A, B, torch.int8, scale_a, scale_b, out, torch.bfloat16)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if out is None else out
    with torch.cuda.device(dev):
        st = lib.i8mp_int8_scaled_mm(layout, M, N, K, _ptr(A), _ld(A), _ptr(scale_a), _ptr(B),
                                     _ld(B), _ptr(scale_b), _ptr(out), _ld(out), _stream(dev))
    _check(st, "i8mp_int8_scaled_mm")
    return out


def int8_mm_i32(layout, A: torch.Tensor, B: torch.Tensor,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """int32 C[M,N] = A(m,:) . B(:,n) (same layouts as int8_scaled_mm)."""
    layout, M, N, K, dev = _mm_args(layout, A, B, torch.int8, out=out, out_dtype=torch.int32)
    out = torch.empty((M, N), dtype=torch.int32, device=dev) if out is None else out
    with torch.cuda.device(dev):
        st = lib.i8mp_int8_mm_i32(layout, M, N, K, _ptr(A), _ld(A), _ptr(B), _ld(B), _ptr(out),
                                  _ld(out), _stream(dev))
    _check(st, "i8mp_int8_mm_i32")
    return out


def philox4x32_10(seed: int, offset: int, n_blocks: int, device="cuda") -> torch.Tensor:
    """uint32 words (returned as int32) [4 * n_blocks] of Philox4x32-10 blocks offset.."""
    if n_blocks < 0:
        raise ValueError(f"n_blocks must be >= 0, got {n_blocks}")
    out = torch.empty(4 * n_blocks, dtype=torch.int32, device=device)
    dev = _device(out)
    with torch.cuda.device(dev):
        st = lib.i8mp_philox4x32_10(seed, offset, n_blocks, _ptr(out), _stream(dev))
    _check(st, "i8mp_philox4x32_10")
    return out


MFMA_PROBE_SINK_INTS = 256 * 512


def mfma_rate_probe(codes: torch.Tensor, rounds: int, sink: torch.Tensor | None = None) -> torch.Tensor:
    """Launch the matrix-core throughput probe (rounds x 2^32 integer operations
    on fragments taken from ``codes``, int8, at least 24 KiB, contiguous) on the
    current stream; returns the int32 sink.  Time it with events around the call."""
    _tensor(codes, "codes", torch.int8)
    if not codes.is_contiguous() or codes.numel() < 24 * 1024:
        raise ValueError("codes: contiguous int8 tensor of at least 24 KiB expected")
    if sink is None:
        sink = torch.empty(MFMA_PROBE_SINK_INTS, dtype=torch.int32, device=codes.device)
    _vec(sink, "sink", MFMA_PROBE_SINK_INTS, torch.int32)
    dev = _device(codes, sink)
    with torch.cuda.device(dev):
        st = lib.i8mp_mfma_rate_probe(_ptr(codes), codes.numel(), rounds, _ptr(sink), _stream(dev))
    _check(st, "i8mp_mfma_rate_probe")
    return sink


# --------------------------------------------------------------------------- linear layer


def linear_workspace_bytes(M: int, N: int, K: int, backward: bool) -> int:
    return lib.i8mp_linear_workspace_bytes(M, N, K, int(backward))


def _opts(rounding, seed, offset):
    return _Opts(_ROUNDING[rounding], seed & (2**64 - 1), offset & (2**64 - 1))


def _fwd_args(X, W, out, workspace):
    """Checks of a forward chain's dense bf16 operands: X [M, K], W [N, K],
    out [M, N]; returns (M, N, K, device)."""
    _mat(X, "X", torch.bfloat16, dense=True)
    M, K = X.shape
    _mat(W, "W", torch.bfloat16, dense=True)
    if W.shape[1] != K:
        raise ValueError(f"W: {K} columns expected (X is {tuple(X.shape)}), got {tuple(W.shape)}")
    N = W.shape[0]
    if out is not None:
        _mat(out, "out", torch.bfloat16, (M, N), dense=True)
    if workspace is not None:
        _workspace(workspace)
    return M, N, K, _device(X, W, out, workspace)


def _bwd_args(dY, X, W, dX, dW, workspace, colmax_x=None, colmax_w=None):
    """Checks of a backward chain's dense bf16 tensors: dY [M, N], X [M, K],
    W [N, K], dX [M, K], dW [N, K], colmax_x / colmax_w fp32 [K]; returns
    (M, N, K, device)."""
    _mat(dY, "dY", torch.bfloat16, dense=True)
    M, N = dY.shape
    _mat(W, "W", torch.bfloat16, dense=True)
    if W.shape[0] != N:
        raise ValueError(f"W: {N} rows expected (dY is {tuple(dY.shape)}), got {tuple(W.shape)}")
    K = W.shape[1]
    _mat(X, "X", torch.bfloat16, (M, K), dense=True)
    if dX is not None:
        _mat(dX, "dX", torch.bfloat16, (M, K), dense=True)
    if dW is not None:
        _mat(dW, "dW", torch.bfloat16, (N, K), dense=True)
    if colmax_x is not None:
        _vec(colmax_x, "colmax_x", K)
    if colmax_w is not None:
        _vec(colmax_w, "colmax_w", K)
    if workspace is not None:
        _workspace(workspace)
    return M, N, K, _device(dY, X, W, dX, dW, workspace, colmax_x, colmax_w)


def linear_fwd(X: torch.Tensor, W: torch.Tensor, rounding="rne", seed: int = 0, offset: int = 0,
               out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Y = X @ W.T with both operands quantized row-wise over K (dense bf16 tensors)."""
    M, N, K, dev = _fwd_args(X, W, out, workspace)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if out is None else out
    need = linear_workspace_bytes(M, N, K, False)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    o = _opts(rounding, seed, offset)
    with torch.cuda.device(dev):
        st = lib.i8mp_linear_fwd(_ptr(X), _ptr(W), _ptr(Y), M, N, K, ctypes.byref(o),
                                 _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "i8mp_linear_fwd")
    return Y


def linear_fwd_colmax(X: torch.Tensor, W: torch.Tensor, rounding="rne", seed: int = 0,
                      offset: int = 0, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None):
    """linear_fwd that also returns the column maxima of X and W (fp32 [K]
    each) for linear_bwd: (Y, colmax_x, colmax_w)."""
    M, N, K, dev = _fwd_args(X, W, out, workspace)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if out is None else out
    cx = torch.empty(K, dtype=torch.float32, device=dev)
    cw = torch.empty(K, dtype=torch.float32, device=dev)
    need = linear_workspace_bytes(M, N, K, False)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    o = _opts(rounding, seed, offset)
    with torch.cuda.device(dev):
        st = lib.i8mp_linear_fwd_colmax(_ptr(X), _ptr(W), _ptr(Y), M, N, K, ctypes.byref(o),
                                        _ptr(cx), _ptr(cw), _ptr(workspace), workspace.numel(),
                                        _stream(dev))
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
    M, N, K, dev = _bwd_args(dY, X, W, dX, dW, workspace, colmax_x, colmax_w)
    if want_dx and dX is None:
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    if want_dw and dW is None:
        dW = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    need = linear_workspace_bytes(M, N, K, True)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    o = _opts(rounding, seed, offset)
    with torch.cuda.device(dev):
        st = lib.i8mp_linear_bwd_colmax(_ptr(dY), _ptr(X), _ptr(W), _ptr(dX if want_dx else None),
                                        _ptr(dW if want_dw else None), M, N, K, ctypes.byref(o),
                                        _ptr(colmax_x), _ptr(colmax_w), _ptr(workspace),
                                        workspace.numel(), _stream(dev))
    _check(st, "i8mp_linear_bwd_colmax")
    return (dX if want_dx else None), (dW if want_dw else None)


# --------------------------------------------------------------------------- FP8 (E4M3) variant


def quantize_rowwise_fp8(x: torch.Tensor, q: torch.Tensor | None = None,
                         scale: torch.Tensor | None = None):
    """Row-wise FP8 quantization of bf16 ``x`` [R, C] -> (E4M3 codes as uint8 [R, C],
    fp32 scale [R]); ``codes.view(torch.float8_e4m3fn)`` gives torch's view of them."""
    _mat(x, "x", torch.bfloat16)
    R, C = x.shape
    if q is not None:
        _mat(q, "q", torch.uint8, (R, C))
    if scale is not None:
        _vec(scale, "scale", R)
    dev = _device(x, q, scale)
    q = _empty_2d(R, C, torch.uint8, dev) if q is None else q
    scale = torch.empty(R, dtype=torch.float32, device=dev) if scale is None else scale
    with torch.cuda.device(dev):
        st = lib.i8mp_quantize_rowwise_fp8(_ptr(x), R, C, _ld(x), _ptr(q), _ld(q), _ptr(scale),
                                           _stream(dev))
    _check(st, "i8mp_quantize_rowwise_fp8")
    return q, scale


def quantize_colwise_fp8(x: torch.Tensor, q: torch.Tensor | None = None,
                         scale: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Column-wise FP8 quantization -> (E4M3 codes uint8 [R, C] in x's layout, fp32 scale [C])."""
    _mat(x, "x", torch.bfloat16)
    R, C = x.shape
    if q is not None:
        _mat(q, "q", torch.uint8, (R, C))
    if scale is not None:
        _vec(scale, "scale", C)
    if workspace is not None:
        _workspace(workspace)
    dev = _device(x, q, scale, workspace)
    q = _empty_2d(R, C, torch.uint8, dev) if q is None else q
    scale = torch.empty(C, dtype=torch.float32, device=dev) if scale is None else scale
    need = colwise_workspace_bytes(R, C)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = lib.i8mp_quantize_colwise_fp8(_ptr(x), R, C, _ld(x), _ptr(q), _ld(q), _ptr(scale),
                                           _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "i8mp_quantize_colwise_fp8")
    return q, scale


def fp8_scaled_mm(layout, A: torch.Tensor, scale_a: torch.Tensor, B: torch.Tensor,
                  scale_b: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 C[M,N] from E4M3 codes (uint8): fp32 sums of the exact products, then
    bf16((sum * scale_a[m]) * scale_b[n]).  Layouts as for int8_scaled_mm; K % 16 == 0."""
    layout, M, N, K, dev = _mm_args(layout, A, B, torch.uint8, scale_a, scale_b, out, torch.bfloat16)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if out is None else out
    with torch.cuda.device(dev):
        st = lib.i8mp_fp8_scaled_mm(layout, M, N, K, _ptr(A), _ld(A), _ptr(scale_a), _ptr(B),
                                    _ld(B), _ptr(scale_b), _ptr(out), _ld(out), _stream(dev))
    _check(st, "i8mp_fp8_scaled_mm")
    return out


def fp8_mm_f32(layout, A: torch.Tensor, B: torch.Tensor,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """float32 C[M,N]: the matrix core's fp32 sums of E4M3 products (same layouts
    as fp8_scaled_mm, no scales)."""
    layout, M, N, K, dev = _mm_args(layout, A, B, torch.uint8, out=out, out_dtype=torch.float32)
    out = torch.empty((M, N), dtype=torch.float32, device=dev) if out is None else out
    with torch.cuda.device(dev):
        st = lib.i8mp_fp8_mm_f32(layout, M, N, K, _ptr(A), _ld(A), _ptr(B), _ld(B), _ptr(out),
                                 _ld(out), _stream(dev))
    _check(st, "i8mp_fp8_mm_f32")
    return out


def linear_fwd_fp8(X: torch.Tensor, W: torch.Tensor, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None):
    """Y = X @ W.T with both operands quantized row-wise to FP8 (E4M3) over K."""
    M, N, K, dev = _fwd_args(X, W, out, workspace)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if out is None else out
    need = linear_workspace_bytes(M, N, K, False)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = lib.i8mp_linear_fwd_fp8(_ptr(X), _ptr(W), _ptr(Y), M, N, K, _ptr(workspace),
                                     workspace.numel(), _stream(dev))
    _check(st, "i8mp_linear_fwd_fp8")
    return Y


def linear_fwd_fp8_colmax(X: torch.Tensor, W: torch.Tensor, out: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None):
    """linear_fwd_fp8 that also returns the column maxima of X and W (fp32 [K]
    each) for linear_bwd_fp8: (Y, colmax_x, colmax_w)."""
    M, N, K, dev = _fwd_args(X, W, out, workspace)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if out is None else out
    cx = torch.empty(K, dtype=torch.float32, device=dev)
    cw = torch.empty(K, dtype=torch.float32, device=dev)
    need = linear_workspace_bytes(M, N, K, False)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = lib.i8mp_linear_fwd_fp8_colmax(_ptr(X), _ptr(W), _ptr(Y), M, N, K, _ptr(cx), _ptr(cw),
                                            _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "i8mp_linear_fwd_fp8_colmax")
    return Y, cx, cw


def linear_bwd_fp8(dY: torch.Tensor, X: torch.Tensor, W: torch.Tensor, want_dx: bool = True,
                   want_dw: bool = True, workspace: torch.Tensor | None = None,
                   dX: torch.Tensor | None = None, dW: torch.Tensor | None = None,
                   colmax_x: torch.Tensor | None = None, colmax_w: torch.Tensor | None = None):
    """(dX = dY @ W, dW = dY.T @ X) with FP8 (E4M3) operands, each quantized along
    its own contraction.  colmax_x / colmax_w: the column maxima from
    linear_fwd_fp8_colmax (optional; the results are the same)."""
    M, N, K, dev = _bwd_args(dY, X, W, dX, dW, workspace, colmax_x, colmax_w)
    if want_dx and dX is None:
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    if want_dw and dW is None:
        dW = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    need = linear_workspace_bytes(M, N, K, True)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = lib.i8mp_linear_bwd_fp8_colmax(_ptr(dY), _ptr(X), _ptr(W), _ptr(dX if want_dx else None),
                                            _ptr(dW if want_dw else None), M, N, K, _ptr(colmax_x),
                                            _ptr(colmax_w), _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "i8mp_linear_bwd_fp8_colmax")
    return (dX if want_dx else None), (dW if want_dw else None)
