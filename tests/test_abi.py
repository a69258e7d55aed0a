"""The C-ABI library on the host (no GPU needed): it loads, it exports every
symbol its header declares, the host-side query functions agree with the
documented layout, and every validation error is reported before any HIP
call is made (so a rejected call launches nothing)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "i8mp.h")

i8 = pytest.importorskip("int8_mixed_precision_rowwise_amd")
L = i8.lib

EINVAL, ERANGE, EDEVICE, EWORKSPACE, ESCRATCH = 1, 2, 3, 5, 6
A16 = 0x10000  # fake, 16-byte aligned device addresses: validation never dereferences them


def fake(n):
    return ctypes.c_void_p(A16 * (n + 1))


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(i8mp_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(i8.EXPORTED_SYMBOLS)


def test_abi_version_and_status_strings():
    assert L.i8mp_abi_version() == 4
    for s in range(7):
        assert L.i8mp_status_str(s)
    assert b"133144" in L.i8mp_status_str(ERANGE)


def test_quantize_rowwise_validation():
    f = L.i8mp_quantize_rowwise
    x, q, s = fake(1), fake(3), fake(5)
    # bad rounding mode, negative sizes, null pointers, ld too small, misaligned
    assert f(x, 4, 8, 8, q, 16, s, 7, 0, 0, None) == EINVAL
    assert f(x, -1, 8, 8, q, 16, s, 0, 0, 0, None) == EINVAL
    assert f(None, 4, 8, 8, q, 16, s, 0, 0, 0, None) == EINVAL
    assert f(x, 4, 8, 4, q, 16, s, 0, 0, 0, None) == EINVAL
    assert f(x, 4, 8, 12, q, 16, s, 0, 0, 0, None) == EINVAL  # 12 bf16 = 24 bytes, not 16-aligned
    assert f(ctypes.c_void_p(A16 + 8), 4, 8, 8, q, 16, s, 0, 0, 0, None) == EINVAL
    assert f(x, 4, 8, 8, q, 8, s, 0, 0, 0, None) == EINVAL  # int8 ld 8 is not 16 bytes
    assert f(x, 4, 8, 8, q, 16, ctypes.c_void_p(A16 * 5 + 2), 0, 0, 0, None) == EINVAL
    # overlapping output and input
    assert f(x, 4, 8, 8, ctypes.c_void_p(A16 * 2 + 16), 16, s, 0, 0, 0, None) == EINVAL
    # nothing to do: no device needed
    assert f(None, 0, 8, 8, None, 16, None, 0, 0, 0, None) == 0


def test_valid_calls_need_a_gfx950_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    x, q, s = fake(1), fake(3), fake(5)
    assert L.i8mp_quantize_rowwise(x, 4, 8, 8, q, 16, s, 0, 0, 0, None) == EDEVICE
    assert L.i8mp_philox4x32_10(0, 0, 4, fake(7), None) == EDEVICE
    assert L.i8mp_int8_mm_i32(0, 4, 4, 16, fake(1), 16, fake(3), 16, fake(5), 4, None) == EDEVICE


def test_gemm_validation():
    f = L.i8mp_int8_scaled_mm
    A, B, C, sa, sb = fake(1), fake(3), fake(5), fake(7), fake(9)
    assert f(3, 4, 4, 16, A, 16, sa, B, 16, sb, C, 4, None) == EINVAL  # layout
    assert f(0, 4, 4, 133145, A, 133152, sa, B, 133152, sb, C, 4, None) == ERANGE
    assert f(0, 4, 4, 16, A, 8, sa, B, 16, sb, C, 4, None) == EINVAL  # lda < K
    assert f(0, 4, 4, 16, A, 16, sa, B, 16, sb, C, 3, None) == EINVAL  # ldc < N
    assert f(0, 4, 4, 16, A, 16, None, B, 16, sb, C, 4, None) == EINVAL  # missing scale
    assert f(0, 4, 4, 16, A, 16, sa, B, 16, sb, ctypes.c_void_p(A16 * 2 + 1), 4, None) == EINVAL
    assert f(0, 4, 4, 16, A, 16, sa, B, 16, sb, ctypes.c_void_p(A16 * 2 + 8), 4, None) == EINVAL  # C overlaps A
    # TN: A is K x M, lda >= M
    assert f(2, 32, 4, 16, A, 16, sa, B, 16, sb, C, 4, None) == EINVAL
    # empty output: OK without a device
    assert f(0, 0, 4, 16, None, 16, None, None, 16, None, None, 4, None) == 0
    g = L.i8mp_int8_mm_i32
    assert g(1, 4, 4, 16, A, 16, B, 8, C, 4, None) == EINVAL  # NN: ldb >= N and 16-aligned


def test_colwise_workspace_rules():
    f = L.i8mp_quantize_colwise
    need = L.i8mp_quantize_colwise_workspace_bytes(4096, 4096)
    assert need > 0 and need % 256 == 0
    x, q, s, w = fake(1), fake(1 << 12), fake(1 << 13), fake(1 << 14)
    assert f(x, 64, 64, 64, q, 64, s, 0, 0, 0, None, 0, None) == EWORKSPACE
    small = L.i8mp_quantize_colwise_workspace_bytes(64, 64)
    assert f(x, 64, 64, 64, q, 64, s, 0, 0, 0, w, small - 1, None) == EWORKSPACE
    assert f(x, 64, 64, 64, q, 64, s, 0, 0, 0, ctypes.c_void_p(A16 * (1 << 14) + 16), small, None) == EWORKSPACE


def test_linear_validation_and_workspace():
    fwd, bwd = L.i8mp_linear_fwd, L.i8mp_linear_bwd
    o = i8._Opts(0, 0, 0)
    bad = i8._Opts(5, 0, 0)
    X, W, Y, ws = fake(1), fake(1 << 12), fake(1 << 13), fake(1 << 14)
    nf = L.i8mp_linear_workspace_bytes(64, 32, 48, 0)
    nb = L.i8mp_linear_workspace_bytes(64, 32, 48, 1)
    assert nf > 0 and nb > nf
    assert fwd(X, W, Y, 64, 32, 48, ctypes.byref(bad), ws, nf, None) == EINVAL
    assert fwd(X, W, Y, 64, 32, 48, None, ws, nf, None) == EINVAL
    assert fwd(X, W, Y, 64, 32, 133145, ctypes.byref(o), ws, nf, None) == ERANGE
    assert fwd(X, W, Y, 64, 32, 44, ctypes.byref(o), ws, nf, None) == EINVAL  # K*2 not 16-aligned
    assert fwd(X, W, Y, 64, 32, 48, ctypes.byref(o), ws, nf - 1, None) == EWORKSPACE
    dY, dX, dW = fake(1 << 15), fake(1 << 16), fake(1 << 17)
    assert bwd(dY, X, W, dX, dW, 133145, 32, 48, ctypes.byref(o), ws, nb, None) == ERANGE
    assert bwd(dY, X, W, dX, None, 133145, 32, 48, ctypes.byref(o), ws, nb, None) != ERANGE
    assert bwd(dY, X, W, dX, dX, 64, 32, 48, ctypes.byref(o), ws, nb, None) == EINVAL
    assert bwd(dY, X, W, None, None, 64, 32, 48, ctypes.byref(o), None, 0, None) == 0


def _split_planes_bytes(M, N, K):
    """Bytes of int32 partial planes the forward chain's NT GEMM (both operands
    K-contiguous, rows padded to 16 bytes) takes: when the output has fewer than
    128 tiles of 256 x 256 and the contraction is a multiple of 16, it splits
    into min(256 // tiles, K // 1024) ranges of whole 64-deep slabs, provided
    that makes at least min(256, 4 * tiles) workgroups."""
    tiles = -(-M // 256) * -(-N // 256)
    if tiles >= 128 or K % 16 or K == 0:
        return 0
    s = min(256 // tiles, K // 1024)
    if s < 2:
        return 0
    kc = -(-K // s)
    kc = -(-kc // 64) * 64
    s = -(-K // kc)
    if s < 2 or s * tiles < min(256, 4 * tiles):  # no more workgroups than 128 x 128 tiles
        return 0
    return s * M * (-(-N // 4) * 4) * 4


@pytest.mark.parametrize("M,N,K", [(2048, 256, 32768), (300, 264, 4096), (4096, 4096, 4096),
                                   (2048, 2048, 2048), (1024, 1024, 8192), (256, 512, 512),
                                   (64, 32, 48), (1000, 8, 4096)])
def test_linear_workspace_holds_contraction_split_planes(M, N, K):
    """The forward chain's workspace: int8 codes and scales of X and W, the
    two row passes' slab maxima (one region each: the passes share a launch),
    and the split GEMM's int32 partial planes, each region 256-byte aligned."""
    up = lambda n: -(-n // 256) * 256  # noqa: E731
    kp = -(-K // 16) * 16
    part = (L.i8mp_quantize_rowwise_colmax_workspace_bytes(M, K)
            + L.i8mp_quantize_rowwise_colmax_workspace_bytes(N, K))
    want = up(M * kp) + up(N * kp) + up(4 * M) + up(4 * N) + part + up(_split_planes_bytes(M, N, K))
    assert L.i8mp_linear_workspace_bytes(M, N, K, 0) == want
    if (M, N, K) == (2048, 256, 32768):  # 8 tiles: 32 ranges of 1024
        assert _split_planes_bytes(M, N, K) == 32 * 2048 * 256 * 4
    if (M, N, K) in ((4096, 4096, 4096), (2048, 2048, 2048)):  # 256 tiles; 2 copies of 64
        assert _split_planes_bytes(M, N, K) == 0
    if (M, N, K) == (1024, 1024, 8192):  # 16 tiles: 8 ranges of 1024
        assert _split_planes_bytes(M, N, K) == 8 * 1024 * 1024 * 4


def _split_bytes(M, N, K, a_kmajor, b_kmajor, lda, ldb):
    """Partial-plane bytes of a chain GEMM with output M x N and contraction K
    (the rule of _split_planes_bytes, with the pipelined kernel's conditions:
    K % 16 == 0, operand tiles under 2^31 bytes, and an output extent that is a
    multiple of 4 along each operand read down its rows)."""
    tiles = -(-M // 256) * -(-N // 256)
    lim = (1 << 31) - 1024
    a_ext = 256 * lda if a_kmajor else K * lda
    b_ext = 256 * ldb if b_kmajor else K * ldb
    mn_ok = (a_kmajor or M % 4 == 0) and (b_kmajor or N % 4 == 0)
    if tiles >= 128 or K == 0 or K % 16 or a_ext >= lim or b_ext >= lim or not mn_ok:
        return 0
    s = min(256 // tiles, K // 1024)
    if s < 2:
        return 0
    kc = -(-K // s)
    kc = -(-kc // 64) * 64
    s = -(-K // kc)
    if s < 2 or s * tiles < min(256, 4 * tiles):
        return 0
    return s * M * (-(-N // 4) * 4) * 4


@pytest.mark.parametrize("M,N,K", [(2048, 256, 32768), (32768, 256, 2048), (300, 4096, 264),
                                   (4112, 200, 296), (4096, 4096, 4096), (1024, 8192, 1024),
                                   (64, 32, 48), (32768, 5632, 2048)])
def test_linear_backward_workspace_layout(M, N, K):
    """The backward chain's workspace: dY's codes (one buffer for its row- and
    column-wise passes), W's and X's codes, the scales, dY's column maxima, the
    largest slab scratch of its quantize passes, and the larger of the
    grad-input (NN) and grad-weight (TN) GEMMs' split planes; 256-byte regions."""
    up = lambda n: -(-n // 256) * 256  # noqa: E731
    kp, np_ = -(-K // 16) * 16, -(-N // 16) * 16
    col = max(L.i8mp_quantize_colwise_workspace_bytes(N, K), L.i8mp_quantize_colwise_workspace_bytes(M, N),
              L.i8mp_quantize_colwise_workspace_bytes(M, K),
              L.i8mp_quantize_rowwise_colmax_workspace_bytes(M, N))
    split = max(_split_bytes(M, K, N, True, False, np_, kp), _split_bytes(N, K, M, False, False, np_, kp))
    want = (up(M * np_) + up(N * kp) + up(M * kp) + up(4 * max(M, N)) + up(4 * K) + up(4 * K)
            + up(4 * N) + col + up(split))
    assert L.i8mp_linear_workspace_bytes(M, N, K, 1) == want
    if (M, N, K) == (32768, 256, 2048):  # grad-weight 256 x 2048 (8 tiles) over 32768 tokens
        assert _split_bytes(N, K, M, False, False, np_, kp) == 32 * 256 * 2048 * 4
    if (M, N, K) == (2048, 256, 32768):  # grad-weight 256 x 32768 has 128 tiles: no split
        assert _split_bytes(N, K, M, False, False, np_, kp) == 0
    if (M, N, K) == (1024, 8192, 1024):  # grad-input: 16 tiles, contraction 8192 in 8 ranges
        assert _split_bytes(M, K, N, True, False, np_, kp) == 8 * 1024 * 1024 * 4


def test_binding_has_no_fallback(monkeypatch, tmp_path):
    """The package refuses to import without its library instead of falling back."""
    import importlib
    import sys
    import int8_mixed_precision_rowwise_amd.build as b
    monkeypatch.setattr(b, "LIB_PATH", str(tmp_path / "missing.so"))
    saved = sys.modules.pop("int8_mixed_precision_rowwise_amd")
    try:
        with pytest.raises(ImportError):
            importlib.import_module("int8_mixed_precision_rowwise_amd")
    finally:
        sys.modules["int8_mixed_precision_rowwise_amd"] = saved


def test_product_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "int8_mixed_precision_rowwise_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in text.lower(), fn


def test_colwise_noalloc_validation():
    """The scratch-free column-wise pass validates like i8mp_quantize_colwise
    and rejects problems whose scratch exceeds the static buffer."""
    f = L.i8mp_quantize_colwise_noalloc
    x, q, s = fake(1), fake(3), fake(5)
    assert f(x, 4, 8, 8, q, 16, s, 7, 0, 0, None) == EINVAL
    assert f(x, 4, 8, 4, q, 16, s, 0, 0, 0, None) == EINVAL
    assert f(None, 4, 0, 8, None, 16, None, 0, 0, 0, None) == 0  # no columns: nothing to do
    cap = i8.STATIC_SCRATCH_BYTES
    big = 1
    while L.i8mp_quantize_colwise_workspace_bytes(4, big) <= cap:
        big *= 2
    assert L.i8mp_quantize_colwise_workspace_bytes(4, big // 2) <= cap
    # rows of `big` columns: x at 2*big bytes per row, q at big
    xb, qb, sb = ctypes.c_void_p(A16 * 1), ctypes.c_void_p(A16 * 1 + 16 * big), ctypes.c_void_p(A16 * 1 + 32 * big)
    assert f(xb, 4, big, big, qb, big, sb, 0, 0, 0, None) == ESCRATCH
    assert b"static" in L.i8mp_status_str(ESCRATCH)


def test_mfma_probe_validation():
    f = L.i8mp_mfma_rate_probe
    codes, sink = fake(1), ctypes.c_void_p(A16 * 100)
    assert f(None, 1 << 20, 4, sink, None) == EINVAL
    assert f(codes, 1000, 4, sink, None) == EINVAL  # fewer than 24 KiB
    assert f(codes, 1 << 20, -1, sink, None) == EINVAL
    assert f(codes, 1 << 20, 4, None, None) == EINVAL
    assert f(codes, 1 << 20, 4, ctypes.c_void_p(A16 * 2), None) == EINVAL  # sink inside codes
