"""GPU parity of the column-maxima path, element by element against the oracle.

* Row-wise quantization that also reports column maxima: codes and scales as
  the oracle's row-wise pass, maxima as the oracle's column maxima, over
  widths that take every kernel variant (one chunk per lane up to 28, the
  4-wave variant above 6144 columns, and the banded two-pass path past 14336:
  one band and many, a partial last 4096-column segment, odd widths),
  padded leading dimensions, canary bytes after every output row.
* Column-wise quantization given those maxima: as the oracle's column-wise
  pass.
* The linear chains that hand X's and W's maxima from forward to backward:
  outputs as the oracle's chains, maxima as the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import (bits_to_bf16, canary_intact, padded, padded_copy, round_up,
                            special_rows_bf16, tensor_bits)
from workloads import LinearShape, linear_inputs

pytestmark = pytest.mark.gpu

i8 = pytest.importorskip("int8_mixed_precision_rowwise_amd")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

ROUNDINGS = [("rne", oracle.RNE), ("sr", oracle.SR)]
SHAPES = [(1, 1), (3, 17), (9, 255), (40, 513), (257, 2048), (100, 4096), (5000, 512),
          (33, 5000), (17, 6144), (21, 6152), (3000, 6200), (12, 8192), (9, 14336),
          (600, 14336), (3, 16385), (2, 30001), (300, 16392), (1030, 20001),
          (33, 7001), (70, 8191), (20, 9000), (64, 12290), (40, 5632)]


def same_f32(t: torch.Tensor, want: np.ndarray, what: str):
    got = t.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, want.view(np.uint32)), what


@pytest.mark.parametrize("rounding,rc", ROUNDINGS)
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_rowwise_colmax_then_colwise_given(rounding, rc, rows, cols):
    rng = np.random.default_rng(rows * 31337 + cols)
    xb = special_rows_bf16(rng, rows, cols)
    x = padded_copy(bits_to_bf16(xb), round_up(cols, 8) + 8)
    qs, q = padded(rows, cols, round_up(cols, 16) + 16, torch.int8)
    seed, off = 91, 2**41 + 5
    _, s, cm = i8.quantize_rowwise_colmax(x, rounding, seed, off, q=q)
    torch.cuda.synchronize()
    qo, so = oracle.quantize_rowwise(xb, rc, seed, off)
    cmo = oracle.col_absmax(xb)
    same_f32(s, so, "row scales")
    assert np.array_equal(q.cpu().numpy(), qo), "row codes"
    assert canary_intact(qs, cols)
    same_f32(cm, cmo, "column maxima")
    qs2, q2 = padded(rows, cols, round_up(cols, 16) + 16, torch.int8)
    _, s2 = i8.quantize_colwise_given_colmax(x, cm, rounding, seed, off + 1, q=q2)
    torch.cuda.synchronize()
    qco, sco = oracle.quantize_colwise(xb, rc, seed, off + 1)
    same_f32(s2, sco, "column scales")
    assert np.array_equal(q2.cpu().numpy(), qco), "column codes"
    assert canary_intact(qs2, cols)


def test_no_rows():
    x = torch.zeros((0, 40), dtype=torch.bfloat16, device="cuda")
    cm = torch.full((40,), 3.0, device="cuda")
    _, s, cm = i8.quantize_rowwise_colmax(x, colmax=cm)
    assert s.shape == (0,) and (cm.cpu() == 0).all()
    sc = torch.full((40,), 3.0, device="cuda")
    i8.quantize_colwise_given_colmax(x, cm, scale=sc)
    assert (sc.cpu() == 0).all()


@pytest.mark.parametrize("rounding,rc", ROUNDINGS)
@pytest.mark.parametrize("M,N,K", [(17, 24, 40), (300, 520, 264), (1000, 72, 600), (64, 6200, 128)])
def test_linear_chains_with_column_maxima(rounding, rc, M, N, K):
    t = linear_inputs(LinearShape("colmax_chain", M, N, K), seed=3, device="cuda")
    X, W, dY = t["X"], t["W"], t["dY"]
    Xb, Wb, dYb = tensor_bits(X), tensor_bits(W), tensor_bits(dY)
    seed, off = 13, 7 << 44
    Y, cx, cw = i8.linear_fwd_colmax(X, W, rounding, seed, off)
    assert np.array_equal(tensor_bits(Y), oracle.linear_fwd(Xb, Wb, rc, seed, off)), "Y"
    same_f32(cx, oracle.col_absmax(Xb), "colmax X")
    same_f32(cw, oracle.col_absmax(Wb), "colmax W")
    dXo, dWo = oracle.linear_bwd(dYb, Xb, Wb, rc, seed, off)
    for want_dx, want_dw in ((True, True), (True, False), (False, True)):
        dX, dW = i8.linear_bwd(dY, X, W, rounding, seed, off, want_dx=want_dx, want_dw=want_dw,
                               colmax_x=cx, colmax_w=cw)
        if want_dx:
            assert np.array_equal(tensor_bits(dX), dXo), f"dX ({want_dx}, {want_dw})"
        if want_dw:
            assert np.array_equal(tensor_bits(dW), dWo), f"dW ({want_dx}, {want_dw})"


# Rows of exactly 512 * NV elements take the row passes without range checks
# (the FULL kernels the 4096^3 step and the Llama-1B K = 2048 layers run, in
# the paired launch of X's and W's rows); K in {1024, 2048, 4096, 8192}.  A
# 4096-wide dY also takes them in the backward (dY's row pass, and W's and
# dY's column passes over whole 512-column tiles).  Every output against the
# oracle, both roundings.
@pytest.mark.parametrize("rounding,rc", ROUNDINGS)
@pytest.mark.parametrize("M,N,K", [(300, 264, 1024), (300, 264, 2048), (300, 264, 4096),
                                   (300, 264, 8192), (136, 4096, 1024)])
def test_linear_chains_with_maxima_full_width_rows(rounding, rc, M, N, K):
    t = linear_inputs(LinearShape("full_rows", M, N, K), seed=K + N, device="cuda")
    X, W, dY = t["X"], t["W"], t["dY"]
    Xb, Wb, dYb = tensor_bits(X), tensor_bits(W), tensor_bits(dY)
    seed, off = 77, 3 << 44
    Y, cx, cw = i8.linear_fwd_colmax(X, W, rounding, seed, off)
    dX, dW = i8.linear_bwd(dY, X, W, rounding, seed, off, colmax_x=cx, colmax_w=cw)
    torch.cuda.synchronize()
    assert np.array_equal(tensor_bits(Y), oracle.linear_fwd(Xb, Wb, rc, seed, off)), "Y"
    same_f32(cx, oracle.col_absmax(Xb), "colmax X")
    same_f32(cw, oracle.col_absmax(Wb), "colmax W")
    dXo, dWo = oracle.linear_bwd(dYb, Xb, Wb, rc, seed, off)
    assert np.array_equal(tensor_bits(dX), dXo), "dX"
    assert np.array_equal(tensor_bits(dW), dWo), "dW"


# The grad-input chain runs dY's row pass and W's column pass in one launch
# when dY's rows take 4 or 8 chunks per lane (N in 1025..4096; the chains
# take widths in whole 16-byte chunks): ragged and whole widths of both
# kinds, W wider than one 4096-column group with a ragged last tile, a single
# token.  Every output against the oracle.
@pytest.mark.parametrize("rounding,rc", ROUNDINGS)
@pytest.mark.parametrize("M,N,K", [(300, 1504, 1000), (129, 2048, 4200), (33, 3000, 704), (200, 4088, 1104),
                                   (1, 2504, 64), (64, 1032, 512), (40, 1032, 4104)])
def test_linear_bwd_row_and_column_pass_in_one_launch(rounding, rc, M, N, K):
    t = linear_inputs(LinearShape("mixed_pair", M, N, K), seed=M + N + K, device="cuda")
    X, W, dY = t["X"], t["W"], t["dY"]
    Xb, Wb, dYb = tensor_bits(X), tensor_bits(W), tensor_bits(dY)
    seed, off = 91, 5 << 44
    _, cx, cw = i8.linear_fwd_colmax(X, W, rounding, seed, off)
    dX, dW = i8.linear_bwd(dY, X, W, rounding, seed, off, colmax_x=cx, colmax_w=cw)
    torch.cuda.synchronize()
    dXo, dWo = oracle.linear_bwd(dYb, Xb, Wb, rc, seed, off)
    assert np.array_equal(tensor_bits(dX), dXo), "dX"
    assert np.array_equal(tensor_bits(dW), dWo), "dW"


def test_chains_with_maxima_and_an_empty_contraction():
    """K = 0 (forward) and N = 0 (grad-input) with column-maxima pointers given
    through the C ABI: the row scales of the empty rows are 0 and the outputs
    +0, whatever the workspace held (filled with NaN bytes first)."""
    import ctypes
    L = i8.lib
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    M, N = 40, 24
    o = i8._Opts(0, 0, 0)
    cx = torch.full((4,), 7.0, device="cuda")
    cw = torch.full((4,), 7.0, device="cuda")
    ws = torch.full((i8.linear_workspace_bytes(M, N, 0, False) + 256,), 0xFF, dtype=torch.uint8,
                    device="cuda")
    for a, b in ((cx, cw), (cx, None), (None, cw)):  # the paired row pass and the single ones
        ws.fill_(0xFF)
        Y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
        st = L.i8mp_linear_fwd_colmax(None, None, P(Y), M, N, 0, ctypes.byref(o),
                                      P(a) if a is not None else None, P(b) if b is not None else None,
                                      P(ws), ws.numel(), sp)
        torch.cuda.synchronize()
        assert st == 0
        assert (tensor_bits(Y) == 0).all(), "Y must be +0"
    # grad-input with an empty contraction (N = 0): dX = dY @ W = 0
    K = 48
    X = torch.ones((M, K), dtype=torch.bfloat16, device="cuda")
    W = torch.ones((0, K), dtype=torch.bfloat16, device="cuda")
    dX = torch.full((M, K), 3.0, dtype=torch.bfloat16, device="cuda")
    cx = torch.ones(K, device="cuda")
    cw = torch.zeros(K, device="cuda")
    wsb = torch.full((i8.linear_workspace_bytes(M, 0, K, True) + 256,), 0xFF, dtype=torch.uint8,
                     device="cuda")
    st = L.i8mp_linear_bwd_colmax(None, P(X), None, P(dX), None, M, 0, K, ctypes.byref(o), P(cx),
                                  P(cw), P(wsb), wsb.numel(), sp)
    torch.cuda.synchronize()
    assert st == 0
    assert (tensor_bits(dX) == 0).all(), "dX must be +0"
