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
          (600, 14336), (3, 16385), (2, 30001), (300, 16392), (1030, 20001)]


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
