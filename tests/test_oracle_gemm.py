"""Pins of the oracle's integer matmul, scale epilogue and linear chains (CPU only).

"Quantized model training", section "Speed benchmarks > Matmul" names the three
operand layouts (A @ B.T, A @ B, A.T @ B); section "INT8 mixed precision
training" says each of the three GEMMs of a linear layer (forward, grad input,
grad weight) runs as a scaled INT8 matmul after dynamic row-wise quantization;
"Integrate INT8 mixed-precision from torchao 0.7" (gau-nernst's reply on
memory) says the result is scaled back to BF16.

Pins: numpy's int64 matmul (a library routine) for every layout; exact
rational brute force for the epilogue; torch's own fp32 -> bf16 rounding for
the integer special case; the int32 headroom bound; the chain's wiring.
"""
from dataclasses import replace
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import exact_ref
from workloads import bf16_bits, gaussian_bf16, linear_inputs, single_linear

LAYOUT_IDS = ["NT", "NN", "TN"]


def storage_shapes(layout, M, N, K):
    if layout == "NT":
        return (M, K), (N, K)
    if layout == "NN":
        return (M, K), (K, N)
    return (K, M), (K, N)


def logical(layout, A, B):
    """A as [M,K] and B as [K,N] (int64 views) for the layout."""
    A = A.astype(np.int64)
    B = B.astype(np.int64)
    if layout == "NT":
        return A, B.T
    if layout == "NN":
        return A, B
    return A.T, B


@pytest.mark.parametrize("layout", LAYOUT_IDS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (17, 33, 65), (64, 48, 257), (5, 130, 1000)])
def test_mm_i32_matches_numpy_int64(layout, M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    sa, sb = storage_shapes(layout, M, N, K)
    A = rng.integers(-127, 128, size=sa).astype(np.int8)
    B = rng.integers(-127, 128, size=sb).astype(np.int8)
    C = oracle.mm_i32(oracle.LAYOUTS[layout], A, B)
    a, b = logical(layout, A, B)
    assert np.array_equal(C.astype(np.int64), a @ b)


@pytest.mark.parametrize("layout", LAYOUT_IDS)
def test_mm_i32_honours_leading_dimension(layout):
    rng = np.random.default_rng(9)
    M, N, K = 9, 11, 13
    sa, sb = storage_shapes(layout, M, N, K)
    A = rng.integers(-127, 128, size=(sa[0], sa[1] + 5)).astype(np.int8)
    B = rng.integers(-127, 128, size=(sb[0], sb[1] + 3)).astype(np.int8)
    Av, Bv = A[:, : sa[1]], B[:, : sb[1]]
    C = oracle.mm_i32(oracle.LAYOUTS[layout], Av, Bv)
    a, b = logical(layout, np.ascontiguousarray(Av), np.ascontiguousarray(Bv))
    assert np.array_equal(C.astype(np.int64), a @ b)


@pytest.mark.parametrize("layout", LAYOUT_IDS)
def test_scaled_mm_matches_exact_rationals(layout):
    rng = np.random.default_rng(10)
    M, N, K = 5, 6, 8
    shp_a, shp_b = storage_shapes(layout, M, N, K)
    A = rng.integers(-127, 128, size=shp_a).astype(np.int8)
    B = rng.integers(-127, 128, size=shp_b).astype(np.int8)
    sa = (rng.random(M) * 10.0 ** rng.integers(-12, 3, size=M)).astype(np.float32)
    sb = (rng.random(N) * 10.0 ** rng.integers(-12, 3, size=N)).astype(np.float32)
    y = oracle.scaled_mm(oracle.LAYOUTS[layout], A, sa, B, sb)
    a, b = logical(layout, A, B)
    acc = a @ b
    for m in range(M):
        for n in range(N):
            want = exact_ref.epilogue_bits(int(acc[m, n]), Fraction(float(sa[m])), Fraction(float(sb[n])))
            assert int(y[m, n]) == want, (m, n)


def test_epilogue_error_bound():
    """|y - acc*sa*sb| is within half a bf16 ulp plus three binary32 roundings."""
    rng = np.random.default_rng(11)
    M, N, K = 32, 32, 512
    A = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    B = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    sa = (rng.random(M) + 0.5).astype(np.float32) * np.float32(1e-3)
    sb = (rng.random(N) + 0.5).astype(np.float32) * np.float32(1e-2)
    y = oracle.scaled_mm(oracle.NT, A, sa, B, sb)
    yf = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    exact = (A.astype(np.int64) @ B.T.astype(np.int64)) * sa.astype(np.float64)[:, None] * sb.astype(np.float64)[None, :]
    tol = np.abs(exact) * (2.0**-8 + 4 * 2.0**-24)  # bf16 unit roundoff 2^-8
    assert (np.abs(yf - exact) <= tol).all()


def test_scale_one_reduces_to_integer_matmul_rounded_by_torch():
    rng = np.random.default_rng(12)
    A = rng.integers(-127, 128, size=(20, 300)).astype(np.int8)
    B = rng.integers(-127, 128, size=(300, 24)).astype(np.int8)
    y = oracle.scaled_mm(oracle.NN, A, np.ones(20, np.float32), B, np.ones(24, np.float32))
    ref = torch.from_numpy(A.astype(np.int64) @ B.astype(np.int64)).to(torch.float32).to(torch.bfloat16)
    assert np.array_equal(y, ref.view(torch.int16).numpy().view(np.uint16))


def test_int32_headroom_bound():
    # worst case at the LM-head grad-input contraction 128256: 127*127*K fits int32
    K = 128256
    A = np.full((1, K), 127, dtype=np.int8)
    B = np.full((1, K), 127, dtype=np.int8)
    C = oracle.mm_i32(oracle.NT, A, B)
    assert int(C[0, 0]) == 127 * 127 * K == 2068641024
    C = oracle.mm_i32(oracle.NT, A, -B)
    assert int(C[0, 0]) == -2068641024
    # one more than floor((2^31 - 1) / 127^2) = 133144 overflows and is reported
    K = 133145
    A = np.full((1, K), 127, dtype=np.int8)
    with pytest.raises(OverflowError):
        oracle.mm_i32(oracle.NT, A, A.copy())


@pytest.mark.parametrize("layout", LAYOUT_IDS)
def test_scaled_mm_at_agrees_with_full(layout):
    rng = np.random.default_rng(13)
    M, N, K = 40, 36, 100
    shp_a, shp_b = storage_shapes(layout, M, N, K)
    A = rng.integers(-127, 128, size=shp_a).astype(np.int8)
    B = rng.integers(-127, 128, size=shp_b).astype(np.int8)
    sa = rng.random(M).astype(np.float32)
    sb = rng.random(N).astype(np.float32)
    full = oracle.scaled_mm(oracle.LAYOUTS[layout], A, sa, B, sb)
    ms = rng.integers(0, M, size=50)
    ns = rng.integers(0, N, size=50)
    acc, y = oracle.scaled_mm_at(oracle.LAYOUTS[layout], A, sa, B, sb, ms, ns)
    a, b = logical(layout, A, B)
    assert np.array_equal(acc.astype(np.int64), (a @ b)[ms, ns])
    assert np.array_equal(y, full[ms, ns])


# ---------------------------------------------------------------------------
# linear chains


def _integer_tensor(rng, rows, cols):
    """Integers in [-126, 126] with a +-127 in every row and every column, so
    every row-wise and column-wise scale is exactly 1."""
    t = rng.integers(-126, 127, size=(rows, cols)).astype(np.float32)
    for i in range(max(rows, cols)):
        t[i % rows, i % cols] = 127.0 if i % 2 == 0 else -127.0
    return (t.view(np.uint32) >> 16).astype(np.uint16), t.astype(np.int64)


def test_linear_chain_with_unit_scales_is_integer_matmul():
    rng = np.random.default_rng(14)
    M, N, K = 24, 20, 36
    X, Xi = _integer_tensor(rng, M, K)
    W, Wi = _integer_tensor(rng, N, K)
    dY, dYi = _integer_tensor(rng, M, N)

    def bf16_of(ints):
        t = torch.from_numpy(ints).to(torch.float32).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)

    Y = oracle.linear_fwd(X, W)
    assert np.array_equal(Y, bf16_of(Xi @ Wi.T))
    dX, dW = oracle.linear_bwd(dY, X, W)
    assert np.array_equal(dX, bf16_of(dYi @ Wi))
    assert np.array_equal(dW, bf16_of(dYi.T @ Xi))


@pytest.mark.parametrize("rounding", [oracle.RNE, oracle.SR])
def test_linear_chain_composes_the_primitives(rounding):
    t = linear_inputs(replace(single_linear(), M=48, N=40, K=56), seed=1)
    X, W, dY = (bf16_bits(t[k]) for k in ("X", "W", "dY"))
    seed, off = 5, 1000
    Y = oracle.linear_fwd(X, W, rounding, seed, off)
    qx, sx = oracle.quantize_rowwise(X, rounding, seed, off + 0 * 2**40)
    qw, sw = oracle.quantize_rowwise(W, rounding, seed, off + 1 * 2**40)
    assert np.array_equal(Y, oracle.scaled_mm(oracle.NT, qx, sx, qw, sw))
    dX, dW = oracle.linear_bwd(dY, X, W, rounding, seed, off)
    qdy, sdy = oracle.quantize_rowwise(dY, rounding, seed, off + 2 * 2**40)
    qwc, swc = oracle.quantize_colwise(W, rounding, seed, off + 3 * 2**40)
    assert np.array_equal(dX, oracle.scaled_mm(oracle.NN, qdy, sdy, qwc, swc))
    qdyc, sdyc = oracle.quantize_colwise(dY, rounding, seed, off + 4 * 2**40)
    qxc, sxc = oracle.quantize_colwise(X, rounding, seed, off + 5 * 2**40)
    assert np.array_equal(dW, oracle.scaled_mm(oracle.TN, qdyc, sdyc, qxc, sxc))
    dX2, none = oracle.linear_bwd(dY, X, W, rounding, seed, off, want_dw=False)
    assert none is None and np.array_equal(dX2, dX)


def test_linear_fwd_close_to_bf16_matmul():
    """Sanity of scale: the INT8 forward tracks the float product to a few percent."""
    t = linear_inputs(single_linear(), seed=0)
    X, W = bf16_bits(t["X"]), bf16_bits(t["W"])
    Y = oracle.linear_fwd(X, W)
    yf = (Y.astype(np.uint32) << 16).view(np.float32)
    ref = (t["X"].float() @ t["W"].float().T).numpy()
    rel = np.linalg.norm(yf - ref) / np.linalg.norm(ref)
    assert rel < 0.05
