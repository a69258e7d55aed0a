"""Pins of the oracle's row-/column-wise quantization (CPU only).

What the pages fix: quantization divides by a scale and clamps, and
dequantization multiplies back ("Add QAT support for distributed
finetuning", summary); the scale is per row and dynamic ("Quantized model
training", section "INT8 mixed precision training").  The bound the
quantize/dequantize round trip must meet under round-to-nearest is half a
scale step per element.  The rest (absmax, /127, ties to even, zero groups)
are readings, each checked here against an independent statement of it.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import exact_ref
from workloads import bf16_bits, gaussian_bf16, linear_inputs, single_linear

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_to_bf16_bits(values):
    """bf16 bit patterns of values that are exactly representable in bf16."""
    a = np.asarray(values, dtype=np.float32)
    u = a.view(np.uint32)
    assert (u & 0xFFFF == 0).all(), "not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# hand-worked fixture


def test_golden_hand_worked_rows():
    """Hand-derived codes for rows whose scale is a power of two (file cites its derivation)."""
    with open(os.path.join(GOLDEN, "quantize_hand_worked.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        x = f32_to_bf16_bits([case["x"]])
        mode = oracle.SR if case.get("rounding") == "sr" else oracle.RNE
        q, s = oracle.quantize_rowwise(x, mode)
        assert s[0] == np.float32(case["scale"]), case["note"]
        assert q[0].tolist() == case["q"], case["note"]


# ---------------------------------------------------------------------------
# brute force against exact rationals


def _random_bits_rows(rng, rows, cols):
    """bf16 patterns across many binades, including subnormals and zeros."""
    sign = rng.integers(0, 2, size=(rows, cols)) << 15
    exp = rng.integers(0, 255, size=(rows, cols))  # 0..254: no inf/nan
    man = rng.integers(0, 128, size=(rows, cols))
    bits = (sign | (exp << 7) | man).astype(np.uint16)
    # per row: narrow the exponent spread for some rows so codes are not all 0
    for r in range(rows):
        if r % 3 == 0:
            base = int(rng.integers(1, 250))
            e = rng.integers(max(0, base - 8), base + 1, size=cols)
            bits[r] = (sign[r] | (e << 7) | man[r]).astype(np.uint16)
        elif r % 3 == 1:
            e = rng.integers(0, 3, size=cols)  # subnormal / tiny
            bits[r] = (sign[r] | (e << 7) | man[r]).astype(np.uint16)
    return bits


def test_rowwise_rne_matches_exact_rationals():
    rng = np.random.default_rng(1)
    x = _random_bits_rows(rng, 36, 24)
    q, s = oracle.quantize_rowwise(x, oracle.RNE)
    for r in range(x.shape[0]):
        codes, sc = exact_ref.quantize_group([int(b) for b in x[r]], "rne")
        assert Fraction(float(s[r])) == sc, r
        assert q[r].tolist() == codes, r


def test_sr_given_u_matches_exact_rationals():
    rng = np.random.default_rng(2)
    x = _random_bits_rows(rng, 12, 16)
    for r in range(x.shape[0]):
        u = (rng.integers(0, 2**24, size=x.shape[1]).astype(np.float64) / 2**24).astype(np.float32)
        codes, sc = exact_ref.quantize_group([int(b) for b in x[r]], "sr",
                                             [Fraction(float(v)) for v in u])
        q = oracle.quantize_given_u(x[r], float(np.float32(float(sc))), oracle.SR, u)
        assert q.tolist() == codes, r


def test_colwise_is_rowwise_of_transpose():
    x = bf16_bits(gaussian_bf16(40, 72, seed=3))
    qr, sr_ = oracle.quantize_rowwise(np.ascontiguousarray(x.T), oracle.RNE)
    qc, sc = oracle.quantize_colwise(x, oracle.RNE)
    assert np.array_equal(sc, sr_)
    assert np.array_equal(qc, qr.T)


def test_colwise_matches_exact_rationals():
    rng = np.random.default_rng(4)
    x = _random_bits_rows(rng, 20, 9).T.copy()  # columns carry the structured groups
    q, s = oracle.quantize_colwise(x, oracle.RNE)
    for c in range(x.shape[1]):
        codes, sc = exact_ref.quantize_group([int(b) for b in x[:, c]], "rne")
        assert Fraction(float(s[c])) == sc
        assert q[:, c].tolist() == codes


# ---------------------------------------------------------------------------
# invariants on realistic data


@pytest.mark.parametrize("which", ["X", "W", "dY"])
def test_rne_invariants_on_layer_data(which):
    t = linear_inputs(single_linear(), seed=0)[which]
    x = bf16_bits(t)
    q, s = oracle.quantize_rowwise(x, oracle.RNE)
    xf = bits_to_f64(x)
    s64 = s.astype(np.float64)[:, None]
    assert np.abs(q.astype(np.int64)).max() <= 127
    # the largest-magnitude element of each row maps to +-127
    idx = np.abs(xf).argmax(axis=1)
    rows = np.arange(x.shape[0])
    assert np.array_equal(q[rows, idx].astype(np.int64), np.sign(xf[rows, idx]).astype(np.int64) * 127)
    # codes never take the opposite sign
    assert (np.sign(q) * np.sign(xf) >= 0).all()
    # round trip error within half a step (plus the binary32 quotient rounding)
    err = np.abs(q * s64 - xf)
    assert (err <= s64 * (0.5 + 2.0**-16)).all()
    # the scale is amax/127 rounded once
    amax = np.abs(xf).max(axis=1)
    assert np.array_equal(s, (amax / 127.0).astype(np.float32))


def test_sr_invariants_on_layer_data():
    t = linear_inputs(single_linear(), seed=0)["X"]
    x = bf16_bits(t)
    q, s = oracle.quantize_rowwise(x, oracle.SR, seed=7, offset=0)
    xf = bits_to_f64(x)
    s64 = s.astype(np.float64)[:, None]
    err = np.abs(q * s64 - xf)
    assert (err < s64 * (1.0 + 2.0**-16)).all()
    assert (np.sign(q) * np.sign(xf) >= 0).all()
    # SR codes are the floor or the ceiling of the exact quotient
    v = xf / s64
    assert ((q == np.floor(v)) | (q == np.ceil(v)) | (np.abs(q) == 127)).all()


# ---------------------------------------------------------------------------
# closed forms and special cases


def test_integer_rows_are_their_own_codes():
    rng = np.random.default_rng(5)
    ints = rng.integers(-127, 128, size=(16, 64))
    ints[:, 7] = 127 * np.where(rng.integers(0, 2, size=16) == 1, 1, -1)
    x = f32_to_bf16_bits(ints.astype(np.float32))
    q, s = oracle.quantize_rowwise(x, oracle.RNE)
    assert (s == 1.0).all()
    assert np.array_equal(q.astype(np.int64), ints)
    # SR leaves integers unchanged too (u < 1 never reaches the next integer)
    q2, _ = oracle.quantize_rowwise(x, oracle.SR, seed=3)
    assert np.array_equal(q2.astype(np.int64), ints)


@pytest.mark.parametrize("e", [-20, -3, 0, 5])
def test_ties_go_to_even(e):
    # amax = 127 * 2^e gives the exact scale 2^e, so x = (k + 1/2) 2^e is an exact tie
    ks = np.arange(-127, 127)
    vals = np.concatenate([[127.0], (ks + 0.5)]) * 2.0**e
    x = f32_to_bf16_bits(vals.astype(np.float32))[None, :]
    q, s = oracle.quantize_rowwise(x, oracle.RNE)
    assert s[0] == np.float32(2.0**e)
    expect = [127] + [int(k) if k % 2 == 0 else int(k) + 1 for k in ks]
    assert q[0].tolist() == expect


def test_zero_rows_and_columns():
    x = np.zeros((3, 10), dtype=np.uint16)
    x[1, 4] = f32_to_bf16_bits([2.5])[0]
    x[2, 0] = 0x8000  # -0.0
    q, s = oracle.quantize_rowwise(x, oracle.RNE)
    assert s.tolist() == [0.0, float(np.float32(2.5) / np.float32(127)), 0.0]
    assert q[0].tolist() == [0] * 10 and q[2].tolist() == [0] * 10
    assert q[1, 4] == 127
    q, s = oracle.quantize_rowwise(x, oracle.SR, seed=1)
    assert q[0].tolist() == [0] * 10 and s[0] == 0.0
    qc, sc = oracle.quantize_colwise(x, oracle.RNE)
    assert (sc[[0, 1, 2, 3, 5, 6, 7, 8, 9]] == 0).all()
    assert qc[1, 4] == 127 and np.count_nonzero(qc) == 1


def test_ragged_leading_dimension():
    x = bf16_bits(gaussian_bf16(9, 40, seed=6))
    big = np.zeros((9, 48), dtype=np.uint16)
    big[:, :40] = x
    q1, s1 = oracle.quantize_rowwise(x, oracle.SR, seed=9, offset=5)
    q2, s2 = oracle.quantize_rowwise(big[:, :40], oracle.SR, seed=9, offset=5)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


# ---------------------------------------------------------------------------
# column maxima on their own (the statistic a row-wise pass also reports)


def test_col_absmax_matches_numpy_and_column_scales():
    x = bf16_bits(gaussian_bf16(37, 53, seed=9))
    # signed zeros, subnormals, the largest finite bf16 and its negative
    x[0, :4] = [0x8000, 0x0001, 0x8001, 0x7F7F]
    x[5, 4] = 0xFF7F
    x[:, 10] = 0x8000
    cm = oracle.col_absmax(x)
    widened = (x.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(cm, np.abs(widened).max(axis=0))
    assert cm[10] == 0.0 and not np.signbit(cm[10])
    _, s = oracle.quantize_colwise(x)
    assert np.array_equal(s, (cm / np.float32(127)).astype(np.float32))
    # a strided view, and no rows at all
    y = np.zeros((6, 20), dtype=np.uint16)
    y[:, :13] = x[:6, :13]
    assert np.array_equal(oracle.col_absmax(y[:, :13]), np.abs(widened[:6, :13]).max(axis=0))
    assert np.array_equal(oracle.col_absmax(x[:0]), np.zeros(53, np.float32))
