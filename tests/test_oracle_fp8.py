"""Pins of the oracle's FP8 (E4M3) variant (CPU only).

The E4M3 format is OCP FP8's ("e4m3fn"); torch's float8_e4m3fn conversion is
an independent implementation of it, used here for the decode of every code
and for the rounding of a sweep of fp32 values that holds every rounding tie
of the format and both neighbours of each.  The quantization readings (scale
amax / 448, IEEE quotient clamped to +-448, a zero element codes as +0) are
checked through invariants; the FP8 matmul against numpy's float64 matmul of
the decoded codes, which is exact at these sizes.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits, gaussian_bf16, linear_inputs, single_linear

F8 = torch.float8_e4m3fn


def torch_e4m3(values: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32)).to(F8).view(torch.uint8).numpy()


def widen(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_decode_every_code():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_to_float(codes)
    want = torch.from_numpy(codes).view(F8).float().numpy()
    nan = (codes & 0x7F) == 0x7F
    assert np.isnan(got[nan]).all() and np.isnan(want[nan]).all()
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    assert got[0x7E] == 448.0 and got[0x01] == 2.0**-9 and got[0x08] == 2.0**-6


def rounding_sweep() -> np.ndarray:
    """fp32 values in [-448, 448]: every exponent the format reaches (and the
    underflow range below it), the top 5 fraction bits, and low fraction bits
    0, 1, all-ones below the tie bit, all-ones: every tie of E4M3 (at binary32
    fraction bit 19 for normals, higher for subnormal results) and both
    neighbours."""
    vals = []
    for e in range(127 - 24, 127 + 9):
        for top in range(32):
            for low in (0, 1, 0x1FFFF, 0x3FFFF):
                vals.append((e << 23) | (top << 18) | low)
    u = np.array(vals, dtype=np.uint32)
    f = u.view(np.float32)
    f = f[np.abs(f) <= 448.0]
    return np.concatenate([f, -f, np.float32([0.0, 448.0, -448.0])])


def test_encode_matches_torch_on_every_tie_and_neighbour():
    v = rounding_sweep()
    assert np.array_equal(oracle.float_to_e4m3(v), torch_e4m3(v))
    rng = np.random.default_rng(3)
    r = (rng.uniform(-1, 1, 20000) * 2.0 ** rng.integers(-14, 9, 20000)).astype(np.float32)
    assert np.array_equal(oracle.float_to_e4m3(r), torch_e4m3(r))
    # saturation past the largest finite value (torch's cast would give NaN there)
    assert oracle.float_to_e4m3(np.float32([449.0, 500.0, 1e30, -1e30])).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]


@pytest.mark.parametrize("which", ["X", "W", "dY"])
def test_rowwise_fp8_codes_and_invariants(which):
    t = linear_inputs(single_linear(), seed=4)
    x = bf16_bits(t[which])
    x[0, :3] = [0x0000, 0x8000, 0x0001]  # +0, -0, the smallest bf16 subnormal
    x[1, :] = 0  # an all-zero row
    q, s = oracle.quantize_rowwise_fp8(x)
    xf = widen(x)
    amax = np.abs(xf).max(axis=1)
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
    assert (q[1] == 0).all() and s[1] == 0
    assert q[0, 0] == 0 and q[0, 1] == 0  # both zeros code as +0
    # codes are torch's E4M3 rounding of the clamped IEEE quotient
    nz = s > 0
    v = np.clip(xf[nz] / s[nz, None], -448, 448).astype(np.float32)
    want = torch_e4m3(v)
    want[xf[nz] == 0] = 0
    assert np.array_equal(q[nz], want)
    # the largest element of each row maps to +-448
    for r in np.nonzero(nz)[0]:
        c = int(np.argmax(np.abs(xf[r])))
        assert q[r, c] in (0x7E, 0xFE)
    # round trip within half a step of the E4M3 grid at that magnitude
    deq = oracle.e4m3_to_float(q).astype(np.float64) * s[:, None]
    mag = np.abs(v.astype(np.float64))
    step = np.where(mag < 2.0**-6, 2.0**-9, 2.0 ** (np.floor(np.log2(np.maximum(mag, 2.0**-6))) - 3))
    err = np.abs(deq[nz] - xf[nz]) / s[nz, None]
    assert (err <= step / 2 * (1 + 2.0**-20) + 2.0**-20).all()


def test_colwise_fp8_is_rowwise_of_transpose():
    x = bf16_bits(gaussian_bf16(70, 33, seed=8))
    qc, sc = oracle.quantize_colwise_fp8(x)
    qr, sr = oracle.quantize_rowwise_fp8(np.ascontiguousarray(x.T))
    assert np.array_equal(qc, qr.T) and np.array_equal(sc, sr)


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (7, 5, 33), (40, 24, 130), (65, 129, 257)])
def test_fp8_scaled_mm_against_float64_matmul(layout, M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    def codes(r, c):
        q = rng.integers(0, 256, (r, c), dtype=np.uint8)
        q[(q & 0x7F) == 0x7F] = 0x7E  # no NaN codes
        return q
    shp = {"NT": ((M, K), (N, K)), "NN": ((M, K), (K, N)), "TN": ((K, M), (K, N))}[layout]
    A, B = codes(*shp[0]), codes(*shp[1])
    sa = rng.uniform(0.01, 2, M).astype(np.float32)
    sb = rng.uniform(0.01, 2, N).astype(np.float32)
    y, acc, absdot = oracle.fp8_scaled_mm(oracle.LAYOUTS[layout], A, sa, B, sb, want_acc=True)
    a = oracle.e4m3_to_float(A).astype(np.float64)
    b = oracle.e4m3_to_float(B).astype(np.float64)
    a = a if layout != "TN" else a.T
    b = b if layout == "NT" else b.T
    exact = a @ b.T  # every product and partial sum is exact in float64 here
    assert np.array_equal(acc, exact.astype(np.float32))
    assert np.array_equal(absdot, np.abs(a) @ np.abs(b).T)
    yf = (acc * sa[:, None]).astype(np.float32) * sb[None, :]
    want = torch.from_numpy(yf.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, want)


def test_sampled_positions_match_full_matmul():
    rng = np.random.default_rng(11)
    A = rng.integers(0, 0x7E, (50, 96), dtype=np.uint8) | (rng.integers(0, 2, (50, 96), dtype=np.uint8) << 7)
    B = rng.integers(0, 0x7E, (40, 96), dtype=np.uint8)
    sa = rng.uniform(0.1, 1, 50).astype(np.float32)
    sb = rng.uniform(0.1, 1, 40).astype(np.float32)
    y, acc, absdot = oracle.fp8_scaled_mm(oracle.NT, A, sa, B, sb, want_acc=True)
    ms, ns = rng.integers(0, 50, 300), rng.integers(0, 40, 300)
    y2, acc2, absdot2 = oracle.fp8_scaled_mm_at(oracle.NT, A, sa, B, sb, ms, ns)
    assert np.array_equal(y2, y[ms, ns]) and np.array_equal(acc2, acc[ms, ns])
    assert np.array_equal(absdot2, absdot[ms, ns])
