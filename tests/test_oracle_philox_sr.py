"""Pins of the oracle's Philox4x32-10 stream and stochastic rounding (CPU only).

"Quantized model training", section "INT8 mixed precision training", offers
stochastic rounding as an option of the quantization step and says nothing of
its mechanism.  The readings pinned here: u = (Philox word >> 8) * 2^-24, one
word per element at logical index e (block offset + e/4, word e mod 4), and
code = floor(RN32(x/s + u)), so that E[code] = x/s up to binary32 rounding.

The random stream is checked against rocRAND's Philox4x32-10 engine, a
separately written library implementation of the same published generator
(Salmon et al., SC'11), compiled here for the host.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from workloads import bf16_bits, linear_inputs, llama_1b_layers

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_words(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND helper")
    exe = str(tmp_path_factory.mktemp("rr") / "rocrand_philox_words")
    src = os.path.join(HERE, "helpers", "rocrand_philox_words.cpp")
    subprocess.run([hipcc, "-O1", "-o", exe, src], check=True, cwd=str(tmp_path_factory.getbasetemp()))

    def words(seed, offset_blocks, n_words):
        out = subprocess.run([exe, str(seed), str(offset_blocks), str(n_words)], check=True,
                             capture_output=True, text=True).stdout.split()
        return np.array([int(w) for w in out], dtype=np.uint32)

    return words


@pytest.mark.parametrize("seed,offset", [
    (0, 0), (1, 0), (0xDEADBEEF, 17), (2**32 + 5, 2**32 - 3), (2**63 + 12345, 2**40 * 3 + 1),
    (123456789, 2**44 - 2),
])
def test_philox_stream_matches_rocrand(rocrand_words, seed, offset):
    n_blocks = 64
    ours = oracle.philox_stream(seed, offset, n_blocks)
    ref = rocrand_words(seed, offset, 4 * n_blocks)
    assert np.array_equal(ours, ref)


def test_philox_block_counter_words_matter():
    # every counter and key word changes the output (a dropped word would not)
    base = oracle.philox_block([1, 2, 3, 4], [5, 6])
    for i in range(4):
        c = [1, 2, 3, 4]
        c[i] ^= 1
        assert not np.array_equal(oracle.philox_block(c, [5, 6]), base)
    for i in range(2):
        k = [5, 6]
        k[i] ^= 1
        assert not np.array_equal(oracle.philox_block([1, 2, 3, 4], k), base)


def test_sr_uses_word_e_mod_4_of_block_offset_plus_e_div_4():
    # Build a row with s = 1 and x = 0 except an amax of 127: codes of the zero
    # elements are floor(u) = 0, so use x = 0.5 instead: code = floor(0.5 + u)
    # is 1 exactly when u >= 0.5, i.e. when the top bit of the word is set.
    cols = 64
    xv = np.full(cols, 0.5, dtype=np.float32)
    xv[0] = 127.0
    x = ((xv.view(np.uint32) >> 16).astype(np.uint16))[None, :]
    for seed, offset in [(3, 0), (99, 2**40 + 7)]:
        q, s = oracle.quantize_rowwise(x, oracle.SR, seed=seed, offset=offset)
        assert s[0] == 1.0
        words = oracle.philox_stream(seed, offset, cols // 4)
        expect = (words >> 31).astype(np.int64)
        expect[0] = 127
        assert np.array_equal(q[0].astype(np.int64), expect)


def test_sr_draws_follow_logical_index_across_rows():
    # element (r, c) of an R x C tensor draws from e = r*C + c in both directions
    rows, cols = 6, 10
    xv = np.full((rows, cols), 0.5, dtype=np.float32)
    xv[:, 0] = 127.0
    xv[0, :] = 127.0
    x = (xv.view(np.uint32) >> 16).astype(np.uint16)
    words = oracle.philox_stream(11, 40, (rows * cols + 3) // 4 + 1)
    up = (words >> 31).astype(np.int64)
    q, _ = oracle.quantize_rowwise(x, oracle.SR, seed=11, offset=40)
    qc, _ = oracle.quantize_colwise(x, oracle.SR, seed=11, offset=40)
    for r in range(1, rows):
        for c in range(1, cols):
            e = r * cols + c
            assert q[r, c] == up[e] and qc[r, c] == up[e]


@pytest.mark.parametrize("v", [0.3, 1.7, 63.25, -5.125, 126.6, -125.5, 0.0009765625])
def test_sr_up_probability_by_enumerating_every_uniform(v):
    """P(code = floor(v) + 1) over all 2^24 uniforms equals frac(v) to within the
    binary32 rounding of v + u (at most half an ulp of 128, i.e. 2^-18)."""
    s = np.float32(1.0)
    xf = np.float32(v)
    xbits = np.uint16(np.array([xf], dtype=np.float32).view(np.uint32)[0] >> 16)
    xval = float(np.array([np.uint32(xbits) << 16], dtype=np.uint32).view(np.float32)[0])
    u = (np.arange(2**24, dtype=np.float64) / 2**24).astype(np.float32)
    q = oracle.quantize_given_u(np.full(2**24, xbits, dtype=np.uint16), float(s), oracle.SR, u)
    lo = np.floor(xval)
    frac = xval - lo
    p_up = np.count_nonzero(q.astype(np.int64) == lo + 1) / 2**24
    assert np.count_nonzero((q != lo) & (q != lo + 1)) == 0
    assert abs(p_up - frac) <= 2.0**-18 + 2.0**-24


def test_sr_clamps_at_127():
    xbits = np.array([np.float32(127.0).view(np.uint32) >> 16], dtype=np.uint16)
    u = np.array([0.999999940395], dtype=np.float32)
    q = oracle.quantize_given_u(xbits, 1.0, oracle.SR, u)
    assert q[0] == 127


def _unbiasedness(q_per_seed, v):
    """Per-element and pooled checks that mean code over seeds is v."""
    n = q_per_seed.shape[0]
    mean = q_per_seed.mean(axis=0)
    f = v - np.floor(v)
    sd = np.sqrt(f * (1 - f) / n)
    assert (np.abs(mean - v) <= 5 * sd + 2.0**-16).all()
    var = f * (1 - f)
    z = (q_per_seed.sum(axis=0) - n * v).sum() / np.sqrt(n * var.sum())
    assert abs(z) < 5


@pytest.mark.slow
def test_sr_unbiased_over_256_seeds_rowwise():
    """Llama-1B activations, row-wise over full 2048-wide rows, [64, 64] slice checked."""
    shape = llama_1b_layers()[0]
    from dataclasses import replace
    small = replace(shape, M=64)
    x = bf16_bits(linear_inputs(small, seed=0, want=("X",))["X"])
    qs = []
    for seed in range(256):
        q, s = oracle.quantize_rowwise(x, oracle.SR, seed=seed, offset=0)
        qs.append(q[:, :64].astype(np.float64))
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    v = xf[:, :64] / s.astype(np.float64)[:, None]
    _unbiasedness(np.stack(qs), v)


@pytest.mark.slow
def test_sr_unbiased_over_256_seeds_colwise():
    """Llama-1B output gradients, column-wise over all rows of a 2048-token band."""
    shape = llama_1b_layers()[0]
    from dataclasses import replace
    small = replace(shape, M=2048)
    dy = bf16_bits(linear_inputs(small, seed=0, want=("dY",))["dY"])
    band = np.ascontiguousarray(dy[:, :64])
    qs = []
    for seed in range(256):
        q, s = oracle.quantize_colwise(band, oracle.SR, seed=seed, offset=2**40 * 4)
        qs.append(q[:64, :].astype(np.float64))
    xf = (band.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    v = xf[:64, :] / s.astype(np.float64)[None, :]
    _unbiasedness(np.stack(qs), v)
