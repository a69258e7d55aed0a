"""GPU parity of the row-wise FP8 (E4M3) variant.

* Quantization (row- and column-wise): codes and scales bit for bit against
  the oracle over ragged shapes with special values, and the exhaustive
  quotient check: every finite bf16 x against every positive finite bf16
  absmax (the FMA quotient, clamp and hardware E4M3 conversion against IEEE
  division and the oracle's E4M3 rounding).
* FP8 matmul in the three layouts.  The matrix core does not sum the 64
  products of one instruction exactly: measured on the device, it aligns them
  to the largest and truncates at about 2^-17 of it (a product of 448 plus 63
  small ones comes out 0.04-0.056 low; the worst error seen over random
  operands is 2^-12.2 of the largest product of the instruction).  So outputs
  are compared with the oracle's exact-sum result within
    |y - y_exact| <= [2^-10 sum_blocks max|a| max|b| + (K/64 + 1) 2^-24 sum|a b|] sa sb
                     + 2^-7 |y_exact| + 2^-133
  (blocks: the 64 contraction values of one instruction; the second term is
  fp32 accumulation across instructions; 2^-7 |y| covers the two bf16
  roundings; 2^-133 the smallest bf16 subnormal).  Most outputs must still be
  identical to the oracle's.
* The linear chains, against the oracle's FP8 quantization and matmul.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import bits_to_bf16, canary_intact, padded, padded_copy, round_up, special_rows_bf16, tensor_bits
from workloads import LinearShape, gaussian_bf16, linear_inputs

pytestmark = pytest.mark.gpu

i8 = pytest.importorskip("int8_mixed_precision_rowwise_amd")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

THREADS = min(16, len(os.sched_getaffinity(0)))


def same_f32(t: torch.Tensor, want: np.ndarray, what: str):
    assert np.array_equal(t.cpu().numpy().view(np.uint32), want.view(np.uint32)), what


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


LUT = None


def decode(codes: np.ndarray) -> np.ndarray:
    global LUT
    if LUT is None:
        LUT = oracle.e4m3_to_float(np.arange(256, dtype=np.uint8)).astype(np.float64)
    return LUT[codes]


def block_max(codes: np.ndarray, k_axis: int) -> np.ndarray:
    """[outer, K/64]: the largest |value| of each 64-long block along k."""
    v = np.abs(decode(codes))
    v = v if k_axis == 1 else v.T
    outer, K = v.shape
    return v.reshape(outer, K // 64, 64).max(axis=2) if K % 64 == 0 else np.stack(
        [v[:, i:i + 64].max(axis=1) for i in range(0, K, 64)], axis=1)


def block_term(layout, A, B):
    """(Am [M, blocks], Bm [N, blocks]) of the operands in their layouts."""
    Am = block_max(A, 1 if layout in ("NT", "NN") else 0)
    Bm = block_max(B, 1 if layout == "NT" else 0)
    return Am, Bm


def within_bound(got_bits, want_bits, absdot, sab, K, what, blocks):
    got, want = bf16_to_f64(got_bits), bf16_to_f64(want_bits)
    acc_err = 2.0**-10 * blocks + (K / 64 + 1) * 2.0**-24 * absdot
    bound = acc_err * sab * (1 + 2.0**-20) + 2.0**-7 * np.abs(want) + 2.0**-133
    bad = np.abs(got - want) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs outside the fp32-summation bound"
    same = float(np.mean(got_bits == want_bits))
    assert same > 0.5, f"{what}: only {same:.3f} of outputs equal the exact-sum result"
    return same


ROW_SHAPES = [(1, 1), (3, 17), (7, 513), (64, 2048), (9, 5000), (5, 14336), (3, 16385)]


@pytest.mark.parametrize("rows,cols", ROW_SHAPES)
def test_quantize_rowwise_fp8(rows, cols):
    rng = np.random.default_rng(rows * 9001 + cols)
    xb = special_rows_bf16(rng, rows, cols)
    x = padded_copy(bits_to_bf16(xb), round_up(cols, 8) + 8)
    qs, q = padded(rows, cols, round_up(cols, 16) + 16, torch.uint8)
    _, s = i8.quantize_rowwise_fp8(x, q=q)
    torch.cuda.synchronize()
    qo, so = oracle.quantize_rowwise_fp8(xb)
    same_f32(s, so, "scales")
    got = q.cpu().numpy()
    if not np.array_equal(got, qo):
        bad = np.argwhere(got != qo)[0]
        raise AssertionError(f"codes differ at {bad.tolist()}: x {xb[bad[0], bad[1]]:#06x} "
                             f"gpu {got[bad[0], bad[1]]:#04x} oracle {qo[bad[0], bad[1]]:#04x}")
    assert canary_intact(qs, cols)


@pytest.mark.parametrize("rows,cols", [(1, 1), (17, 3), (513, 7), (2048, 64), (1000, 513), (300, 5632)])
def test_quantize_colwise_fp8(rows, cols):
    rng = np.random.default_rng(rows * 31 + cols)
    xb = np.ascontiguousarray(special_rows_bf16(rng, cols, rows).T)
    x = padded_copy(bits_to_bf16(xb), round_up(cols, 8) + 8)
    qs, q = padded(rows, cols, round_up(cols, 16) + 16, torch.uint8)
    _, s = i8.quantize_colwise_fp8(x, q=q)
    torch.cuda.synchronize()
    qo, so = oracle.quantize_colwise_fp8(xb)
    same_f32(s, so, "scales")
    assert np.array_equal(q.cpu().numpy(), qo)
    assert canary_intact(qs, cols)


def test_quotient_exhaustive_fp8():
    """Row i holds every bf16 pattern whose magnitude is at most absmax a_i
    (others 0); all positive finite bf16 a_i."""
    amax = np.arange(1, 0x7F80, dtype=np.uint32)
    cols = 65536
    pats = np.arange(cols, dtype=np.uint32)
    mag = pats & 0x7FFF
    finite = mag < 0x7F80
    band = 2048
    for r0 in range(0, len(amax), band):
        a = amax[r0:r0 + band]
        keep = finite[None, :] & (mag[None, :] <= a[:, None])
        xb = np.where(keep, pats[None, :], 0).astype(np.uint16)
        xg = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
        q, s = i8.quantize_rowwise_fp8(xg)
        step = -(-len(a) // THREADS)
        qo = np.empty((len(a), cols), np.uint8)
        so = np.empty(len(a), np.float32)

        def work(i0):
            qq, ss = oracle.quantize_rowwise_fp8(xb[i0:i0 + step])
            qo[i0:i0 + step], so[i0:i0 + step] = qq, ss

        with cf.ThreadPoolExecutor(THREADS) as ex:
            list(ex.map(work, range(0, len(a), step)))
        assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
        qn = q.cpu().numpy()
        if not np.array_equal(qn, qo):
            bad = np.argwhere(qn != qo)[0]
            raise AssertionError(f"x bits {xb[bad[0], bad[1]]:#06x} amax bits {a[bad[0]]:#06x}: "
                                 f"gpu {qn[bad[0], bad[1]]:#04x} oracle {qo[bad[0], bad[1]]:#04x}")
        del xg, q


def fp8_operands(layout, M, N, K, seed):
    """E4M3 codes and scales of Gaussian bf16 operands, quantized by the oracle
    along the contraction (row-wise for K-contiguous operands, column-wise else)."""
    if layout == "NT":
        a, b = gaussian_bf16(M, K, seed=seed), gaussian_bf16(N, K, seed=seed + 1, std=0.02)
        (A, sa), (B, sb) = oracle.quantize_rowwise_fp8(tensor_bits(a)), oracle.quantize_rowwise_fp8(tensor_bits(b))
    elif layout == "NN":
        a, b = gaussian_bf16(M, K, seed=seed), gaussian_bf16(K, N, seed=seed + 1, std=0.02)
        (A, sa), (B, sb) = oracle.quantize_rowwise_fp8(tensor_bits(a)), oracle.quantize_colwise_fp8(tensor_bits(b))
    else:
        a, b = gaussian_bf16(K, M, seed=seed, std=1e-3), gaussian_bf16(K, N, seed=seed + 1)
        (A, sa), (B, sb) = oracle.quantize_colwise_fp8(tensor_bits(a)), oracle.quantize_colwise_fp8(tensor_bits(b))
    return A, sa, B, sb


def gpu_mm(layout, A, sa, B, sb):
    """The GPU matmul with both operands in storage whose rows are padded to
    16 bytes plus 16 (canary-filled), as the ABI asks of every operand."""
    dev = lambda v: torch.from_numpy(v).cuda()  # noqa: E731
    pad = lambda v: padded_copy(dev(v), round_up(v.shape[1], 16) + 16)  # noqa: E731
    return tensor_bits(i8.fp8_scaled_mm(layout, pad(A), dev(sa), pad(B), dev(sb)))


# every layout takes output extents that are multiples of 4; NT (both operands
# K-contiguous) any extents
FP8_SHAPES = [("NT", 1, 1, 16), ("NT", 17, 33, 64), ("NT", 255, 130, 512)] + [
    (lay, M, N, K) for lay in ("NT", "NN", "TN")
    for M, N, K in ((4, 4, 16), (12, 4, 32), (20, 36, 64), (256, 132, 512), (300, 260, 1008), (1024, 1024, 1024))]


@pytest.mark.parametrize("layout,M,N,K", FP8_SHAPES)
def test_fp8_scaled_mm(layout, M, N, K):
    A, sa, B, sb = fp8_operands(layout, M, N, K, seed=M + N + K)
    got = gpu_mm(layout, A, sa, B, sb)
    want, _, absdot = oracle.fp8_scaled_mm(oracle.LAYOUTS[layout], A, sa, B, sb, want_acc=True)
    Am, Bm = block_term(layout, A, B)
    within_bound(got, want, absdot, np.abs(sa[:, None] * sb[None, :]).astype(np.float64), K,
                 f"{layout} {M}x{N}x{K}", Am @ Bm.T)


def test_fp8_shape_rules():
    z = lambda r, c: torch.zeros((r, c), dtype=torch.uint8, device="cuda")  # noqa: E731
    s = lambda n: torch.ones(n, device="cuda")  # noqa: E731
    # K = 24 (not a multiple of 16); N = 3 read down B's rows; M = 3 read down A's rows
    for layout, A, B, M, N in (("NT", z(4, 24), z(4, 24), 4, 4), ("NN", z(4, 16), z(16, 3), 4, 3),
                               ("TN", z(16, 3), z(16, 4), 3, 4)):
        with pytest.raises(i8.I8mpError) as e:
            i8.fp8_scaled_mm(layout, A, s(M), B, s(N))
        assert e.value.status == 1


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_fp8_scaled_mm_4096_sampled(layout):
    n = 4096
    A, sa, B, sb = fp8_operands(layout, n, n, n, seed=5)
    got = gpu_mm(layout, A, sa, B, sb)
    rng = np.random.default_rng(9)
    ms = np.concatenate([rng.integers(0, n, 4096), np.repeat([0, n - 1], n)])
    ns = np.concatenate([rng.integers(0, n, 4096), np.tile(np.arange(n), 2)])
    y, _, absdot = oracle.fp8_scaled_mm_at(oracle.LAYOUTS[layout], A, sa, B, sb, ms, ns)
    Am, Bm = block_term(layout, A, B)
    within_bound(got[ms, ns], y, absdot, np.abs(sa[ms] * sb[ns]).astype(np.float64), n, f"{layout} 4096",
                 np.einsum("ij,ij->i", Am[ms], Bm[ns]))


@pytest.mark.parametrize("M,N,K", [(32, 48, 64), (256, 512, 512), (1008, 272, 608), (512, 4096, 256)])
def test_linear_chains_fp8(M, N, K):
    t = linear_inputs(LinearShape("fp8_chain", M, N, K), seed=2, device="cuda")
    X, W, dY = t["X"], t["W"], t["dY"]
    Xb, Wb, dYb = tensor_bits(X), tensor_bits(W), tensor_bits(dY)
    Y = tensor_bits(i8.linear_fwd_fp8(X, W))
    dX, dW = (tensor_bits(v) for v in i8.linear_bwd_fp8(dY, X, W))
    qx, sx = oracle.quantize_rowwise_fp8(Xb)
    qw, sw = oracle.quantize_rowwise_fp8(Wb)
    y, _, ad = oracle.fp8_scaled_mm(oracle.NT, qx, sx, qw, sw, want_acc=True)
    Am, Bm = block_term("NT", qx, qw)
    within_bound(Y, y, ad, np.abs(sx[:, None] * sw[None, :]).astype(np.float64), K, "Y", Am @ Bm.T)
    qdy, sdy = oracle.quantize_rowwise_fp8(dYb)
    qwc, swc = oracle.quantize_colwise_fp8(Wb)
    y, _, ad = oracle.fp8_scaled_mm(oracle.NN, qdy, sdy, qwc, swc, want_acc=True)
    Am, Bm = block_term("NN", qdy, qwc)
    within_bound(dX, y, ad, np.abs(sdy[:, None] * swc[None, :]).astype(np.float64), N, "dX", Am @ Bm.T)
    qdyc, sdyc = oracle.quantize_colwise_fp8(dYb)
    qxc, sxc = oracle.quantize_colwise_fp8(Xb)
    y, _, ad = oracle.fp8_scaled_mm(oracle.TN, qdyc, sdyc, qxc, sxc, want_acc=True)
    Am, Bm = block_term("TN", qdyc, qxc)
    within_bound(dW, y, ad, np.abs(sdyc[:, None] * sxc[None, :]).astype(np.float64), M, "dW", Am @ Bm.T)
    # With both gradients the chain takes dY's column maxima from its row-wise
    # pass; its gradients equal, byte for byte, the FP8 GEMMs of the public
    # quantize passes' codes (same codes, same deterministic GEMM).
    gx, gw = i8.linear_bwd_fp8(dY, X, W)
    qa, sa = i8.quantize_rowwise_fp8(dY)
    qb, sb = i8.quantize_colwise_fp8(W)
    want_dx = i8.fp8_scaled_mm("NN", qa, sa, qb, sb)
    qa, sa = i8.quantize_colwise_fp8(dY)
    qb, sb = i8.quantize_colwise_fp8(X)
    want_dw = i8.fp8_scaled_mm("TN", qa, sa, qb, sb)
    torch.cuda.synchronize()
    assert torch.equal(gx.view(torch.int16), want_dx.view(torch.int16)), "dX differs from the primitives"
    assert torch.equal(gw.view(torch.int16), want_dw.view(torch.int16)), "dW differs from the primitives"


@pytest.mark.parametrize("K", [64, 1024])
def test_fp8_sums_against_exact(K):
    """The raw fp32 sums (no epilogue) within the truncation bound above, and
    the worst error of one instruction well inside it."""
    A, _, B, _ = fp8_operands("NT", 256, 256, K, seed=K)
    dev = lambda v: torch.from_numpy(v).cuda()  # noqa: E731
    pad = lambda v: padded_copy(dev(v), round_up(v.shape[1], 16) + 16)  # noqa: E731
    got = i8.fp8_mm_f32("NT", pad(A), pad(B)).cpu().numpy().astype(np.float64)
    a, b = decode(A), decode(B)
    exact = a @ b.T
    absdot = np.abs(a) @ np.abs(b).T
    Am, Bm = block_term("NT", A, B)
    bound = 2.0**-10 * (Am @ Bm.T) + (K / 64 + 1) * 2.0**-24 * absdot
    assert (np.abs(got - exact) <= bound).all()
