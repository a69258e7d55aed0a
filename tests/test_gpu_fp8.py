"""GPU parity of the row-wise FP8 (E4M3) variant.

* Quantization (row- and column-wise): codes and scales bit for bit against
  the oracle over ragged shapes with special values, and the exhaustive
  quotient check: every finite bf16 x against every positive finite bf16
  absmax (the FMA quotient, clamp and hardware E4M3 conversion against IEEE
  division and the oracle's E4M3 rounding).
* FP8 matmul in the three layouts.  The matrix core does not sum exactly,
  and the summation of v_mfma_scale_f32_32x32x64_f8f6f4 is characterized on
  the device (test_fp8_group_truncation_rule pins it with constructed
  operands): the products of each group of 8 consecutive contraction indices
  are truncated toward zero to multiples of 2^(E_g - 13), E_g the largest
  e(a) + e(b) of the group (e: the operand's exponent, -6 for subnormals);
  the group sums then enter the fp32 accumulator with at most fp32-level
  error per instruction.  Derived bound on an accumulator (every product of
  E4M3 values is exact, so at most 7 products of a group lose bits, each less
  than 2^(E_g - 13); the accumulation is charged 2^-21 of the accumulator
  and the instruction's products per instruction, eight times the largest
  error observed, about 1.5 * 2^-24):
    |acc - exact| <= 7 * 2^-13 * sum_groups 2^E_g + ceil(K/64) * 2^-21 * sum|a b|
  and for the bf16 outputs that times sa sb, plus 2^-7 |y_exact| (the two
  bf16 roundings) and 2^-133 (the smallest bf16 subnormal).  The tests report
  the largest error as a fraction of the bound and the share of outputs equal
  to the exact-sum result; the exact share is not part of the bound.
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


def exps(codes: np.ndarray) -> np.ndarray:
    """e(v) of each E4M3 code as the matrix core aligns by: floor(log2 |v|) for
    normal values, -6 for subnormals; a large negative sentinel for zeros."""
    c = codes.astype(np.int16)
    f = (c >> 3) & 15
    e = np.where(f == 0, -6, f - 7)
    return np.where((c & 0x7F) == 0, -1000, e).astype(np.int16)


def group_term(layout, A, B, ms=None, ns=None):
    """sum over the groups of 8 consecutive contraction indices of 2^E_g, E_g
    the largest e(a_k) + e(b_k) over the group's nonzero products, for every
    output [M, N] (or for the output pairs ms, ns)."""
    ea = exps(A) if layout in ("NT", "NN") else exps(A).T  # [M, K]
    eb = exps(B) if layout == "NT" else exps(B).T  # [N, K]
    K = ea.shape[1]
    pad = (-K) % 8
    if pad:
        ea = np.pad(ea, ((0, 0), (0, pad)), constant_values=-1000)
        eb = np.pad(eb, ((0, 0), (0, pad)), constant_values=-1000)
    G = ea.shape[1] // 8

    def reduce(E):  # [..., K'] -> [...]
        Eg = E.reshape(*E.shape[:-1], G, 8).max(axis=-1).astype(np.float64)
        return np.where(Eg < -200, 0.0, np.exp2(Eg)).sum(axis=-1)

    if ms is not None:
        out = np.empty(len(ms))
        for i in range(0, len(ms), 2048):
            out[i:i + 2048] = reduce(ea[ms[i:i + 2048]] + eb[ns[i:i + 2048]])
        return out
    M, N = ea.shape[0], eb.shape[0]
    out = np.empty((M, N))
    step = max(1, (1 << 24) // (N * ea.shape[1]))
    for m0 in range(0, M, step):
        out[m0:m0 + step] = reduce(ea[m0:m0 + step, None, :] + eb[None, :, :])
    return out


BOUND_REPORT = []


def within_bound(got_bits, want_bits, absdot, sab, K, what, groups):
    got, want = bf16_to_f64(got_bits), bf16_to_f64(want_bits)
    acc_err = 7 * 2.0**-13 * groups + -(-K // 64) * 2.0**-21 * absdot
    bound = acc_err * sab * (1 + 2.0**-20) + 2.0**-7 * np.abs(want) + 2.0**-133
    err = np.abs(got - want)
    bad = err > bound
    same = float(np.mean(got_bits == want_bits))
    ratio = float((err / bound).max()) if err.size else 0.0
    BOUND_REPORT.append((what, ratio, same))
    print(f"[fp8 bound] {what}: max |error| / bound = {ratio:.4f}, outputs equal to the exact-sum result: {same:.4f}")
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs outside the derived summation bound"
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


# Any shape: the pipelined kernel's (K a multiple of 16, extents read down
# an operand's rows multiples of 4) and the general kernel's (the rest: K of
# 8, 24, 40, 1000; odd M and N in every layout).
FP8_SHAPES = [("NT", 1, 1, 16), ("NT", 17, 33, 64), ("NT", 255, 130, 512)] + [
    (lay, M, N, K) for lay in ("NT", "NN", "TN")
    for M, N, K in ((4, 4, 16), (12, 4, 32), (20, 36, 64), (256, 132, 512), (300, 260, 1008), (1024, 1024, 1024),
                    (1, 1, 8), (3, 5, 24), (17, 33, 40), (255, 130, 1000), (129, 257, 520))]


@pytest.mark.parametrize("layout,M,N,K", FP8_SHAPES)
def test_fp8_scaled_mm(layout, M, N, K):
    A, sa, B, sb = fp8_operands(layout, M, N, K, seed=M + N + K)
    got = gpu_mm(layout, A, sa, B, sb)
    want, _, absdot = oracle.fp8_scaled_mm(oracle.LAYOUTS[layout], A, sa, B, sb, want_acc=True)
    within_bound(got, want, absdot, np.abs(sa[:, None] * sb[None, :]).astype(np.float64), K,
                 f"{layout} {M}x{N}x{K}", group_term(layout, A, B))


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_fp8_general_kernel_equals_pipelined(layout):
    """Shapes the pipelined kernel cannot take run on the general kernel, which
    issues the same instruction on the same operand placement: its sums are
    the pipelined kernel's, bit for bit.  NT: K = 40 (general) against the same
    operands with 8 zero contraction columns appended (K = 48, pipelined; zero
    codes add nothing).  NN / TN: an output extent read down an operand's rows
    of 255 (general) against the same operands at 256 (pipelined), rows /
    columns in common compared."""
    dev = lambda v: torch.from_numpy(np.ascontiguousarray(v)).cuda()  # noqa: E731
    if layout == "NT":
        A, sa, B, sb = fp8_operands("NT", 300, 260, 40, seed=11)
        A48 = np.pad(A, ((0, 0), (0, 8)))
        B48 = np.pad(B, ((0, 0), (0, 8)))
        got = gpu_mm("NT", A, sa, B, sb)
        want = gpu_mm("NT", A48, sa, B48, sb)
        assert np.array_equal(got, want)
        f_got = i8.fp8_mm_f32("NT", padded_copy(dev(A), 64), padded_copy(dev(B), 64))
        f_want = i8.fp8_mm_f32("NT", dev(A48), dev(B48))
        torch.cuda.synchronize()
        assert torch.equal(f_got.view(torch.int32), f_want.view(torch.int32)), "fp32 sums"
        return
    A, sa, B, sb = fp8_operands(layout, 256, 256, 520, seed=12)
    if layout == "NN":  # N read down B's rows: 255 columns of B
        got = gpu_mm("NN", A, sa, B[:, :255], sb[:255])
        want = gpu_mm("NN", A, sa, B, sb)
        assert np.array_equal(got, want[:, :255])
    else:  # TN: M read down A's rows, N down B's: 255 columns of A
        got = gpu_mm("TN", A[:, :255], sa[:255], B, sb)
        want = gpu_mm("TN", A, sa, B, sb)
        assert np.array_equal(got, want[:255])


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_fp8_scaled_mm_4096_sampled(layout):
    n = 4096
    A, sa, B, sb = fp8_operands(layout, n, n, n, seed=5)
    got = gpu_mm(layout, A, sa, B, sb)
    rng = np.random.default_rng(9)
    ms = np.concatenate([rng.integers(0, n, 4096), np.repeat([0, n - 1], n)])
    ns = np.concatenate([rng.integers(0, n, 4096), np.tile(np.arange(n), 2)])
    y, _, absdot = oracle.fp8_scaled_mm_at(oracle.LAYOUTS[layout], A, sa, B, sb, ms, ns)
    within_bound(got[ms, ns], y, absdot, np.abs(sa[ms] * sb[ns]).astype(np.float64), n, f"{layout} 4096",
                 group_term(layout, A, B, ms, ns))


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
    within_bound(Y, y, ad, np.abs(sx[:, None] * sw[None, :]).astype(np.float64), K, f"chain Y {M}x{N}x{K}",
                 group_term("NT", qx, qw))
    qdy, sdy = oracle.quantize_rowwise_fp8(dYb)
    qwc, swc = oracle.quantize_colwise_fp8(Wb)
    y, _, ad = oracle.fp8_scaled_mm(oracle.NN, qdy, sdy, qwc, swc, want_acc=True)
    within_bound(dX, y, ad, np.abs(sdy[:, None] * swc[None, :]).astype(np.float64), N, f"chain dX {M}x{N}x{K}",
                 group_term("NN", qdy, qwc))
    qdyc, sdyc = oracle.quantize_colwise_fp8(dYb)
    qxc, sxc = oracle.quantize_colwise_fp8(Xb)
    y, _, ad = oracle.fp8_scaled_mm(oracle.TN, qdyc, sdyc, qxc, sxc, want_acc=True)
    within_bound(dW, y, ad, np.abs(sdyc[:, None] * sxc[None, :]).astype(np.float64), M, f"chain dW {M}x{N}x{K}",
                 group_term("TN", qdyc, qxc))
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


def oracle_fp8_chain_check(Y, dX, dW, Xb, Wb, dYb, tag):
    """Y, dX, dW of an FP8 chain against the oracle's quantization and exact
    sums, within the derived bound."""
    M, K = Xb.shape
    N = Wb.shape[0]
    qx, sx = oracle.quantize_rowwise_fp8(Xb)
    qw, sw = oracle.quantize_rowwise_fp8(Wb)
    y, _, ad = oracle.fp8_scaled_mm(oracle.NT, qx, sx, qw, sw, want_acc=True)
    within_bound(Y, y, ad, np.abs(sx[:, None] * sw[None, :]).astype(np.float64), K, f"{tag} Y",
                 group_term("NT", qx, qw))
    qdy, sdy = oracle.quantize_rowwise_fp8(dYb)
    qwc, swc = oracle.quantize_colwise_fp8(Wb)
    y, _, ad = oracle.fp8_scaled_mm(oracle.NN, qdy, sdy, qwc, swc, want_acc=True)
    within_bound(dX, y, ad, np.abs(sdy[:, None] * swc[None, :]).astype(np.float64), N, f"{tag} dX",
                 group_term("NN", qdy, qwc))
    qdyc, sdyc = oracle.quantize_colwise_fp8(dYb)
    qxc, sxc = oracle.quantize_colwise_fp8(Xb)
    y, _, ad = oracle.fp8_scaled_mm(oracle.TN, qdyc, sdyc, qxc, sxc, want_acc=True)
    within_bound(dW, y, ad, np.abs(sdyc[:, None] * sxc[None, :]).astype(np.float64), M, f"{tag} dW",
                 group_term("TN", qdyc, qxc))


# The chains that hand X's and W's column maxima from the forward to the
# backward: the paired launches (X and W rows; dY rows with W columns, dY
# rows of 4 or 8 chunks per lane, whole and ragged; dY and X columns), the
# maxima folded in the GEMMs, rows over 14336 elements (the forward's maxima
# then from a pass of their own), contractions that are not multiples of 16
# (general GEMM kernel).  Outputs equal the plain chains' byte for byte, the
# maxima equal the oracle's, and the outputs are within the bound of the
# oracle's exact sums.
@pytest.mark.parametrize("M,N,K", [(300, 264, 1024), (136, 2048, 1024), (64, 3000, 512), (96, 4096, 520),
                                   (40, 24, 15000), (33, 40, 40), (1, 1032, 4104)])
def test_linear_chains_fp8_with_column_maxima(M, N, K):
    t = linear_inputs(LinearShape("fp8_colmax", M, N, K), seed=M + N + K, device="cuda")
    X, W, dY = t["X"], t["W"], t["dY"]
    Xb, Wb, dYb = tensor_bits(X), tensor_bits(W), tensor_bits(dY)
    Y, cx, cw = i8.linear_fwd_fp8_colmax(X, W)
    dX, dW = i8.linear_bwd_fp8(dY, X, W, colmax_x=cx, colmax_w=cw)
    Y0 = i8.linear_fwd_fp8(X, W)
    dX0, dW0 = i8.linear_bwd_fp8(dY, X, W)
    torch.cuda.synchronize()
    same_f32(cx, oracle.col_absmax(Xb), "colmax X")
    same_f32(cw, oracle.col_absmax(Wb), "colmax W")
    for got, want, what in ((Y, Y0, "Y"), (dX, dX0, "dX"), (dW, dW0, "dW")):
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{what} differs from the plain chain's"
    oracle_fp8_chain_check(tensor_bits(Y), tensor_bits(dX), tensor_bits(dW), Xb, Wb, dYb, f"colmax chain {M}x{N}x{K}")


# Few output tiles and a long contraction: the chain GEMM sums its
# contraction in slices into fp32 planes (forward at 256 x 256 x 8192,
# grad-input at 256 x 8192 x 256, grad-weight at 8192 x 256 x 256), plain and
# with column maxima (the same bytes), within the bound of the exact sums.
@pytest.mark.parametrize("M,N,K", [(256, 256, 8192), (256, 8192, 256), (8192, 256, 256)])
def test_linear_chains_fp8_contraction_split(M, N, K):
    t = linear_inputs(LinearShape("fp8_split", M, N, K), seed=7, device="cuda")
    X, W, dY = t["X"], t["W"], t["dY"]
    Xb, Wb, dYb = tensor_bits(X), tensor_bits(W), tensor_bits(dY)
    Y, cx, cw = i8.linear_fwd_fp8_colmax(X, W)
    dX, dW = i8.linear_bwd_fp8(dY, X, W, colmax_x=cx, colmax_w=cw)
    Y0 = i8.linear_fwd_fp8(X, W)
    dX0, dW0 = i8.linear_bwd_fp8(dY, X, W)
    torch.cuda.synchronize()
    for got, want, what in ((Y, Y0, "Y"), (dX, dX0, "dX"), (dW, dW0, "dW")):
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{what}: column-maxima chain differs"
    oracle_fp8_chain_check(tensor_bits(Y), tensor_bits(dX), tensor_bits(dW), Xb, Wb, dYb, f"split chain {M}x{N}x{K}")


def test_fp8_group_truncation_rule():
    """The summation property the FP8 bound rests on, on constructed operands
    (one 64-deep instruction; every expected sum is exact in fp32): a product
    in the group of 8 contraction indices of a larger product is truncated
    toward zero to a multiple of 2^(E_g - 13), E_g = e(a) + e(b) of the
    group's largest (e of a subnormal: -6); in another group it is exact."""
    cases = [  # ([(position, a, b)], expected fp32 sum)
        ([(0, 16.0, 16.0), (7, 2.0**-5, 1.0)], 256 + 2.0**-5),   # 2^(8-13): kept
        ([(0, 16.0, 16.0), (7, 2.0**-6, 1.0)], 256.0),           # below it: lost
        ([(0, 16.0, 16.0), (8, 2.0**-6, 1.0)], 256 + 2.0**-6),   # next group: exact
        ([(0, 30.0, 30.0), (3, 2.0**-5, 1.0)], 900 + 2.0**-5),   # E = 4 + 4, not floor(log2 900) = 9
        ([(0, 30.0, 30.0), (3, 2.0**-6, 1.0)], 900.0),
        ([(0, 2.0**-9, 448.0), (3, 2.0**-6, 2.0**-5)], 0.875 + 2.0**-11),  # subnormal a: E = -6 + 8
        ([(0, 2.0**-9, 448.0), (3, 2.0**-6, 2.0**-6)], 0.875),
        ([(0, 16.0, 16.0), (2, 1.875 * 2.0**-2, 1.875 * 2.0**-2)], 256 + 7 * 2.0**-5),   # 0.2197 -> 0.21875
        ([(0, 16.0, 16.0), (2, -1.875 * 2.0**-2, 1.875 * 2.0**-2)], 256 - 7 * 2.0**-5),  # toward zero
    ]
    n, K = len(cases), 64
    A = np.zeros((n, K), np.float32)
    B = np.zeros((n, K), np.float32)
    for i, (entries, _) in enumerate(cases):
        for pos, x, y in entries:
            A[i, pos], B[i, pos] = x, y
    Ac, Bc = oracle.float_to_e4m3(A.ravel()).reshape(n, K), oracle.float_to_e4m3(B.ravel()).reshape(n, K)
    assert np.array_equal(decode(Ac), A) and np.array_equal(decode(Bc), B)  # exactly representable
    pad = lambda v: padded_copy(torch.from_numpy(v).cuda(), round_up(K, 16) + 16)  # noqa: E731
    got = np.diag(i8.fp8_mm_f32("NT", pad(Ac), pad(Bc)).cpu().numpy())
    want = np.array([w for _, w in cases], np.float32)
    assert np.array_equal(got, want), list(zip(got.tolist(), want.tolist()))


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
    bound = 7 * 2.0**-13 * group_term("NT", A, B) + -(-K // 64) * 2.0**-21 * absdot
    err = np.abs(got - exact)
    print(f"[fp8 bound] raw sums K={K}: max |error| / bound = {float((err / bound).max()):.4f}, "
          f"exact: {float(np.mean(err == 0)):.4f}")
    assert (err <= bound).all()


def test_fp8_chains_4096_equal_primitives():
    """The FP8 chains at M = N = K = 4096: every quantized operand against the
    oracle in full, and Y, dX, dW byte for byte, in full, against the public
    FP8 GEMM on the public quantize passes' codes (whose outputs are checked
    against the oracle's exact sums within the bound above)."""
    n = 4096
    t = linear_inputs(LinearShape("fp8_4096", n, n, n), seed=4, device="cuda")
    X, W, dY = t["X"], t["W"], t["dY"]
    Y = i8.linear_fwd_fp8(X, W)
    dX, dW = i8.linear_bwd_fp8(dY, X, W)
    px, pw = i8.quantize_rowwise_fp8(X), i8.quantize_rowwise_fp8(W)
    pdy, pwc = i8.quantize_rowwise_fp8(dY), i8.quantize_colwise_fp8(W)
    pdc, pxc = i8.quantize_colwise_fp8(dY), i8.quantize_colwise_fp8(X)
    for (q, s), src, rowwise, what in ((px, X, True, "X row"), (pw, W, True, "W row"), (pdy, dY, True, "dY row"),
                                      (pwc, W, False, "W col"), (pdc, dY, False, "dY col"), (pxc, X, False, "X col")):
        qo, so = (oracle.quantize_rowwise_fp8 if rowwise else oracle.quantize_colwise_fp8)(tensor_bits(src))
        same_f32(s, so, what + " scales")
        assert np.array_equal(q.cpu().numpy(), qo), what + " codes"
    for got, want, what in ((Y, i8.fp8_scaled_mm("NT", *px, *pw), "Y"),
                            (dX, i8.fp8_scaled_mm("NN", *pdy, *pwc), "dX"),
                            (dW, i8.fp8_scaled_mm("TN", *pdc, *pxc), "dW")):
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{what} differs from the primitives"


def test_fp8_chains_on_two_streams_give_the_same_bytes():
    """The FP8 chains of two layers (the first splits its forward contraction
    into fp32 planes, added in a fixed order; the second takes the paired
    full-width row passes) run once in order on the current stream, then
    concurrently on two other streams of the default priority in the other
    order, with the workspaces refilled with junk: byte-identical outputs."""
    from workloads import LinearShape, linear_inputs
    shapes = [LinearShape("det8_a", 256, 512, 8192), LinearShape("det8_b", 1024, 768, 4096)]
    jobs = []
    for k, s in enumerate(shapes):
        t = linear_inputs(s, seed=200 + k, device="cuda")
        ws_f = torch.empty(i8.linear_workspace_bytes(s.M, s.N, s.K, False), dtype=torch.uint8, device="cuda")
        ws_b = torch.empty(i8.linear_workspace_bytes(s.M, s.N, s.K, True), dtype=torch.uint8, device="cuda")
        outs = [torch.empty((s.M, s.N), dtype=torch.bfloat16, device="cuda"),
                torch.empty((s.M, s.K), dtype=torch.bfloat16, device="cuda"),
                torch.empty((s.N, s.K), dtype=torch.bfloat16, device="cuda")]
        jobs.append((t["X"], t["W"], t["dY"], ws_f, ws_b, outs))

    def step(job):
        X, W, dY, ws_f, ws_b, (Y, dX, dW) = job
        _, cx, cw = i8.linear_fwd_fp8_colmax(X, W, out=Y, workspace=ws_f)
        i8.linear_bwd_fp8(dY, X, W, workspace=ws_b, dX=dX, dW=dW, colmax_x=cx, colmax_w=cw)

    step(jobs[0])
    step(jobs[1])
    torch.cuda.synchronize()
    ref = [[o.clone() for o in job[5]] for job in jobs]
    for job in jobs:
        for o in job[5]:
            o.fill_(0)
        job[3].fill_(0xA5)
        job[4].fill_(0x5A)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s2):
        step(jobs[1])
    with torch.cuda.stream(s1):
        step(jobs[0])
    torch.cuda.synchronize()
    for k, job in enumerate(jobs):
        for got, want, what in zip(job[5], ref[k], ("Y", "dX", "dW")):
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"layer {k} {what}"
