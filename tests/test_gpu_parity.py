"""GPU parity: the HIP path through the C ABI against the CPU oracle, element
by element.  int8 codes, fp32 scales, Philox words and int32 accumulators
must match bit for bit; bf16 outputs must match bit for bit as well (the
tolerance the method allows is 1 bf16 ulp; the fixed epilogue order makes
them identical, and the tests report the ulp distance if they ever are not).

Sizes span several tiles with ragged tails, leading dimensions are padded,
and canary bytes around every output row catch writes outside the rows."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import (bits_to_bf16, canary_intact, padded, padded_copy, random_codes,
                            round_up, special_rows_bf16, tensor_bits)

pytestmark = pytest.mark.gpu

i8 = pytest.importorskip("int8_mixed_precision_rowwise_amd")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

ROUNDINGS = [("rne", oracle.RNE), ("sr", oracle.SR)]


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> int:
    """Largest distance in bf16 ulps (ordered integer encoding) between two bit arrays."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + x)
    return int(np.abs(ordered(a) - ordered(b)).max()) if a.size else 0


def assert_bf16_equal(got: np.ndarray, want: np.ndarray, what: str):
    if not np.array_equal(got, want):
        d = bf16_ulp_distance(got, want)
        n = int(np.count_nonzero(got != want))
        raise AssertionError(f"{what}: {n} of {got.size} bf16 outputs differ, max {d} ulp")


# --------------------------------------------------------------------------- Philox


@pytest.mark.parametrize("seed,offset", [(0, 0), (1, 3), (2**32 + 7, 2**32 - 5),
                                         (0xFEDCBA9876543210, 2**40 * 5 + 11)])
def test_philox_words(seed, offset):
    n = 1000
    got = i8.philox4x32_10(seed, offset, n).cpu().numpy().view(np.uint32)
    want = oracle.philox_stream(seed, offset, n)
    assert np.array_equal(got, want)


# --------------------------------------------------------------------------- quantization

ROW_SHAPES = [(1, 1), (3, 17), (5, 255), (7, 513), (64, 2048), (9, 5000), (6, 5632), (4, 8192),
              (5, 14336), (3, 16385), (2, 30001), (2, 128256), (33, 7001), (70, 8191),
              (20, 9000), (11, 12290)]


@pytest.mark.parametrize("rounding,rc", ROUNDINGS)
@pytest.mark.parametrize("rows,cols", ROW_SHAPES)
def test_quantize_rowwise(rounding, rc, rows, cols):
    rng = np.random.default_rng(rows * 100003 + cols)
    xb = special_rows_bf16(rng, rows, cols)
    ldx = round_up(cols, 8) + 8
    x = padded_copy(bits_to_bf16(xb), ldx)
    qs, q = padded(rows, cols, round_up(cols, 16) + 16, torch.int8)
    seed, off = 77, 2**40 + 3
    _, s = i8.quantize_rowwise(x, rounding, seed, off, q=q)
    torch.cuda.synchronize()
    qo, so = oracle.quantize_rowwise(xb, rc, seed, off)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), qo)
    assert canary_intact(qs, cols)


COL_SHAPES = [(1, 1), (17, 3), (255, 5), (513, 7), (2048, 64), (1000, 513), (33, 1030),
              (4096, 40), (300, 5632)]


@pytest.mark.parametrize("rounding,rc", ROUNDINGS)
@pytest.mark.parametrize("rows,cols", COL_SHAPES)
def test_quantize_colwise(rounding, rc, rows, cols):
    rng = np.random.default_rng(rows * 7919 + cols)
    xb = np.ascontiguousarray(special_rows_bf16(rng, cols, rows).T)  # structured columns
    ldx = round_up(cols, 8) + 8
    x = padded_copy(bits_to_bf16(xb), ldx)
    qs, q = padded(rows, cols, round_up(cols, 16) + 16, torch.int8)
    seed, off = 5, 123456789
    _, s = i8.quantize_colwise(x, rounding, seed, off, q=q)
    torch.cuda.synchronize()
    qo, so = oracle.quantize_colwise(xb, rc, seed, off)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), qo)
    assert canary_intact(qs, cols)


def test_quantize_empty_and_zero_width():
    x = torch.zeros((0, 8), dtype=torch.bfloat16, device="cuda")
    q, s = i8.quantize_rowwise(x)
    assert q.shape == (0, 8) and s.shape == (0,)
    # zero-width rows: amax over nothing is 0, so every scale is 0
    x = torch.zeros((5, 0), dtype=torch.bfloat16, device="cuda")
    s = torch.full((5,), 7.0, device="cuda")
    i8.quantize_rowwise(x, scale=s)
    assert (s.cpu() == 0).all()
    x = torch.zeros((0, 9), dtype=torch.bfloat16, device="cuda")
    s = torch.full((9,), 7.0, device="cuda")
    i8.quantize_colwise(x, scale=s)
    assert (s.cpu() == 0).all()


# --------------------------------------------------------------------------- GEMM


def storage_shapes(layout, M, N, K):
    return {"NT": ((M, K), (N, K)), "NN": ((M, K), (K, N)), "TN": ((K, M), (K, N))}[layout]


def make_operands(layout, M, N, K, seed, pad=True):
    rng = np.random.default_rng(seed)
    (ar, ac), (br, bc) = storage_shapes(layout, M, N, K)
    A = random_codes(rng, (ar, ac))
    B = random_codes(rng, (br, bc))
    sa = (rng.random(M) * 0.02 + 1e-4).astype(np.float32)
    sb = (rng.random(N) * 0.002 + 1e-5).astype(np.float32)
    lda = round_up(ac, 16) + (16 if pad else 0)
    ldb = round_up(bc, 16) + (16 if pad else 0)
    Ag = padded_copy(torch.from_numpy(A).cuda(), lda)
    Bg = padded_copy(torch.from_numpy(B).cuda(), ldb)
    return A, B, sa, sb, Ag, Bg


# the contraction a multiple of 16 with ragged output extents, down to one
# row or column, takes the pipelined kernel (or, for extents that are not a
# multiple of 4 along an operand read down its rows, the general one)
GEMM_SHAPES = [(1, 1, 1), (17, 33, 65), (255, 130, 513), (256, 512, 512), (300, 257, 1000),
               (513, 255, 17), (129, 1025, 200), (40, 24, 4100), (1, 1, 16), (17, 33, 64),
               (5, 130, 48), (37, 36, 80), (300, 260, 1008)]


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_i32_and_scaled(layout, M, N, K):
    A, B, sa, sb, Ag, Bg = make_operands(layout, M, N, K, seed=M * 31 + N * 7 + K)
    L = oracle.LAYOUTS[layout]
    cs, C = padded(M, N, round_up(N, 4) + 4, torch.int32)
    i8.int8_mm_i32(layout, Ag, Bg, out=C)
    ys, Y = padded(M, N, N + 3, torch.bfloat16)
    i8.int8_scaled_mm(layout, Ag, torch.from_numpy(sa).cuda(), Bg, torch.from_numpy(sb).cuda(), out=Y)
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy(), oracle.mm_i32(L, A, B))
    assert_bf16_equal(tensor_bits(Y), oracle.scaled_mm(L, A, sa, B, sb), f"{layout} {M}x{N}x{K}")
    assert canary_intact(cs, N) and canary_intact(ys, N)


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_gemm_1024_full(layout):
    n = 1024
    A, B, sa, sb, Ag, Bg = make_operands(layout, n, n, n, seed=1024, pad=False)
    Y = i8.int8_scaled_mm(layout, Ag, torch.from_numpy(sa).cuda(), Bg, torch.from_numpy(sb).cuda())
    torch.cuda.synchronize()
    assert_bf16_equal(tensor_bits(Y), oracle.scaled_mm(oracle.LAYOUTS[layout], A, sa, B, sb), layout)


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
@pytest.mark.parametrize("n", [2048, 4096])
def test_gemm_square_sampled(layout, n):
    """Full-size square GEMMs in the benchmarked launch configuration, checked on
    sampled outputs plus one whole 32-row band of int32 accumulators."""
    A, B, sa, sb, Ag, Bg = make_operands(layout, n, n, n, seed=n, pad=False)
    L = oracle.LAYOUTS[layout]
    Y = i8.int8_scaled_mm(layout, Ag, torch.from_numpy(sa).cuda(), Bg, torch.from_numpy(sb).cuda())
    C = i8.int8_mm_i32(layout, Ag, Bg)
    torch.cuda.synchronize()
    rng = np.random.default_rng(n + 1)
    ms = rng.integers(0, n, size=4096)
    ns = rng.integers(0, n, size=4096)
    acc, y = oracle.scaled_mm_at(L, A, sa, B, sb, ms, ns)
    Yb = tensor_bits(Y)
    Cn = C.cpu().numpy()
    assert np.array_equal(Cn[ms, ns], acc)
    assert_bf16_equal(Yb[ms, ns], y, f"{layout} {n}^3 sampled")
    band = slice(n - 32, n)
    bm = np.repeat(np.arange(n - 32, n), n)
    bn = np.tile(np.arange(n), 32)
    acc_b, y_b = oracle.scaled_mm_at(L, A, sa, B, sb, bm, bn)
    assert np.array_equal(Cn[band].ravel(), acc_b)
    assert_bf16_equal(Yb[band].ravel(), y_b, f"{layout} {n}^3 last band")


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_gemm_int32_headroom_worst_case(layout):
    """All codes +127 (and -127 against +127) at the longest contraction the
    Llama-3-8B LM head needs, K = 128256: |acc| = 2,068,641,024, inside int32."""
    M, N, K = 48, 80, 128256
    (ar, ac), (br, bc) = storage_shapes(layout, M, N, K)
    Ag = torch.full((ar, ac), 127, dtype=torch.int8, device="cuda")
    Bg = torch.full((br, bc), 127, dtype=torch.int8, device="cuda")
    if layout == "NT":
        Bg[: N // 2] = -127
    else:
        Bg[:, : N // 2] = -127
    C = i8.int8_mm_i32(layout, Ag, Bg).cpu().numpy().astype(np.int64)
    assert (C[:, : N // 2] == -2068641024).all() and (C[:, N // 2:] == 2068641024).all()


def test_gemm_k_zero_writes_zeros():
    Ag = torch.zeros((5, 0), dtype=torch.int8, device="cuda")
    Bg = torch.zeros((7, 0), dtype=torch.int8, device="cuda")
    Y = torch.full((5, 7), 3.0, dtype=torch.bfloat16, device="cuda")
    i8.int8_scaled_mm("NT", Ag, torch.ones(5, device="cuda"), Bg, torch.ones(7, device="cuda"), out=Y)
    assert (Y.float().cpu() == 0).all()


def test_gemm_contraction_bound_is_enforced():
    Ag = torch.zeros((1, 133152), dtype=torch.int8, device="cuda")[:, :133145]
    with pytest.raises(i8.I8mpError) as e:
        i8.int8_mm_i32("NT", Ag, Ag)
    assert e.value.status == 2


# --------------------------------------------------------------------------- linear layer


@pytest.mark.parametrize("rounding,rc", ROUNDINGS)
def test_linear_single_layer_full(rounding, rc):
    """X [256, 512] ~ N(0,1) with outlier channels, W [512, 512] ~ N(0, 0.02),
    dY ~ N(0, 1e-3): forward and both backward GEMMs, every output."""
    from workloads import bf16_bits, linear_inputs, single_linear
    t = linear_inputs(single_linear(), seed=0)
    X, W, dY = (t[k].cuda() for k in ("X", "W", "dY"))
    seed, off = 42, 2**20
    Y = i8.linear_fwd(X, W, rounding, seed, off)
    dX, dW = i8.linear_bwd(dY, X, W, rounding, seed, off)
    torch.cuda.synchronize()
    Xb, Wb, dYb = (bf16_bits(t[k]) for k in ("X", "W", "dY"))
    assert_bf16_equal(tensor_bits(Y), oracle.linear_fwd(Xb, Wb, rc, seed, off), "Y")
    dXo, dWo = oracle.linear_bwd(dYb, Xb, Wb, rc, seed, off)
    assert_bf16_equal(tensor_bits(dX), dXo, "dX")
    assert_bf16_equal(tensor_bits(dW), dWo, "dW")
    # either gradient alone gives the same values
    dX2, none = i8.linear_bwd(dY, X, W, rounding, seed, off, want_dw=False)
    none2, dW2 = i8.linear_bwd(dY, X, W, rounding, seed, off, want_dx=False)
    assert none is None and none2 is None
    assert torch.equal(dX2, dX) and torch.equal(dW2, dW)


# (300, 264, 4096): the forward GEMM splits its contraction in four;
# (300, 4096, 264): the grad-input GEMM does; (4112, 200, 296): the
# grad-weight GEMM splits its 4112 tokens in four (3 x 1088 + 848).
@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (17, 24, 40), (130, 264, 72), (1000, 8, 520),
                                   (300, 264, 4096), (300, 4096, 264), (4112, 200, 296)])
def test_linear_ragged(M, N, K):
    from workloads import LinearShape, bf16_bits, linear_inputs
    t = linear_inputs(LinearShape("ragged", M, N, K), seed=M + N + K)
    X, W, dY = (t[k].cuda() for k in ("X", "W", "dY"))
    Y = i8.linear_fwd(X, W, "sr", 3, 9)
    dX, dW = i8.linear_bwd(dY, X, W, "sr", 3, 9)
    torch.cuda.synchronize()
    Xb, Wb, dYb = (bf16_bits(t[k]) for k in ("X", "W", "dY"))
    assert_bf16_equal(tensor_bits(Y), oracle.linear_fwd(Xb, Wb, oracle.SR, 3, 9), "Y")
    dXo, dWo = oracle.linear_bwd(dYb, Xb, Wb, oracle.SR, 3, 9)
    assert_bf16_equal(tensor_bits(dX), dXo, "dX")
    assert_bf16_equal(tensor_bits(dW), dWo, "dW")


# Ragged chains with the column maxima handed from forward to backward (the
# paired and fused quantize launches), against the oracle in full: forward
# splits (few tiles, contraction 4496 / 8816), grad-input splits (dY 5968 /
# 8352 wide), grad-weight splits (5744 / 2384 tokens), both roundings.
@pytest.mark.parametrize("M,N,K,rounding", [(144, 64, 4496, "rne"), (208, 32, 8816, "sr"),
                                            (205, 5968, 152, "sr"), (114, 8352, 256, "rne"),
                                            (5744, 64, 16, "rne"), (2384, 120, 208, "sr")])
def test_linear_chains_with_maxima_ragged_splits(M, N, K, rounding):
    from workloads import LinearShape, bf16_bits, linear_inputs
    rc = oracle.SR if rounding == "sr" else oracle.RNE
    t = linear_inputs(LinearShape("ragged_split", M, N, K), seed=M + N + K, device="cuda")
    X, W, dY = t["X"], t["W"], t["dY"]
    off = 7 << 44
    Y, cx, cw = i8.linear_fwd_colmax(X, W, rounding, 11, off)
    dX, dW = i8.linear_bwd(dY, X, W, rounding, 11, off, colmax_x=cx, colmax_w=cw)
    torch.cuda.synchronize()
    Xb, Wb, dYb = tensor_bits(X), tensor_bits(W), tensor_bits(dY)
    assert_bf16_equal(tensor_bits(Y), oracle.linear_fwd(Xb, Wb, rc, 11, off), "Y")
    dXo, dWo = oracle.linear_bwd(dYb, Xb, Wb, rc, 11, off)
    assert_bf16_equal(tensor_bits(dX), dXo, "dX")
    assert_bf16_equal(tensor_bits(dW), dWo, "dW")


@pytest.mark.parametrize("M,N,K", [(300, 264, 4096), (4112, 200, 296), (2048, 256, 32768),
                                   (1024, 8192, 1024)])
def test_contraction_split_equals_unsplit_gemm(M, N, K):
    """The linear chains split the contraction of few-tile GEMMs into int32
    partial planes; their outputs equal the public unsplit GEMM's on the same
    codes, bit for bit."""
    from workloads import LinearShape, linear_inputs
    t = linear_inputs(LinearShape("split", M, N, K), seed=5, device="cuda")
    X, W, dY = t["X"], t["W"], t["dY"]
    Y = i8.linear_fwd(X, W, "rne")
    dX, dW = i8.linear_bwd(dY, X, W, "rne")
    qx, sx = i8.quantize_rowwise(X)
    qw, sw = i8.quantize_rowwise(W)
    qdy, sdy = i8.quantize_rowwise(dY)
    qwc, swc = i8.quantize_colwise(W)
    qdyc, sdyc = i8.quantize_colwise(dY)
    qxc, sxc = i8.quantize_colwise(X)
    for got, want, what in ((Y, i8.int8_scaled_mm("NT", qx, sx, qw, sw), "Y"),
                            (dX, i8.int8_scaled_mm("NN", qdy, sdy, qwc, swc), "dX"),
                            (dW, i8.int8_scaled_mm("TN", qdyc, sdyc, qxc, sxc), "dW")):
        torch.cuda.synchronize()
        assert_bf16_equal(tensor_bits(got), tensor_bits(want), f"{what} {M}x{N}x{K}")


def test_repeat_runs_are_byte_identical():
    from workloads import linear_inputs, square
    t = linear_inputs(square(1024), seed=3)
    X, W, dY = (t[k].cuda() for k in ("X", "W", "dY"))
    outs = []
    for _ in range(3):
        Y = i8.linear_fwd(X, W, "sr", 1, 2)
        dX, dW = i8.linear_bwd(dY, X, W, "sr", 1, 2)
        outs.append((Y, dX, dW))
    torch.cuda.synchronize()
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_two_streams_and_reordered_launches_give_the_same_bytes():
    """Two layers' training steps (stochastic rounding; the first splits its
    forward contraction, the second takes the paired full-width row passes)
    run once on the current stream in order A then B, then again concurrently
    on two other streams of the default priority, B's launches first: every
    output is byte-identical (no kernel depends on timing, launch order or
    what a previous call left in a workspace)."""
    from workloads import LinearShape, linear_inputs
    shapes = [LinearShape("det_a", 256, 512, 8192), LinearShape("det_b", 1024, 768, 4096)]
    jobs = []
    for k, s in enumerate(shapes):
        t = linear_inputs(s, seed=100 + k, device="cuda")
        ws_f = torch.empty(i8.linear_workspace_bytes(s.M, s.N, s.K, False), dtype=torch.uint8, device="cuda")
        ws_b = torch.empty(i8.linear_workspace_bytes(s.M, s.N, s.K, True), dtype=torch.uint8, device="cuda")
        outs = [torch.empty((s.M, s.N), dtype=torch.bfloat16, device="cuda"),
                torch.empty((s.M, s.K), dtype=torch.bfloat16, device="cuda"),
                torch.empty((s.N, s.K), dtype=torch.bfloat16, device="cuda")]
        jobs.append((t["X"], t["W"], t["dY"], ws_f, ws_b, outs))

    def step(job, seed):
        X, W, dY, ws_f, ws_b, (Y, dX, dW) = job
        _, cx, cw = i8.linear_fwd_colmax(X, W, "sr", seed, 5 << 44, out=Y, workspace=ws_f)
        i8.linear_bwd(dY, X, W, "sr", seed, 5 << 44, dX=dX, dW=dW, workspace=ws_b, colmax_x=cx, colmax_w=cw)

    step(jobs[0], 1)
    step(jobs[1], 2)
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
        step(jobs[1], 2)
    with torch.cuda.stream(s1):
        step(jobs[0], 1)
    torch.cuda.synchronize()
    for k, job in enumerate(jobs):
        for got, want, what in zip(job[5], ref[k], ("Y", "dX", "dW")):
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"layer {k} {what}"
