"""GPU parity at the full sizes of the benchmarked and named workloads.

* Every quantized operand (codes and scales) is compared with the CPU oracle
  in full, bit for bit.
* GEMM outputs of the library's linear forward / backward are compared on
  sampled positions plus whole bands of rows, bit for bit, against the
  oracle's scaled matmul of the oracle's own quantized operands, and in full,
  byte for byte, against the public scaled GEMM applied to the public
  quantize passes' codes (which are oracle-checked in full): the chains'
  own kernels (paired and split launches, the column maxima reduced in a
  GEMM's prologue) reproduce every output of the primitives.
* Stochastic rounding is additionally checked for unbiasedness over 256
  seeds on a [64, 64] slice, on the GPU's own draws.
* The quotient x / s the kernels evaluate is checked exhaustively: every
  finite bf16 value against every positive finite bf16 absmax.

Inputs are seeded synthetic tensors with the layer shapes and distributions
of the source pages' runs (see workloads.py); they are drawn on the GPU and
copied to the host for the oracle.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import tensor_bits
from workloads import linear_inputs, llama3_8b_layers, llama_1b_layers, square

pytestmark = pytest.mark.gpu

i8 = pytest.importorskip("int8_mixed_precision_rowwise_amd")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

THREADS = min(16, len(os.sched_getaffinity(0)))
RC = {"rne": oracle.RNE, "sr": oracle.SR}


def oracle_rowwise(xb, rounding, seed, offset):
    """The oracle's row-wise quantization, split over row bands in threads (rows
    are independent; a band starting at row r0 draws from offset + r0*cols/4)."""
    rows, cols = xb.shape
    if rows * cols < 1 << 22 or cols % 4:
        return oracle.quantize_rowwise(xb, RC[rounding], seed, offset)
    q = np.empty((rows, cols), np.int8)
    s = np.empty(rows, np.float32)
    step = -(-rows // THREADS)

    def work(r0):
        r1 = min(rows, r0 + step)
        qq, ss = oracle.quantize_rowwise(xb[r0:r1], RC[rounding], seed, offset + r0 * cols // 4)
        q[r0:r1], s[r0:r1] = qq, ss

    with cf.ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(work, range(0, rows, step)))
    return q, s


def oracle_colwise(xb, rounding, seed, offset):
    """The oracle's column-wise quantization; under RNE split over column bands
    (columns are independent), under SR in one call (draws index the whole row)."""
    rows, cols = xb.shape
    if rounding == "sr" or rows * cols < 1 << 22:
        return oracle.quantize_colwise(xb, RC[rounding], seed, offset)
    q = np.empty((rows, cols), np.int8)
    s = np.empty(cols, np.float32)
    step = -(-cols // THREADS)

    def work(c0):
        c1 = min(cols, c0 + step)
        qq, ss = oracle.quantize_colwise(xb[:, c0:c1], RC[rounding], seed, offset)
        q[:, c0:c1], s[c0:c1] = qq, ss

    with cf.ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(work, range(0, cols, step)))
    return q, s


def check_quant(got, want, what):
    q, s = got
    qo, so = want
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32)), f"{what}: scales"
    qn = q.cpu().numpy()
    if not np.array_equal(qn, qo):
        bad = np.argwhere(qn != qo)
        raise AssertionError(f"{what}: {len(bad)} codes differ, first at {bad[0].tolist()}")


def sampled_positions(M, N, K, rng):
    """4096 random outputs plus whole rows at both ends, sized so the oracle's
    exact dot products stay near 2^29 multiply-adds."""
    budget = 1 << 29
    n = max(256, min(4096, budget // K))
    band = max(1, min(16, budget // (2 * N * K)))
    ms = rng.integers(0, M, size=n)
    ns = rng.integers(0, N, size=n)
    rows = np.concatenate([np.arange(min(band, M)), np.arange(max(0, M - band), M)])
    bm = np.repeat(rows, N)
    bn = np.tile(np.arange(N), len(rows))
    return np.concatenate([ms, bm]), np.concatenate([ns, bn])


def check_gemm(layout, Y, qa, sa, qb, sb, rng, what):
    M, N = Y.shape
    K = qa.shape[1] if layout in ("NT", "NN") else qa.shape[0]
    ms, ns = sampled_positions(M, N, K, rng)
    _, y = oracle.scaled_mm_at(oracle.LAYOUTS[layout], qa, sa, qb, sb, ms, ns)
    got = tensor_bits(Y)[ms, ns]
    if not np.array_equal(got, y):
        bad = int(np.count_nonzero(got != y))
        raise AssertionError(f"{what}: {bad} of {len(ms)} sampled bf16 outputs differ")


def same_in_full(chain_out, prim_out, what):
    """The chain's bf16 output against the public GEMM's on the public codes,
    every element, on the GPU."""
    eq = chain_out.view(torch.int16) == prim_out.view(torch.int16)
    if not bool(eq.all()):
        bad = torch.nonzero(~eq)
        raise AssertionError(f"{what}: {bad.shape[0]} of {eq.numel()} outputs differ from the public "
                             f"GEMM on the public codes, first at {bad[0].tolist()}")


def run_layer(shape, rounding, seed=0, offset=0, gemms=("fwd", "dgrad", "wgrad"), colmax=False):
    """All quantized operands in full, the GEMM outputs against the oracle on
    samples and against the public GEMM on the public codes in full.  With
    colmax, the forward also returns X's and W's column maxima (checked in
    full) and the backward takes them."""
    t = linear_inputs(shape, seed=0, device="cuda")
    X, W, dY = t["X"], t["W"], t["dY"]
    Xb, Wb, dYb = tensor_bits(X), tensor_bits(W), tensor_bits(dY)
    rng = np.random.default_rng(shape.M + shape.N + shape.K)
    po = lambda j: offset + (j << 40)  # noqa: E731
    name = f"{shape.name} {rounding}"
    if "fwd" in gemms:
        ox = oracle_rowwise(Xb, rounding, seed, po(0))
        ow = oracle_rowwise(Wb, rounding, seed, po(1))
        px, pw = i8.quantize_rowwise(X, rounding, seed, po(0)), i8.quantize_rowwise(W, rounding, seed, po(1))
        check_quant(px, ox, name + " X row")
        check_quant(pw, ow, name + " W row")
        cx = cw = None
        if colmax:
            Y, cx, cw = i8.linear_fwd_colmax(X, W, rounding, seed, offset)
            for got, src, what in ((cx, Xb, " colmax X"), (cw, Wb, " colmax W")):
                assert np.array_equal(got.cpu().numpy().view(np.uint32),
                                      oracle.col_absmax(src).view(np.uint32)), name + what
        else:
            Y = i8.linear_fwd(X, W, rounding, seed, offset)
        check_gemm("NT", Y, ox[0], ox[1], ow[0], ow[1], rng, name + " Y")
        same_in_full(Y, i8.int8_scaled_mm("NT", px[0], px[1], pw[0], pw[1]), name + " Y")
        del Y, ox, ow, px, pw
    else:
        cx = cw = None
    dX, dW = i8.linear_bwd(dY, X, W, rounding, seed, offset,
                           want_dx="dgrad" in gemms, want_dw="wgrad" in gemms,
                           colmax_x=cx, colmax_w=cw)
    if "dgrad" in gemms:
        ody = oracle_rowwise(dYb, rounding, seed, po(2))
        owc = oracle_colwise(Wb, rounding, seed, po(3))
        pdy, pwc = i8.quantize_rowwise(dY, rounding, seed, po(2)), i8.quantize_colwise(W, rounding, seed, po(3))
        check_quant(pdy, ody, name + " dY row")
        check_quant(pwc, owc, name + " W col")
        check_gemm("NN", dX, ody[0], ody[1], owc[0], owc[1], rng, name + " dX")
        same_in_full(dX, i8.int8_scaled_mm("NN", pdy[0], pdy[1], pwc[0], pwc[1]), name + " dX")
        del ody, owc, pdy, pwc
    if "wgrad" in gemms:
        odc = oracle_colwise(dYb, rounding, seed, po(4))
        oxc = oracle_colwise(Xb, rounding, seed, po(5))
        pdc, pxc = i8.quantize_colwise(dY, rounding, seed, po(4)), i8.quantize_colwise(X, rounding, seed, po(5))
        check_quant(pdc, odc, name + " dY col")
        check_quant(pxc, oxc, name + " X col")
        check_gemm("TN", dW, odc[0], odc[1], oxc[0], oxc[1], rng, name + " dW")
        same_in_full(dW, i8.int8_scaled_mm("TN", pdc[0], pdc[1], pxc[0], pxc[1]), name + " dW")
    torch.cuda.empty_cache()


@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_square_4096_step(rounding):
    """The benchmarked workload: one linear step at M = N = K = 4096."""
    run_layer(square(4096), rounding, seed=1234)


@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_square_4096_step_with_column_maxima(rounding):
    """The benchmarked step through the chains that hand X's and W's column
    maxima from forward to backward."""
    run_layer(square(4096), rounding, seed=99, colmax=True)


@pytest.mark.parametrize("rounding", ["rne", "sr"])
@pytest.mark.parametrize("M,N,K", [(1024, 1024, 8192), (1024, 8192, 1024), (2048, 2048, 2048)])
def test_step_contraction_split(rounding, M, N, K):
    """Chains whose forward (1024 x 1024 outputs, contraction 8192) or
    grad-input GEMM (contraction 8192) splits its contraction eight ways into
    int32 partial planes, and 2048^3, which runs unsplit on 128 x 128 tiles."""
    from workloads import LinearShape
    run_layer(LinearShape(f"split_{M}x{N}x{K}", M, N, K), rounding, seed=7, offset=3, colmax=True)


@pytest.mark.parametrize("layer", ["llama1b_down_proj", "llama1b_gate_proj", "llama1b_k_proj"])
def test_llama1b_layer_with_column_maxima(layer):
    """Llama-1B linears at 32768 tokens (5632-wide rows of X, resp. dY) through
    the column-maxima chains."""
    shape = next(s for s in llama_1b_layers() if s.name == layer)
    run_layer(shape, "rne", colmax=True)


@pytest.mark.parametrize("layer", [s.name for s in llama_1b_layers()])
def test_llama1b_layer_rne(layer):
    """Llama-style 1B decoder linears at 16 x 2048 = 32768 tokens, RNE."""
    shape = next(s for s in llama_1b_layers() if s.name == layer)
    run_layer(shape, "rne")


@pytest.mark.parametrize("layer", [s.name for s in llama_1b_layers()])
def test_llama1b_layer_sr(layer):
    """The same layers with stochastic rounding in every quantize pass."""
    shape = next(s for s in llama_1b_layers() if s.name == layer)
    run_layer(shape, "sr", seed=7, offset=3)


def test_sr_unbiased_over_256_seeds_on_gpu():
    """GPU stochastic rounding: mean code over seeds 0..255 equals x/s on a
    [64, 64] slice (row-wise over full 2048-wide rows of Llama-1B activations,
    column-wise over all 32768 rows of its output gradients)."""
    shape = next(s for s in llama_1b_layers() if s.name == "llama1b_q_proj")
    t = linear_inputs(shape, seed=0, device="cuda")
    X = t["X"][:64]
    dY = t["dY"]
    acc_r = torch.zeros((64, 64), dtype=torch.float64, device="cuda")
    acc_c = torch.zeros((64, 64), dtype=torch.float64, device="cuda")
    for seed in range(256):
        q, s_r = i8.quantize_rowwise(X, "sr", seed, 0)
        acc_r += q[:, :64].double()
        qc, s_c = i8.quantize_colwise(dY[:, :64].contiguous(), "sr", seed, 0)
        acc_c += qc[:64].double()
    for acc, v in ((acc_r, X[:, :64].double() / s_r.double()[:, None]),
                   (acc_c, dY[:64, :64].double() / s_c.double()[None, :])):
        mean = (acc / 256).cpu().numpy()
        v = v.cpu().numpy()
        f = v - np.floor(v)
        sd = np.sqrt(f * (1 - f) / 256)
        assert (np.abs(mean - v) <= 5 * sd + 2.0**-16).all()
        z = (acc.cpu().numpy() - 256 * v).sum() / np.sqrt(256 * (f * (1 - f)).sum())
        assert abs(z) < 5


@pytest.mark.parametrize("layer", [s.name for s in llama3_8b_layers()])
def test_llama3_8b_layer_rne(layer):
    """Llama-3-8B-shaped linears at 8192 tokens, including the 128256-wide LM
    head (grad-input contraction 128256, inside the int32 bound)."""
    shape = next(s for s in llama3_8b_layers() if s.name == layer)
    run_layer(shape, "rne")


@pytest.mark.parametrize("layer", ["llama3_8b_gate_proj", "llama3_8b_down_proj"])
def test_llama3_8b_layer_sr_with_column_maxima(layer):
    """Stochastic rounding on 14336-wide rows (dY of gate_proj; X and W of
    down_proj): the plain row passes take the block-per-row kernel and the
    chains' row passes with column maxima the banded two-read kernels, since
    the row with its uniforms no longer fits one wave's registers."""
    shape = next(s for s in llama3_8b_layers() if s.name == layer)
    run_layer(shape, "sr", seed=11, offset=5, colmax=True)


def test_llama3_8b_lm_head_with_column_maxima():
    """The LM head [4096 -> 128256] at 8192 tokens through the column-maxima
    chains: dY's 128256-wide rows take the banded two-pass row kernel, and its
    column maxima are reduced in the grad-input GEMM's prologue or launch."""
    shape = next(s for s in llama3_8b_layers() if s.name == "llama3_8b_lm_head")
    run_layer(shape, "rne", seed=5, colmax=True)


@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_quotient_exhaustive(rounding):
    """Every finite bf16 x against every positive finite bf16 absmax a, |x| <= a:
    row i holds all bf16 bit patterns b with (b & 0x7fff) <= a_i (others 0), so
    its absmax is a_i; codes must equal the oracle's (IEEE division) codes."""
    amax = np.arange(1, 0x7F80, dtype=np.uint32)  # positive finite bf16 patterns
    cols = 65536
    pats = np.arange(cols, dtype=np.uint32)
    mag = pats & 0x7FFF
    finite = mag < 0x7F80
    band = 4096
    for r0 in range(0, len(amax), band):
        a = amax[r0:r0 + band]
        keep = finite[None, :] & (mag[None, :] <= a[:, None])
        xb = np.where(keep, pats[None, :], 0).astype(np.uint16)
        xg = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
        q, s = i8.quantize_rowwise(xg, rounding, 11, r0 * cols // 4)
        qo, so = oracle_rowwise(xb, rounding, 11, r0 * cols // 4)
        assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
        qn = q.cpu().numpy()
        if not np.array_equal(qn, qo):
            bad = np.argwhere(qn != qo)[0]
            raise AssertionError(f"x bits {xb[bad[0], bad[1]]:#06x} amax bits {a[bad[0]]:#06x}: "
                                 f"gpu {qn[bad[0], bad[1]]} oracle {qo[bad[0], bad[1]]}")
        del xg, q


def test_quantize_and_gemm_past_2_31_elements():
    """Tensors of more than 2^31 elements, where any 32-bit element or byte
    index would wrap: the row pass (both roundings) and the row pass with
    column maxima plus the column pass given them (RNE) over 524289 rows of
    4096 bf16 values (4.3 GB; the last row starts at element 2^31), and an NT
    GEMM with 65536 x 32776 outputs (2.1e9) at contraction 64.  Sampled rows,
    whole 8-column slices and sampled outputs against the oracle."""
    rows, cols = 524289, 4096
    print(f"case: {rows} x {cols} quantize, 65536 x 32776 x 64 NT", flush=True)
    g = torch.Generator(device="cuda").manual_seed(31)
    x = torch.randn((rows, cols), generator=g, device="cuda", dtype=torch.bfloat16)
    sample_rows = [0, 1, 262144, 524286, 524287, 524288]
    seed, off = 29, 3 << 40
    for rounding in ("rne", "sr"):
        q, s = i8.quantize_rowwise(x, rounding, seed, off)
        torch.cuda.synchronize()
        for r in sample_rows:
            xb = tensor_bits(x[r:r + 1])
            qo, so = oracle.quantize_rowwise(xb, RC[rounding], seed, off + r * cols // 4)
            assert np.array_equal(q[r:r + 1].cpu().numpy(), qo), f"{rounding} row {r} codes"
            assert np.array_equal(s[r:r + 1].cpu().numpy().view(np.uint32), so.view(np.uint32)), f"row {r} scale"
        del q, s
    q, s, cm = i8.quantize_rowwise_colmax(x)
    q2, s2 = i8.quantize_colwise_given_colmax(x, cm)
    torch.cuda.synchronize()
    for c0 in (0, 2048, cols - 8):
        xb = tensor_bits(x[:, c0:c0 + 8])
        assert np.array_equal(cm[c0:c0 + 8].cpu().numpy().view(np.uint32),
                              oracle.col_absmax(xb).view(np.uint32)), f"column maxima at {c0}"
        qo, so = oracle.quantize_colwise(xb, oracle.RNE, 0, 0)
        assert np.array_equal(q2[:, c0:c0 + 8].cpu().numpy(), qo), f"column codes at {c0}"
        assert np.array_equal(s2[c0:c0 + 8].cpu().numpy().view(np.uint32), so.view(np.uint32)), f"scales at {c0}"
    for r in sample_rows:
        qo, so = oracle.quantize_rowwise(tensor_bits(x[r:r + 1]), oracle.RNE, 0, 0)
        assert np.array_equal(q[r:r + 1].cpu().numpy(), qo), f"row {r} codes (with maxima)"
    del x, q, s, cm, q2, s2
    torch.cuda.empty_cache()

    M, N, K = 65536, 32776, 64
    rng = np.random.default_rng(7)
    qa = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    qb = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    sa = rng.uniform(1e-3, 2e-3, size=M).astype(np.float32)
    sb = rng.uniform(1e-3, 2e-3, size=N).astype(np.float32)
    Y = i8.int8_scaled_mm("NT", torch.from_numpy(qa).cuda(), torch.from_numpy(sa).cuda(),
                          torch.from_numpy(qb).cuda(), torch.from_numpy(sb).cuda())
    torch.cuda.synchronize()
    ms = np.concatenate([rng.integers(0, M, 2048), np.arange(M - 16, M).repeat(4)])
    ns = np.concatenate([rng.integers(0, N, 2048), np.tile(np.array([0, 1, N - 2, N - 1]), 16)])
    _, y = oracle.scaled_mm_at(oracle.LAYOUTS["NT"], qa, sa, qb, sb, ms, ns)
    got = tensor_bits(Y[torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()])
    assert np.array_equal(got, y), f"{int(np.count_nonzero(got != y))} sampled outputs differ"
    del Y
    torch.cuda.empty_cache()


def test_chains_past_2_31_elements():
    """The forward chain with column maxima and the grad-input chain with
    X of 524289 x 4096 (2^31 + 4096 elements; its codes fill more than 2 GB
    of the workspace) and dX of the same size: sampled rows of Y and dX against
    the oracle's quantized operands and scaled matmul."""
    M, N, K = 524289, 256, 4096
    print(f"case: chains {M} x {N} x {K}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(37)
    X = torch.randn((M, K), generator=g, device="cuda", dtype=torch.bfloat16)
    W = (0.02 * torch.randn((N, K), generator=g, device="cuda")).to(torch.bfloat16)
    dY = (1e-3 * torch.randn((M, N), generator=g, device="cuda")).to(torch.bfloat16)
    seed, off = 5, 1 << 44
    Y, cx, cw = i8.linear_fwd_colmax(X, W, "rne", seed, off)
    dX, _ = i8.linear_bwd(dY, X, W, "rne", seed, off, want_dw=False, colmax_x=cx, colmax_w=cw)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 262144, 524286, 524287, 524288])
    Wb = tensor_bits(W)
    qw, sw = oracle.quantize_rowwise(Wb, oracle.RNE)
    qwc, swc = oracle.quantize_colwise(Wb, oracle.RNE)
    for r in rows:
        qx, sx = oracle.quantize_rowwise(tensor_bits(X[r:r + 1]), oracle.RNE)
        _, y = oracle.scaled_mm_at(oracle.LAYOUTS["NT"], qx, sx, qw, sw, np.zeros(N, np.int64), np.arange(N))
        assert np.array_equal(tensor_bits(Y[r]), y), f"Y row {r}"
        qd, sd = oracle.quantize_rowwise(tensor_bits(dY[r:r + 1]), oracle.RNE)
        _, dx = oracle.scaled_mm_at(oracle.LAYOUTS["NN"], qd, sd, qwc, swc, np.zeros(K, np.int64), np.arange(K))
        assert np.array_equal(tensor_bits(dX[r]), dx), f"dX row {r}"
    del X, W, dY, Y, dX, cx, cw
    torch.cuda.empty_cache()


def _bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of finite float32 values, round to nearest even."""
    b = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("layout", ["TN", "NN"])
def test_gemm_operand_past_2_31_bytes(layout):
    """An operand read down its rows that spans 2^31 bytes (TN: A stored
    32768 x 65536; NN: B stored 32768 x 65536), which the pipelined kernel
    addresses with one descriptor per slab.  INT8 outputs sampled against the
    oracle; FP8 outputs against the fp32 sums of the FP8 hook (the general
    kernel, whose sums the pipelined kernel reproduces bit for bit) with the
    epilogue applied on the host in the same order."""
    M, N, K = (65536, 256, 32768) if layout == "TN" else (256, 65536, 32768)
    a_shape = (K, M) if layout == "TN" else (M, K)
    b_shape = (K, N)
    print(f"case: {layout} {M} x {N} x {K}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(41)
    rng = np.random.default_rng(41)
    ms = np.concatenate([rng.integers(0, M, 512), [0, M - 1, M - 1, 0]])
    ns = np.concatenate([rng.integers(0, N, 512), [0, N - 1, 0, N - 1]])
    ms_t, ns_t = torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()
    sa = torch.rand(M, generator=g, device="cuda") * 1e-3 + 1e-3
    sb = torch.rand(N, generator=g, device="cuda") * 1e-3 + 1e-3
    A = torch.randint(-127, 128, a_shape, generator=g, device="cuda", dtype=torch.int8)
    B = torch.randint(-127, 128, b_shape, generator=g, device="cuda", dtype=torch.int8)
    Y = i8.int8_scaled_mm(layout, A, sa, B, sb)
    torch.cuda.synchronize()
    _, y = oracle.scaled_mm_at(oracle.LAYOUTS[layout], A.cpu().numpy(), sa.cpu().numpy(), B.cpu().numpy(),
                               sb.cpu().numpy(), ms, ns)
    got = tensor_bits(Y[ms_t, ns_t])
    assert np.array_equal(got, y), f"INT8 {layout}: {int(np.count_nonzero(got != y))} sampled outputs differ"
    del A, B, Y
    torch.cuda.empty_cache()
    # E4M3 codes, the two NaN patterns moved to the largest finite magnitude
    A8 = torch.randint(0, 256, a_shape, generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
    B8 = torch.randint(0, 256, b_shape, generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
    for t in (A8, B8):  # elementwise: boolean-mask indexing does not take 2^31 elements
        t.sub_(((t & 0x7F) == 0x7F).to(torch.uint8))
    Y8 = i8.fp8_scaled_mm(layout, A8, sa, B8, sb)
    F = i8.fp8_mm_f32(layout, A8, B8)
    torch.cuda.synchronize()
    f = F[ms_t, ns_t].cpu().numpy()
    want = _bf16_rne_bits((f * sa.cpu().numpy()[ms]).astype(np.float32) * sb.cpu().numpy()[ns])
    got8 = tensor_bits(Y8[ms_t, ns_t])
    assert np.array_equal(got8, want), f"FP8 {layout}: {int(np.count_nonzero(got8 != want))} sampled outputs differ"
    del A8, B8, Y8, F
    torch.cuda.empty_cache()


def test_lm_head_grad_weight_at_32768_tokens():
    """The Llama-3 LM head's grad-weight chain at 32768 tokens: dY of
    32768 x 128256 (8.4 GB) quantized column-wise, and dW = dY.T @ X on the
    pipelined kernel with per-slab descriptors (dY's 4.2 GB of codes are read
    down their rows).  Sampled 8 x 8 blocks of dW against the oracle, from
    8-column slices of dY and X (column-wise quantization treats columns
    independently under RNE)."""
    M, N, K = 32768, 128256, 4096
    print(f"case: lm head grad-weight {M} x {N} x {K}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(43)
    X = torch.randn((M, K), generator=g, device="cuda", dtype=torch.bfloat16)
    W = (0.02 * torch.randn((N, K), generator=g, device="cuda")).to(torch.bfloat16)
    dY = (1e-3 * torch.randn((M, N), generator=g, device="cuda")).to(torch.bfloat16)
    _, dW = i8.linear_bwd(dY, X, W, "rne", 0, 0, want_dx=False)
    torch.cuda.synchronize()
    for n0, k0 in ((0, 0), (64000, 2048), (N - 8, K - 8)):
        qd, sd = oracle.quantize_colwise(tensor_bits(dY[:, n0:n0 + 8]), oracle.RNE)
        qx, sx = oracle.quantize_colwise(tensor_bits(X[:, k0:k0 + 8]), oracle.RNE)
        ms, ns = np.repeat(np.arange(8), 8), np.tile(np.arange(8), 8)
        _, y = oracle.scaled_mm_at(oracle.LAYOUTS["TN"], qd, sd, qx, sx, ms, ns)
        got = tensor_bits(dW[n0:n0 + 8, k0:k0 + 8]).reshape(-1)
        assert np.array_equal(got, y), f"dW block at ({n0}, {k0})"
    del X, W, dY, dW
    torch.cuda.empty_cache()
