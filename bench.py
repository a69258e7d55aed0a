"""Benchmark: one INT8 mixed-precision linear-layer training step on one MI355X.

A step is the whole hot path once: forward Y = X @ W.T, grad-input dX = dY @ W
and grad-weight dW = dY.T @ X, each GEMM quantizing its two bf16 operands
along its contraction (6 quantize passes: X row, W row, dY row, W col, dY col,
X col) and running the scaled INT8 matmul (NT, NN, TN) with the fp32 scale
epilogue to bf16.  Workload: the square GEMM sweep's largest size,
M = N = K = 4096 (X ~ N(0,1) with outlier channels, W ~ N(0,0.02),
dY ~ N(0,1e-3), bf16, synthetic, seeded).

Every launch goes through the C ABI on torch's current stream.  Two timed
regions run the same steps.  The first runs them as the library's linear
chains (i8mp_linear_fwd_colmax, i8mp_linear_bwd_colmax: the forward's two
row-wise passes share one launch, the backward's two column-wise passes too)
with nothing between the launches, and gives the step time (`value`,
`ms_per_step`).  The second runs the same computation as separate primitive
launches with a HIP event on that stream between every two, and gives each
kernel's duration (`breakdown`, `roofline`).  Both produce the same bytes
(checked before timing).  Recording an event costs a few microseconds of
stream time, which is why the step time comes from the event-free region.
Inputs rotate over several sets (more bytes than the 256 MB MALL) so every
step reads its operands from HBM.

Printed: one JSON line (rank 0).  `value` is the step's INT8 GEMM throughput,
3 * 2*M*N*K / step time, in TOPS; `roofline` describes the GEMM with the
largest share of the step; `cpu_baseline` times the CPU oracle on a bounded
sample of the same step (64 of the 4096 tokens).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0  # MI355X dense INT8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
METRIC = "INT8 scaled-GEMM TOPS (fwd/dgrad/wgrad) as % of INT8 MFMA peak; quant GB/s"
COUNTERS = os.path.join(ROOT, "profiles", "gemm_counters_square_4096.txt")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--size", type=int, default=4096, help="M = N = K")
    ap.add_argument("--rounding", default="rne", choices=["rne", "sr"])
    ap.add_argument("--sets", type=int, default=4, help="rotating input sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=64)
    ap.add_argument("--no-context", action="store_true",
                    help="skip the square-sweep and Llama-1B context measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, copy one 256 MiB buffer with torch (a plain "
                         "copy kernel of known size for scaling HBM byte counters)")
    return ap.parse_args()


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in ("gemm.hip", "internal.h"):
        with open(os.path.join(ROOT, "int8_mixed_precision_rowwise_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str):
    """HBM bytes per dispatch of `kernel` from the committed counter summary,
    if it was taken on the current GEMM source; else None."""
    if not os.path.exists(COUNTERS):
        return None
    fields = {}
    for line in open(COUNTERS):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_digest():
        return None
    key = f"hbm_bytes_per_dispatch_{kernel}"
    return float(fields[key]) if key in fields else None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); sharding this path "
              "over several GPUs is described in the design notes, not implemented.", file=sys.stderr)
        sys.exit(2)

    import torch

    import int8_mixed_precision_rowwise_amd as i8
    from workloads import linear_inputs, square

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n = args.size
    M = N = K = n
    shape = square(n)
    sets = []
    for s in range(args.sets):
        t = linear_inputs(shape, seed=s, device=dev)
        sets.append((t["X"], t["W"], t["dY"]))
    L = i8.lib
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    r = 0 if args.rounding == "rne" else 1
    seed = 1234

    def p(t):
        return ctypes.c_void_p(t.data_ptr())

    # outputs and int8 intermediates (dense, K and N multiples of 16 here)
    qX = torch.empty((M, K), dtype=torch.int8, device=dev)
    qW = torch.empty((N, K), dtype=torch.int8, device=dev)
    qdY = torch.empty((M, N), dtype=torch.int8, device=dev)
    qWc = torch.empty((N, K), dtype=torch.int8, device=dev)
    qdYc = torch.empty((M, N), dtype=torch.int8, device=dev)
    qXc = torch.empty((M, K), dtype=torch.int8, device=dev)
    sX = torch.empty(M, device=dev)
    sW = torch.empty(N, device=dev)
    sdY = torch.empty(M, device=dev)
    sWc = torch.empty(K, device=dev)
    sdYc = torch.empty(N, device=dev)
    sXc = torch.empty(K, device=dev)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    cX = torch.empty(K, device=dev)  # column maxima from the row-wise passes
    cW = torch.empty(K, device=dev)
    cdY = torch.empty(N, device=dev)
    wsb = max(L.i8mp_quantize_rowwise_colmax_workspace_bytes(M, K),
              L.i8mp_quantize_rowwise_colmax_workspace_bytes(N, K),
              L.i8mp_quantize_rowwise_colmax_workspace_bytes(M, N))
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    # each row-wise pass also reports its tensor's column maxima, so each
    # column-wise pass reads its tensor once (i8mp_linear_fwd_colmax /
    # i8mp_linear_bwd_colmax run the same launches)
    names = ["quant_row_X", "quant_row_W", "gemm_NT_fwd", "quant_row_dY", "quant_col_W",
             "gemm_NN_dgrad", "quant_col_dY", "quant_col_X", "gemm_TN_wgrad"]

    def launches(X, W, dY, step):
        off = step << 44
        ro = lambda j: off + (j << 40)  # noqa: E731  (per-pass Philox offsets)
        return [
            lambda: L.i8mp_quantize_rowwise_colmax(p(X), M, K, K, p(qX), K, p(sX), p(cX), r, seed, ro(0),
                                                   p(ws), wsb, sp),
            lambda: L.i8mp_quantize_rowwise_colmax(p(W), N, K, K, p(qW), K, p(sW), p(cW), r, seed, ro(1),
                                                   p(ws), wsb, sp),
            lambda: L.i8mp_int8_scaled_mm(0, M, N, K, p(qX), K, p(sX), p(qW), K, p(sW), p(Y), N, sp),
            lambda: L.i8mp_quantize_rowwise_colmax(p(dY), M, N, N, p(qdY), N, p(sdY), p(cdY), r, seed,
                                                   ro(2), p(ws), wsb, sp),
            lambda: L.i8mp_quantize_colwise_given_colmax(p(W), N, K, K, p(cW), p(qWc), K, p(sWc), r, seed,
                                                         ro(3), sp),
            lambda: L.i8mp_int8_scaled_mm(1, M, K, N, p(qdY), N, p(sdY), p(qWc), K, p(sWc), p(dX), K, sp),
            lambda: L.i8mp_quantize_colwise_given_colmax(p(dY), M, N, N, p(cdY), p(qdYc), N, p(sdYc), r,
                                                         seed, ro(4), sp),
            lambda: L.i8mp_quantize_colwise_given_colmax(p(X), M, K, K, p(cX), p(qXc), K, p(sXc), r, seed,
                                                         ro(5), sp),
            lambda: L.i8mp_int8_scaled_mm(2, N, K, M, p(qdYc), N, p(sdYc), p(qXc), K, p(sXc), p(dW), K, sp),
        ]

    plans = [launches(*sets[s], 0) for s in range(args.sets)]

    def run_step(i, events=None):
        plan = plans[i % args.sets]
        for j, f in enumerate(plan):
            if events is not None:
                events[j].record(stream)
            st = f()
            if st != 0:
                raise RuntimeError(f"{names[j]} failed with status {st}")
        if events is not None:
            events[len(plan)].record(stream)

    # the primitive chain is the library's linear_fwd / linear_bwd chain
    run_step(0)
    Yc, dXc, dWc = Y.clone(), dX.clone(), dW.clone()
    X0, W0, dY0 = sets[0]
    Yl, cx0, cw0 = i8.linear_fwd_colmax(X0, W0, args.rounding, seed, 0)
    ok = (torch.equal(Yl.view(torch.int16), Yc.view(torch.int16))
          and torch.equal(cx0, cX) and torch.equal(cw0, cW)
          and all(torch.equal(a.view(torch.int16), b.view(torch.int16))
                  for a, b in zip(i8.linear_bwd(dY0, X0, W0, args.rounding, seed, 0,
                                                colmax_x=cx0, colmax_w=cw0), (dXc, dWc))))
    if not ok:
        raise RuntimeError("primitive chain differs from linear_fwd_colmax/linear_bwd")

    # The step as the library runs it: i8mp_linear_fwd_colmax then
    # i8mp_linear_bwd_colmax (the forward's two row-wise passes share one
    # launch, the backward's two column-wise passes too, and dY's column
    # maxima are finalized in the launch of W's column pass: 8 launches).  Same
    # kernels' arithmetic as the 12 primitive launches above, same outputs.
    ws_fwd = torch.empty(L.i8mp_linear_workspace_bytes(M, N, K, 0), dtype=torch.uint8, device=dev)
    ws_bwd = torch.empty(L.i8mp_linear_workspace_bytes(M, N, K, 1), dtype=torch.uint8, device=dev)

    def chain_step(i, rr=r):
        X, W, dY = sets[i % args.sets]
        o = i8._Opts(rr, seed, 0)
        st = L.i8mp_linear_fwd_colmax(p(X), p(W), p(Y), M, N, K, ctypes.byref(o), p(cX), p(cW), p(ws_fwd),
                                      ws_fwd.numel(), sp)
        st = st or L.i8mp_linear_bwd_colmax(p(dY), p(X), p(W), p(dX), p(dW), M, N, K, ctypes.byref(o),
                                            p(cX), p(cW), p(ws_bwd), ws_bwd.numel(), sp)
        if st != 0:
            raise RuntimeError(f"linear chain step failed with status {st}")

    chain_step(0)
    if not (torch.equal(Y.view(torch.int16), Yc.view(torch.int16))
            and torch.equal(dX.view(torch.int16), dXc.view(torch.int16))
            and torch.equal(dW.view(torch.int16), dWc.view(torch.int16))):
        raise RuntimeError("the chains' step differs from the primitive launches")

    for i in range(args.warmup):
        chain_step(i)
        run_step(i)
    # timed region 1: the step time through the chains, nothing between the launches
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(args.steps):
        chain_step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = t0.elapsed_time(t1) / args.steps
    # timed region 2: the same steps with an event between every two launches
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    t2 = torch.cuda.Event(enable_timing=True)
    t3 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t2.record(stream)
    for i in range(args.steps):
        run_step(i, ev[i])
    t3.record(stream)
    torch.cuda.synchronize()
    step_ms_events = t2.elapsed_time(t3) / args.steps

    per = {nm: 0.0 for nm in names}
    for i in range(args.steps):
        for j, nm in enumerate(names):
            per[nm] += ev[i][j].elapsed_time(ev[i][j + 1])
    per = {nm: v / args.steps for nm, v in per.items()}  # ms per launch (row-wise: 2 kernels)

    gemm_ops = 2.0 * M * N * K
    breakdown = {}
    for nm, ms in per.items():
        d = {"us": round(ms * 1e3, 2)}
        if nm.startswith("gemm"):
            tops = gemm_ops / (ms * 1e-3) / 1e12
            d.update(tops=round(tops, 1), frac_int8_peak=round(tops / PEAK_INT8_TOPS, 4))
        else:
            tensor = {"X": (M, K), "W": (N, K), "dY": (M, N)}[nm.split("_")[-1]]
            nscale = tensor[0] if "_row_" in nm else tensor[1]
            algo = 3.0 * tensor[0] * tensor[1] + 4.0 * nscale
            gbs = algo / (ms * 1e-3) / 1e9
            d.update(gbs=round(gbs, 1), frac_hbm_peak=round(gbs / PEAK_HBM_GBS, 4))
        breakdown[nm] = d
    gemms = [nm for nm in names if nm.startswith("gemm")]
    dom = max(gemms, key=lambda nm: per[nm])
    achieved = gemm_ops / (per[dom] * 1e-3) / 1e12
    traffic = read_traffic(dom)
    value = 3 * gemm_ops / (step_ms * 1e-3) / 1e12

    # context: torch bf16 matmul (hipBLASLt) at the same shape and layouts
    a = sets[0][0]
    b = sets[0][1]
    ctx = {}
    for lay, fn in (("NT", lambda: a @ b.t()), ("NN", lambda: a @ b), ("TN", lambda: a.t() @ b)):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ctx[lay] = round(gemm_ops / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e12, 1)

    # context: the same layer step (forward + backward) through the autograd
    # integration, against torch's bf16 nn.Linear at the same shape
    from int8_mixed_precision_rowwise_amd.training import (Int8MixedPrecisionConfig,
                                                           Int8MixedPrecisionLinear)
    X0, W0, dY0 = sets[0]
    lin8 = Int8MixedPrecisionLinear(K, N, Int8MixedPrecisionConfig(
        stochastic_rounding=args.rounding == "sr", seed=seed), device=dev)
    lin16 = torch.nn.Linear(K, N, bias=False, device=dev, dtype=torch.bfloat16)
    with torch.no_grad():
        lin8.weight.copy_(W0)
        lin16.weight.copy_(W0)
    xg = X0.clone().requires_grad_()

    def layer_step(lin):
        xg.grad = None
        lin.weight.grad = None
        lin(xg).backward(dY0)

    autograd_ms = {}
    for tag, lin in (("int8", lin8), ("bf16", lin16)):
        for _ in range(5):
            layer_step(lin)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(20):
            layer_step(lin)
        e1.record(stream)
        torch.cuda.synchronize()
        autograd_ms[tag] = round(e0.elapsed_time(e1) / 20, 4)
    autograd_ms["speedup_vs_bf16"] = round(autograd_ms["bf16"] / autograd_ms["int8"], 3)

    # context: the same step with FP8 (E4M3) codes in place of INT8 (the
    # library's FP8 chains: same passes, FP8 matrix-core GEMMs)
    fp8 = None
    if K % 16 == 0 and N % 16 == 0 and M % 16 == 0:
        wsf = torch.empty(max(i8.linear_workspace_bytes(M, N, K, False),
                              i8.linear_workspace_bytes(M, N, K, True)), dtype=torch.uint8, device=dev)

        def fp8_step(i):
            X, W, dY = sets[i % args.sets]
            i8.linear_fwd_fp8(X, W, out=Y, workspace=wsf)
            i8.linear_bwd_fp8(dY, X, W, workspace=wsf)

        for i in range(5):
            fp8_step(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(20):
            fp8_step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        fp8_ms = e0.elapsed_time(e1) / 20
        fp8 = {"ms_per_step": round(fp8_ms, 4), "tops": round(3 * gemm_ops / (fp8_ms * 1e-3) / 1e12, 1),
               "note": "linear_fwd_fp8 + linear_bwd_fp8 (allocating their dX, dW), same inputs"}

    # context: the same step with the other rounding mode (stochastic rounding
    # draws Philox4x32-10 words in every quantize pass)
    other = 1 - r
    for i in range(args.warmup):
        chain_step(i, other)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        chain_step(i, other)
    e1.record(stream)
    torch.cuda.synchronize()
    other_ms = e0.elapsed_time(e1) / args.steps
    rounding_ctx = {"rounding": "sr" if other == 1 else "rne", "ms_per_step": round(other_ms, 4),
                    "tops": round(3 * gemm_ops / (other_ms * 1e-3) / 1e12, 1),
                    "time_vs_this_step": round(other_ms / step_ms, 3)}

    sweep = None if args.no_context else context_square_sweep(i8, dev, stream)
    qctx = None if args.no_context else context_quantize_large(i8, dev, stream)
    llama = None if args.no_context else context_llama1b_layers(i8, dev, stream)
    llama8b = None if args.no_context else context_llama3_8b_layers(i8, dev, stream)

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_tokens, N, K, args.rounding)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "ms_per_step_with_kernel_events": round(step_ms_events, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"linear_fwd_bwd_square_{n}", "M": M, "N": N, "K": K,
                   "rounding": args.rounding, "input_sets": args.sets},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_INT8_TOPS, 4), "traffic": traffic},
        "cpu_baseline": cpu,
        "breakdown": breakdown,
        "step_gemm_frac_int8_peak": round(value / PEAK_INT8_TOPS, 4),
        "context_torch_bf16_matmul_tflops": ctx,
        "context_autograd_layer_step_ms": autograd_ms,
        "context_fp8_step": fp8,
        "context_other_rounding_step": rounding_ctx,
        "context_square_sweep_vs_torch_bf16": sweep,
        "context_quantize_llama1b_sizes": qctx,
        "context_llama1b_7_linears_fwd_bwd": llama,
        "context_llama3_8b_linears_and_lm_head_fwd_bwd": llama8b,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


def _time_us(fn, stream, iters):
    import torch
    for _ in range(3):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters * 1e3


def context_square_sweep(i8, dev, stream):
    """The square GEMM sweep M = N = K in {1024, 2048, 4096} in the three
    layouts: the scaled INT8 GEMM on quantized Gaussian operands against
    torch's bf16 matmul on the same bf16 operands (the form of the pages'
    speed-up tables; quantization not included on either side)."""
    import torch
    from workloads import gaussian_bf16
    out = {}
    for n in (1024, 2048, 4096):
        a = gaussian_bf16(n, n, seed=11, device=dev)
        b = gaussian_bf16(n, n, seed=12, device=dev)
        y = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
        ops = 2.0 * n * n * n
        it = 50 if n < 4096 else 20
        row = {}
        for lay in ("NT", "NN", "TN"):
            qa, sa = i8.quantize_rowwise(a) if lay != "TN" else i8.quantize_colwise(a)
            qb, sb = i8.quantize_rowwise(b) if lay == "NT" else i8.quantize_colwise(b)
            t8 = _time_us(lambda: i8.int8_scaled_mm(lay, qa, sa, qb, sb, y), stream, it)
            f16 = {"NT": lambda: torch.matmul(a, b.t(), out=y), "NN": lambda: torch.matmul(a, b, out=y),
                   "TN": lambda: torch.matmul(a.t(), b, out=y)}[lay]
            t16 = _time_us(f16, stream, it)
            row[lay] = {"int8_us": round(t8, 2), "int8_tops": round(ops / t8 / 1e6, 1),
                        "bf16_us": round(t16, 2), "speedup": round(t16 / t8, 3)}
        out[str(n)] = row
    return out


def context_quantize_large(i8, dev, stream):
    """The quantize passes at the Llama-1B activation sizes (X 32768 x 2048,
    dY 32768 x 5632), in algorithmic GB/s (3 bytes per element + 4 per scale)
    against the 8 TB/s HBM peak, with a torch bf16 copy of the same tensor
    (4 bytes per element moved) for scale.  Inputs rotate over more bytes than
    the 256 MB MALL, so every pass reads HBM."""
    import ctypes
    import torch
    from workloads import gaussian_bf16
    L = i8.lib
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    out = {}
    for name, (R, C) in (("X_32768x2048", (32768, 2048)), ("dY_32768x5632", (32768, 5632))):
        nset = max(2, (3 << 28) // (R * C * 2) + 1)
        xs = [gaussian_bf16(R, C, seed=20 + i, device=dev) for i in range(nset)]
        q = torch.empty((R, C), dtype=torch.int8, device=dev)
        srow = torch.empty(R, device=dev)
        scol = torch.empty(C, device=dev)
        cm = torch.empty(C, device=dev)
        ws = torch.empty(i8.rowwise_colmax_workspace_bytes(R, C), dtype=torch.uint8, device=dev)
        y = torch.empty((R, C), dtype=torch.bfloat16, device=dev)
        k = [0]

        def nxt():
            k[0] += 1
            return xs[k[0] % nset]

        def chk(st):
            if st != 0:
                raise RuntimeError(f"quantize context: status {st}")

        passes = {
            "row": lambda: chk(L.i8mp_quantize_rowwise(P(nxt()), R, C, C, P(q), C, P(srow), 0, 0, 0, sp)),
            "row_with_colmax": lambda: chk(L.i8mp_quantize_rowwise_colmax(
                P(nxt()), R, C, C, P(q), C, P(srow), P(cm), 0, 0, 0, P(ws), ws.numel(), sp)),
            "col_given_colmax": lambda: chk(L.i8mp_quantize_colwise_given_colmax(
                P(nxt()), R, C, C, P(cm), P(q), C, P(scol), 0, 0, 0, sp)),
        }
        row = {}
        for pn, fn in passes.items():
            us = _time_us(fn, stream, 20)
            nscale = R if pn.startswith("row") else C
            gbs = (3.0 * R * C + 4.0 * nscale) / us / 1e3
            row[pn] = {"us": round(us, 1), "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
        us = _time_us(lambda: y.copy_(nxt()), stream, 20)
        row["torch_bf16_copy"] = {"us": round(us, 1), "gbs": round(4.0 * R * C / us / 1e3, 1)}
        out[name] = row
        del xs, q, y, ws
    torch.cuda.empty_cache()
    return out


def context_llama1b_layers(i8, dev, stream):
    """The seven Llama-1B decoder linears at 16 x 2048 = 32768 tokens."""
    from workloads import llama_1b_layers
    return context_layers(i8, dev, stream, llama_1b_layers(), "llama1b_", 10)


def context_llama3_8b_layers(i8, dev, stream):
    """The seven Llama-3-8B decoder linears and the LM head [4096 -> 128256]
    at 8192 tokens."""
    from workloads import llama3_8b_layers
    return context_layers(i8, dev, stream, llama3_8b_layers(), "llama3_8b_", 5)


def context_layers(i8, dev, stream, shapes, prefix, iters):
    """Each linear's training step through the chains (forward with column
    maxima, then both gradients: 6 quantize passes + 3 INT8 GEMMs), against
    the three bf16 torch matmuls of the same step (no quantization)."""
    import torch
    from workloads import linear_inputs
    tot8 = tot16 = 0.0
    ops = 0.0
    per = {}
    for shape in shapes:
        M, N, K = shape.M, shape.N, shape.K
        t = linear_inputs(shape, seed=0, device=dev)
        X, W, dY = t["X"], t["W"], t["dY"]
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        dW = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        wsf = torch.empty(i8.linear_workspace_bytes(M, N, K, False), dtype=torch.uint8, device=dev)
        wsb = torch.empty(i8.linear_workspace_bytes(M, N, K, True), dtype=torch.uint8, device=dev)

        def step8():
            _, cx, cw = i8.linear_fwd_colmax(X, W, out=Y, workspace=wsf)
            i8.linear_bwd(dY, X, W, dX=dX, dW=dW, workspace=wsb, colmax_x=cx, colmax_w=cw)

        def step16():
            torch.matmul(X, W.t(), out=Y)
            torch.matmul(dY, W, out=dX)
            torch.matmul(dY.t(), X, out=dW)

        t8 = _time_us(step8, stream, iters)
        t16 = _time_us(step16, stream, iters)
        per[shape.name.replace(prefix, "")] = {"int8_us": round(t8, 1), "bf16_us": round(t16, 1)}
        tot8 += t8
        tot16 += t16
        ops += 3 * 2.0 * M * N * K
        del t, X, W, dY, Y, dX, dW, wsf, wsb
    torch.cuda.empty_cache()
    return {"int8_us": round(tot8, 1), "bf16_gemms_us": round(tot16, 1),
            "speedup_vs_bf16": round(tot16 / tot8, 3), "int8_tops": round(ops / tot8 / 1e6, 1),
            "per_linear": per,
            "note": f"tokens {shapes[0].M}; int8 includes all quantize passes, bf16 is the GEMMs alone"}


def cpu_baseline(tokens: int, N: int, K: int, rounding: str):
    """The CPU oracle, as it is, on the same layer step with `tokens` of the
    tokens (X [tokens, K], dY [tokens, N], W [N, K] in full)."""
    import oracle
    from workloads import LinearShape, bf16_bits, linear_inputs

    t = linear_inputs(LinearShape("cpu_sample", tokens, N, K), seed=0)
    X, W, dY = (bf16_bits(t[k]) for k in ("X", "W", "dY"))
    r = oracle.RNE if rounding == "rne" else oracle.SR
    t0 = time.perf_counter()
    oracle.linear_fwd(X, W, r, 1234, 0)
    oracle.linear_bwd(dY, X, W, r, 1234, 0)
    dt = time.perf_counter() - t0
    ops = 3 * 2.0 * tokens * N * K
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"oracle linear fwd+bwd (6 quantize passes + NT/NN/TN) at {tokens} of the "
                      f"tokens: X [{tokens},{K}], W [{N},{K}], dY [{tokens},{N}], single thread"}


if __name__ == "__main__":
    main()
