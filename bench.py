"""Benchmark: one INT8 mixed-precision linear-layer training step on one MI355X.

A step is the whole hot path once: forward Y = X @ W.T, grad-input dX = dY @ W
and grad-weight dW = dY.T @ X, each GEMM quantizing its two bf16 operands
along its contraction (6 quantize passes: X row, W row, dY row, W col, dY col,
X col) and running the scaled INT8 matmul (NT, NN, TN) with the fp32 scale
epilogue to bf16.  Workload: the square GEMM sweep's largest size,
M = N = K = 4096 (X ~ N(0,1) with outlier channels, W ~ N(0,0.02),
dY ~ N(0,1e-3), bf16, synthetic, seeded), round to nearest even.

Every launch goes through the C ABI on torch's current stream.  The step runs
as the library's linear chains (i8mp_linear_fwd_colmax, i8mp_linear_bwd_colmax)
with nothing between the launches; inputs rotate over several sets (more bytes
than the 256 MB MALL), so every step reads its operands from HBM.  Five
trials of exactly --steps steps each are timed with HIP events on that stream
(synchronized on both sides); `value` and `ms_per_step` are the median
trial's.

Each kernel of the step is also timed on its own: --kernel-iters back-to-back
launches between two events on the launch stream (quantize passes rotating
over 1 GiB of inputs, four times the MALL), so the per-launch figure carries no
event overhead.  `roofline`
describes the GEMM with the largest time; `breakdown` every pass.

Printed: one JSON line.  `value` is the step's INT8 GEMM throughput,
3 * 2*M*N*K / step time, in TOPS.  `records` holds one entry per (config,
shape, layout, kernel) measured; `cpu_baseline` times the CPU oracle on a
bounded sample of the same step, on one core and on all the host's cores.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0  # MI355X dense INT8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
# VALU issue rate: 256 CUs x 4 SIMDs x 16 lanes per clock at 2.4 GHz (a wave64
# instruction of full rate occupies a SIMD for 4 clocks): 39.3e12 lane
# operations per second (the fp32 vector peak of 157.3 TFLOP/s counts an FMA
# as 2 and packed fp32 as 2 lanes per slot).
PEAK_VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
TARGET_GEMM_FRAC = 0.60  # of the INT8 peak at 4096^3
TARGET_QUANT_FRAC = 0.70  # of the HBM peak
METRIC = "INT8 scaled-GEMM TOPS (fwd/dgrad/wgrad) as % of INT8 MFMA peak; quant GB/s"
PROFILES = os.path.join(ROOT, "profiles")
GEMM_COUNTERS = os.path.join(PROFILES, "gemm_counters_square_4096.txt")
VALU_COUNTERS = os.path.join(PROFILES, "quantize_valu_counters_square_4096.txt")
TRIALS = 5
CONTEXTS = ("other_rounding", "sr_passes", "elementwise", "cold_warm", "mfma_ceiling", "hip_graph", "torch_bf16",
            "torch_int8",
            "autograd", "fp8", "single_linear", "square_sweep", "quantize_large", "llama1b", "ablation", "llama3_8b")


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--size", type=int, default=4096, help="M = N = K")
    ap.add_argument("--rounding", default="rne", choices=["rne", "sr"])
    ap.add_argument("--sets", type=int, default=4, help="rotating input sets")
    ap.add_argument("--kernel-iters", type=int, default=20,
                    help="back-to-back launches per kernel in the per-kernel timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=64)
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context measurements (sweep, Llama layers, ablation, ...)")
    ap.add_argument("--context", default=None,
                    help="comma-separated context measurements to run (and no others): " + ", ".join(CONTEXTS))
    ap.add_argument("--only-step", action="store_true",
                    help="the timed step and its per-kernel timing only (for profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, copy one 256 MiB buffer with torch (a plain "
                         "copy kernel of known size for scaling HBM byte counters)")
    args = ap.parse_args(argv)
    if args.context is not None:
        unknown = sorted(set(args.context.split(",")) - set(CONTEXTS))
        if unknown:
            ap.error(f"--context: unknown name(s) {unknown}")
    return args


# --------------------------------------------------------------------------- counter summaries


def source_digest(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "int8_mixed_precision_rowwise_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_summary(path: str, files) -> dict | None:
    """key: value lines of a committed counter summary, if it was taken on the
    current sources (its kernel_source_sha256_16 matches); else None."""
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != source_digest(files):
        return None
    return fields


def read_traffic(kernel: str):
    """HBM bytes per dispatch of a GEMM from the committed counter summary."""
    f = read_summary(GEMM_COUNTERS, ("gemm.hip", "internal.h"))
    key = f"hbm_bytes_per_dispatch_{kernel}"
    return float(f[key]) if f and key in f else None


# --------------------------------------------------------------------------- timing helpers


def time_us(fn, stream, iters, warm=3):
    """Average microseconds per call of `iters` back-to-back calls between two
    HIP events on `stream` (after `warm` untimed calls)."""
    import torch
    for _ in range(warm):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters * 1e3


def quant_bytes(rows: int, cols: int, nscale: int) -> float:
    """Algorithmic bytes of one quantize pass: 2 read + 1 written per element,
    4 per scale."""
    return 3.0 * rows * cols + 4.0 * nscale


def gemm_entry(us, M, N, K):
    tops = 2.0 * M * N * K / us / 1e6
    return {"us": round(us, 2), "tops": round(tops, 1), "frac_int8_peak": round(tops / PEAK_INT8_TOPS, 4)}


def quant_entry(us, rows, cols, nscale):
    gbs = quant_bytes(rows, cols, nscale) / us / 1e3
    return {"us": round(us, 2), "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


class Abi:
    """ctypes helpers over the library for the hand-built launch sequences."""

    def __init__(self, i8, stream):
        self.i8, self.L = i8, i8.lib
        self.sp = ctypes.c_void_p(stream.cuda_stream)

    @staticmethod
    def p(t):
        return ctypes.c_void_p(t.data_ptr())

    @staticmethod
    def ok(st, what):
        if st != 0:
            raise RuntimeError(f"{what} failed with status {st}")


# --------------------------------------------------------------------------- the timed step


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
    stream = torch.cuda.current_stream(dev)
    A = Abi(i8, stream)
    L, p, sp = A.L, A.p, A.sp
    n = args.size
    M = N = K = n
    sets = []
    for s in range(args.sets):
        t = linear_inputs(square(n), seed=s, device=dev)
        sets.append((t["X"], t["W"], t["dY"]))
    r = 0 if args.rounding == "rne" else 1
    seed = 1234

    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    cX = torch.empty(K, device=dev)
    cW = torch.empty(K, device=dev)
    ws_fwd = torch.empty(L.i8mp_linear_workspace_bytes(M, N, K, 0), dtype=torch.uint8, device=dev)
    ws_bwd = torch.empty(L.i8mp_linear_workspace_bytes(M, N, K, 1), dtype=torch.uint8, device=dev)

    def chain_step(i, rr=r, on=None):
        """The step as the library runs it: i8mp_linear_fwd_colmax (X's and W's
        row passes in one launch, leaving slab maxima of their columns; the NT
        GEMM, which reduces those slabs to X's and W's column maxima in its
        prologue), then i8mp_linear_bwd_colmax (dY's row pass and W's column
        pass in one launch; the NN GEMM, reducing dY's slabs in its prologue;
        dY's and X's column passes in one launch; the TN GEMM): 6 launches, on
        the bench's stream or on the stream `on` (a ctypes pointer)."""
        X, W, dY = sets[i % args.sets]
        o = i8._Opts(rr, seed, (i % 1024) << 44)
        s_ = sp if on is None else on
        st = L.i8mp_linear_fwd_colmax(p(X), p(W), p(Y), M, N, K, ctypes.byref(o), p(cX), p(cW), p(ws_fwd),
                                      ws_fwd.numel(), s_)
        st = st or L.i8mp_linear_bwd_colmax(p(dY), p(X), p(W), p(dX), p(dW), M, N, K, ctypes.byref(o),
                                            p(cX), p(cW), p(ws_bwd), ws_bwd.numel(), s_)
        A.ok(st, "linear chain step")

    # the chains' outputs equal the public primitives' (one quantize pass and
    # one GEMM per launch) on the same inputs
    prim = primitive_step(A, sets[0], r, seed, 0)
    chain_step(0)
    torch.cuda.synchronize()
    for got, want, what in ((Y, prim["Y"], "Y"), (dX, prim["dX"], "dX"), (dW, prim["dW"], "dW")):
        if not torch.equal(got.view(torch.int16), want.view(torch.int16)):
            raise RuntimeError(f"the chains' {what} differs from the primitive launches'")

    for i in range(args.warmup):
        chain_step(i)
    trials = []
    wall0 = time.perf_counter()
    for _ in range(TRIALS):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(args.steps):
            chain_step(i)
        t1.record(stream)
        torch.cuda.synchronize()
        trials.append(t0.elapsed_time(t1) / args.steps)
    wall = time.perf_counter() - wall0
    step_ms = statistics.median(trials)
    gemm_ops = 2.0 * M * N * K
    value = 3 * gemm_ops / (step_ms * 1e-3) / 1e12

    # each kernel of the step on its own, back to back
    pool = cold_pool(sets, n, dev)
    breakdown = step_breakdown(A, sets, pool, prim, r, seed, args.kernel_iters, stream)
    gemms = [k for k in breakdown if k.startswith("gemm")]
    dom = max(gemms, key=lambda k: breakdown[k]["us"])
    achieved = gemm_ops / (breakdown[dom]["us"] * 1e-6) / 1e12
    frac = achieved / PEAK_INT8_TOPS
    quant_frac = {k: v["frac_hbm_peak"] for k, v in breakdown.items() if k.startswith("quant")}

    # the chain's quantize launches (paired, with the column maxima reduced in
    # the GEMM prologues) cannot be timed apart through the C ABI: charge them
    # the step's time beyond its three GEMMs (each timed on the step's codes)
    q_us = step_ms * 1e3 - sum(breakdown[k]["us"] for k in gemms)
    q_bytes = 6 * quant_bytes(n, n, n)
    chain_quant = {"us": round(q_us, 2), "gbs": round(q_bytes / (q_us * 1e-6) / 1e9, 1),
                   "frac_hbm_peak": round(q_bytes / (q_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                   "note": "step time minus the three GEMMs' times, against the six passes' algorithmic bytes; "
                           "the prologue work of the chain's GEMMs counts as quantize time"}

    records = [{"config": f"square_{n}_step", "shape": [M, N, K], "layout": k.split("_")[1] if k.startswith("gemm") else None,
                "kernel": k, **v} for k, v in breakdown.items()]
    records.append({"config": f"square_{n}_step", "shape": [M, N, K], "layout": None,
                    "kernel": "linear_fwd_colmax+linear_bwd_colmax", "ms": round(step_ms, 4),
                    "tops": round(value, 1)})

    ctx = {}
    runs = (
        ("step", "other_rounding", "context_other_rounding_step",
         lambda: other_rounding(chain_step, r, step_ms, args, stream, gemm_ops)),
        ("step", "sr_passes", "context_sr_quantize_passes", lambda: sr_passes(A, pool, n, args.kernel_iters, stream)),
        ("step", "elementwise", "context_elementwise_reference", lambda: elementwise_reference(pool, args.kernel_iters, stream)),
        ("step", "cold_warm", "context_gemm_cold_vs_warm", lambda: gemm_cold_warm(A, n, args.kernel_iters, stream, records)),
        ("step", "mfma_ceiling", "context_mfma_power_ceiling", lambda: mfma_ceiling(A, prim["qX"], breakdown, stream)),
        ("step", "hip_graph", "context_step_as_hip_graph",
         lambda: graph_step(chain_step, (Y, dX, dW), args, stream, step_ms)),
        ("wide", "torch_bf16", "context_torch_bf16_matmul_tflops", lambda: torch_bf16(sets[0], stream, gemm_ops)),
        ("wide", "torch_int8", "context_torch_int_mm_hipblaslt", lambda: torch_int8_mm(sets, prim, args.kernel_iters,
                                                                                        stream, gemm_ops)),
        ("wide", "autograd", "context_autograd_layer_step_ms",
         lambda: autograd_step(i8, sets[0], args.rounding, seed, stream)),
        ("wide", "fp8", "context_fp8_step", lambda: fp8_step(i8, sets, M, N, K, stream, gemm_ops)),
        ("wide", "single_linear", "context_single_linear_256x512x512", lambda: single_linear_ctx(i8, stream, records)),
        ("wide", "square_sweep", "context_square_sweep_vs_torch_bf16",
         lambda: context_square_sweep(i8, dev, stream, records)),
        ("wide", "quantize_large", "context_quantize_llama1b_sizes", lambda: context_quantize_large(i8, dev, stream, records)),
        ("wide", "llama1b", "context_llama1b_7_linears_fwd_bwd", lambda: context_layers_both(i8, dev, stream, records)),
        ("wide", "ablation", "context_llama1b_ablation_int8_gemms", lambda: context_ablation(i8, dev, stream, records)),
        ("wide", "llama3_8b", "context_llama3_8b_linears_and_lm_head_fwd_bwd",
         lambda: context_llama3_8b_layers(i8, dev, stream, records)),
    )
    chosen = None if args.context is None else set(args.context.split(","))
    assert {nm for _, nm, _, _ in runs} == set(CONTEXTS)
    for group, nm, key, fn in runs:
        if chosen is not None:
            on = nm in chosen
        else:
            on = not args.only_step and (group == "step" or not args.no_context)
        if on:
            ctx[key] = fn()

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_tokens, N, K, args.rounding)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "trials_ms_per_step": [round(t, 4) for t in trials],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"linear_fwd_bwd_square_{n}", "M": M, "N": N, "K": K,
                   "rounding": args.rounding, "input_sets": args.sets},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": PEAK_INT8_TOPS, "unit": "TOPS", "frac": round(frac, 4),
                     "traffic": read_traffic(dom)},
        "cpu_baseline": cpu,
        "targets": {
            "gemm_frac_int8_peak": {"target": TARGET_GEMM_FRAC, **{k: breakdown[k]["frac_int8_peak"] for k in gemms},
                                    "share_of_target_dominant": round(frac / TARGET_GEMM_FRAC, 3)},
            "quant_frac_hbm_peak": {"target": TARGET_QUANT_FRAC, **quant_frac,
                                    "share_of_target_worst": round(min(quant_frac.values()) / TARGET_QUANT_FRAC, 3),
                                    "chain_passes_by_subtraction": chain_quant},
        },
        "breakdown": breakdown,
        "step_gemm_frac_int8_peak": round(value / PEAK_INT8_TOPS, 4),
        **ctx,
        "records": records,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


def primitive_step(A, inputs, r, seed, off):
    """The step as 12 public primitive launches (row passes with column
    maxima, column passes given the maxima, the three GEMMs); returns the
    outputs and the intermediate codes and scales (which the per-kernel
    timing reuses)."""
    import torch
    i8 = A.i8
    X, W, dY = inputs
    M, K = X.shape
    N = W.shape[0]
    ro = lambda j: off + (j << 40)  # noqa: E731  (per-pass Philox offsets)
    rnd = "rne" if r == 0 else "sr"
    out = {}
    out["qX"], out["sX"], out["cX"] = i8.quantize_rowwise_colmax(X, rnd, seed, ro(0))
    out["qW"], out["sW"], out["cW"] = i8.quantize_rowwise_colmax(W, rnd, seed, ro(1))
    out["Y"] = i8.int8_scaled_mm("NT", out["qX"], out["sX"], out["qW"], out["sW"])
    out["qdY"], out["sdY"], out["cdY"] = i8.quantize_rowwise_colmax(dY, rnd, seed, ro(2))
    out["qWc"], out["sWc"] = i8.quantize_colwise_given_colmax(W, out["cW"], rnd, seed, ro(3))
    out["dX"] = i8.int8_scaled_mm("NN", out["qdY"], out["sdY"], out["qWc"], out["sWc"])
    out["qdYc"], out["sdYc"] = i8.quantize_colwise_given_colmax(dY, out["cdY"], rnd, seed, ro(4))
    out["qXc"], out["sXc"] = i8.quantize_colwise_given_colmax(X, out["cX"], rnd, seed, ro(5))
    out["dW"] = i8.int8_scaled_mm("TN", out["qdYc"], out["sdYc"], out["qXc"], out["sXc"])
    torch.cuda.synchronize()
    return out


def cold_pool(sets, n, dev, nbytes=1 << 30, most=128):
    """n x n bf16 tensors totalling at least `nbytes` (4x the 256 MB MALL),
    at most `most` of them: the step's inputs, then standard normal draws.
    Quantize passes and the copy reference rotate over them, so every timed
    call reads cold HBM (at the default size: 32 tensors of 32 MiB)."""
    import torch
    pool = [t for s in sets for t in s]
    g = torch.Generator(device=dev).manual_seed(4321)
    while len(pool) * n * n * 2 < nbytes and len(pool) < most:
        pool.append(torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16))
    return pool


def step_breakdown(A, sets, pool, prim, r, seed, iters, stream):
    """Each primitive pass of the step timed as `iters` back-to-back launches:
    quantize passes rotate over the cold pool (each reads HBM), GEMMs run on
    the step's codes (warm, as right after their quantize passes)."""
    import torch
    L, p, sp = A.L, A.p, A.sp
    M, K = sets[0][0].shape
    N = sets[0][1].shape[0]
    q = torch.empty((max(M, N), max(K, N)), dtype=torch.int8, device=sets[0][0].device)
    srow = torch.empty(max(M, N), device=q.device)
    scol = torch.empty(max(K, N), device=q.device)
    cm = torch.empty(max(K, N), device=q.device)
    wsb = max(L.i8mp_quantize_rowwise_colmax_workspace_bytes(M, K), L.i8mp_quantize_rowwise_colmax_workspace_bytes(N, K),
              L.i8mp_quantize_rowwise_colmax_workspace_bytes(M, N))
    ws = torch.empty(wsb, dtype=torch.uint8, device=q.device)
    k = [0]

    def pick(j):  # every step tensor is n x n: any pool tensor stands in for tensor j
        k[0] += 1
        return pool[k[0] % len(pool)]

    def row(j, R, C):
        return lambda: A.ok(L.i8mp_quantize_rowwise_colmax(p(pick(j)), R, C, C, p(q), C, p(srow), p(cm), r, seed, 0,
                                                           p(ws), wsb, sp), "row pass")

    def col(j, R, C, cmax):
        return lambda: A.ok(L.i8mp_quantize_colwise_given_colmax(p(pick(j)), R, C, C, p(cmax), p(q), C, p(scol), r,
                                                                 seed, 0, sp), "column pass")

    out = torch.empty((max(M, N), max(N, K)), dtype=torch.bfloat16, device=q.device)
    ld = A.i8._ld

    def gemm(lay, Mo, No, Ko, a, sa, b, sb):
        return lambda: A.ok(L.i8mp_int8_scaled_mm(lay, Mo, No, Ko, p(a), ld(a), p(sa), p(b), ld(b), p(sb), p(out), No,
                                                  sp), "GEMM")

    P = prim
    b = {}
    b["quant_row_X"] = quant_entry(time_us(row(0, M, K), stream, iters), M, K, M)
    b["quant_row_W"] = quant_entry(time_us(row(1, N, K), stream, iters), N, K, N)
    b["gemm_NT_fwd"] = gemm_entry(time_us(gemm(0, M, N, K, P["qX"], P["sX"], P["qW"], P["sW"]), stream, iters), M, N, K)
    b["quant_row_dY"] = quant_entry(time_us(row(2, M, N), stream, iters), M, N, M)
    b["quant_col_W"] = quant_entry(time_us(col(1, N, K, P["cW"]), stream, iters), N, K, K)
    b["gemm_NN_dgrad"] = gemm_entry(time_us(gemm(1, M, K, N, P["qdY"], P["sdY"], P["qWc"], P["sWc"]), stream, iters),
                                    M, K, N)
    b["quant_col_dY"] = quant_entry(time_us(col(2, M, N, P["cdY"]), stream, iters), M, N, N)
    b["quant_col_X"] = quant_entry(time_us(col(0, M, K, P["cX"]), stream, iters), M, K, K)
    b["gemm_TN_wgrad"] = gemm_entry(time_us(gemm(2, N, K, M, P["qdYc"], P["sdYc"], P["qXc"], P["sXc"]), stream, iters),
                                    N, K, M)
    for nm in ("quant_row_X", "quant_row_W", "quant_row_dY"):
        b[nm]["note"] = ("public i8mp_quantize_rowwise_colmax: the row pass (slab maxima) + a colmax_finalize "
                         "launch; the chain pairs X's and W's row passes in one launch and reduces the slabs "
                         "in the next GEMM's prologue")
    return b


# --------------------------------------------------------------------------- context measurements


def graph_step(chain_step, outs, args, stream, step_ms):
    """The step captured as a HIP graph (torch.cuda.CUDAGraph; the library
    allocates, clears and synchronizes nothing, so the capture holds the six
    kernel launches of each step), one step per input set, then replayed
    back to back: ms per step against the eager launches'.  The last replay's
    outputs are checked against the eager step's on the same inputs."""
    import torch
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i in range(args.sets):
            chain_step(i, on=cs)
    reps = max(1, args.steps // args.sets)
    us = time_us(g.replay, stream, reps, warm=2)
    got = [t.clone() for t in outs]
    chain_step(args.sets - 1)
    torch.cuda.synchronize()
    if not all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(got, outs)):
        raise RuntimeError("the graph replay's outputs differ from the eager step's")
    del g
    ms = us / 1e3 / args.sets
    return {"ms_per_step": round(ms, 4), "time_vs_eager": round(ms / step_ms, 3),
            "steps_per_replay": args.sets, "replays": reps}


def other_rounding(chain_step, r, step_ms, args, stream, gemm_ops):
    """The same step with the other rounding (stochastic rounding draws
    Philox4x32-10 words in every quantize pass), median of the trials."""
    import torch
    other = 1 - r
    for i in range(args.warmup):
        chain_step(i, other)
    trials = []
    for _ in range(TRIALS):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            chain_step(i, other)
        e1.record(stream)
        torch.cuda.synchronize()
        trials.append(e0.elapsed_time(e1) / args.steps)
    ms = statistics.median(trials)
    return {"rounding": "sr" if other == 1 else "rne", "ms_per_step": round(ms, 4),
            "tops": round(3 * gemm_ops / (ms * 1e-3) / 1e12, 1), "time_vs_this_step": round(ms / step_ms, 3)}


def sr_passes(A, pool, n, iters, stream):
    """The step's quantize passes at n x n under both roundings, in
    algorithmic GB/s against the HBM peak and, for stochastic rounding, in
    VALU lane operations against the VALU issue peak.  VALU operations per
    element come from the committed rocprofv3 counter summary (SQ_INSTS_VALU
    per dispatch of the same kernels on the current sources); null otherwise."""
    import torch
    L, p, sp = A.L, A.p, A.sp
    q = torch.empty((n, n), dtype=torch.int8, device=pool[0].device)
    s = torch.empty(n, device=q.device)
    cm = torch.empty(n, device=q.device)
    wsb = max(L.i8mp_quantize_rowwise_colmax_workspace_bytes(n, n), 1)
    ws = torch.empty(wsb, dtype=torch.uint8, device=q.device)
    maxima = [A.i8.quantize_rowwise_colmax(t)[2] for t in pool]  # each tensor's column maxima
    k = [0]

    def nxt():
        k[0] += 1
        return pool[k[0] % len(pool)], maxima[k[0] % len(pool)]

    def row_pass(rr):
        x, _ = nxt()
        A.ok(L.i8mp_quantize_rowwise_colmax(p(x), n, n, n, p(q), n, p(s), p(cm), rr, 5, 0, p(ws), wsb, sp), "row")

    def col_pass(rr):
        x, c = nxt()
        A.ok(L.i8mp_quantize_colwise_given_colmax(p(x), n, n, n, p(c), p(q), n, p(s), rr, 5, 0, sp), "col")

    counters = read_summary(VALU_COUNTERS, ("quantize.hip", "philox.h", "internal.h"))
    out = {}
    for rr, tag in ((0, "rne"), (1, "sr")):
        row = time_us(lambda: row_pass(rr), stream, iters)
        col = time_us(lambda: col_pass(rr), stream, iters)
        for nm, us in (("row_with_colmax", row), ("col_given_colmax", col)):
            e = quant_entry(us, n, n, n)
            key = f"valu_lane_ops_per_elem_{nm}_{tag}"
            if counters and key in counters:
                per = float(counters[key])
                ach = per * n * n / (us * 1e-6)
                e["valu"] = {"lane_ops_per_elem": per, "achieved": round(ach / 1e12, 2), "peak": round(PEAK_VALU_LANE_OPS / 1e12, 2),
                             "unit": "T lane-ops/s", "frac": round(ach / PEAK_VALU_LANE_OPS, 4)}
            out[f"{nm}_{tag}"] = e
    return out


def elementwise_reference(pool, iters, stream):
    """What a plain streaming kernel reaches on the same bytes and the same
    cold inputs: torch's bf16 copy of an n x n tensor (4 bytes moved per
    element) and of two such tensors stacked (the paired passes' byte count),
    its source rotating over the cold pool as the quantize passes' do."""
    import torch
    src1 = pool
    src2 = [torch.cat([src1[i], src1[(i + 1) % len(src1)]]) for i in range(0, len(src1), 2)]
    d1 = torch.empty_like(src1[0])
    d2 = torch.empty_like(src2[0])
    k = [0]

    def copy(dst, srcs):
        def f():
            k[0] += 1
            dst.copy_(srcs[k[0] % len(srcs)])
        return f

    out = {}
    for nm, fn, src in (("copy_bf16_single", copy(d1, src1), src1[0]), ("copy_bf16_pair", copy(d2, src2), src2[0])):
        us = time_us(fn, stream, iters)
        gbs = src.numel() * 4 / (us * 1e-6) / 1e9
        out[nm] = {"us": round(us, 2), "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    del src2, d1, d2
    torch.cuda.empty_cache()
    return out


def torch_int8_mm(sets, prim, iters, stream, gemm_ops):
    """hipBLASLt's int8 GEMM through torch._int_mm (int32 output, no scales)
    on the step's codes in the forward layout, as a library reference for the
    GEMM's fraction of the INT8 peak."""
    import torch
    a, b = prim["qX"], prim["qW"]
    try:
        out = torch._int_mm(a, b.t())
        torch.cuda.synchronize()
    except Exception as e:  # not every torch build routes int8 GEMMs to hipBLASLt
        return {"unavailable": str(e).splitlines()[0][:200]}
    us = time_us(lambda: torch._int_mm(a, b.t()), stream, iters)
    del out
    return {"layout": "NT", "us": round(us, 2), "tops": round(gemm_ops / us / 1e6, 1),
            "frac_int8_peak": round(gemm_ops / us / 1e6 / PEAK_INT8_TOPS, 4), "output": "int32"}


def gemm_cold_warm(A, n, iters, stream, records):
    """The n^3 GEMM in each layout with warm operands (the same codes every
    launch: they stay in L2 and the MALL, as right after their quantize
    passes) and cold ones (rotating over operand pairs holding more than the
    256 MB MALL)."""
    import torch
    L, p, sp = A.L, A.p, A.sp
    dev = torch.device("cuda")
    g = torch.Generator(device=dev).manual_seed(77)
    npairs = max(2, (384 << 20) // (2 * n * n) + 1)
    ops = [(torch.randint(-127, 128, (n, n), generator=g, dtype=torch.int8, device=dev),
            torch.randint(-127, 128, (n, n), generator=g, dtype=torch.int8, device=dev)) for _ in range(npairs)]
    sa = torch.rand(n, generator=g, device=dev) * 1e-2
    sb = torch.rand(n, generator=g, device=dev) * 1e-2
    out = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    res = {}
    for lay, name in ((0, "NT"), (1, "NN"), (2, "TN")):
        k = [0]

        def run(cold):
            if cold:
                k[0] += 1
            a, b = ops[k[0] % npairs]
            A.ok(L.i8mp_int8_scaled_mm(lay, n, n, n, p(a), n, p(sa), p(b), n, p(sb), p(out), n, sp), "GEMM")

        warm = time_us(lambda: run(False), stream, iters)
        cold = time_us(lambda: run(True), stream, iters)
        res[name] = {"warm": gemm_entry(warm, n, n, n), "cold": gemm_entry(cold, n, n, n)}
        for tag, us in (("warm", warm), ("cold", cold)):
            records.append({"config": f"gemm_{n}_{tag}_operands", "shape": [n, n, n], "layout": name,
                            "kernel": "int8_scaled_mm", **gemm_entry(us, n, n, n)})
    res["note"] = f"uniform random int8 codes; cold rotates over {npairs} operand pairs ({npairs * 2 * n * n >> 20} MiB)"
    del ops
    torch.cuda.empty_cache()
    return res


def mfma_ceiling(A, codes, breakdown, stream):
    """The matrix cores' sustained rate on the GEMM's own work with the data
    path taken away (i8mp_mfma_rate_probe: the GEMM's launch shape and wave
    tile, operands in registers, 32 rounds = 2 * 4096^3 operations, the op
    count of one 4096^3 GEMM), on the step's quantized Gaussian codes and on
    uniform random bytes (the chip's power draw depends on the bits).  The
    GEMMs' share of this ceiling says how much of the gap to the 5.0 POP/s
    figure the kernel itself leaves."""
    import torch
    i8 = A.i8
    flat = codes.reshape(-1)
    rnd = torch.randint(-128, 128, (flat.numel(),), dtype=torch.int8, device=flat.device,
                        generator=torch.Generator(device=flat.device).manual_seed(3))
    sink = torch.empty(i8.MFMA_PROBE_SINK_INTS, dtype=torch.int32, device=flat.device)
    rounds = 32
    ops = rounds * 2.0**32
    out = {}
    for tag, c in (("quantized_gaussian_codes", flat), ("uniform_random_bytes", rnd)):
        us = time_us(lambda: i8.mfma_rate_probe(c, rounds, sink), stream, 20, warm=5)
        tops = ops / us / 1e6
        out[tag] = {"us": round(us, 2), "tops": round(tops, 1), "frac_int8_peak": round(tops / PEAK_INT8_TOPS, 4)}
    ceil = out["quantized_gaussian_codes"]["tops"]
    out["gemm_share_of_ceiling"] = {k: round(breakdown[k]["tops"] / ceil, 4)
                                    for k in ("gemm_NT_fwd", "gemm_NN_dgrad", "gemm_TN_wgrad")}
    return out


def torch_bf16(inputs, stream, gemm_ops):
    """torch's bf16 matmul (hipBLASLt) at the same shape and layouts."""
    a, b = inputs[0], inputs[1]
    out = {}
    for lay, fn in (("NT", lambda: a @ b.t()), ("NN", lambda: a @ b), ("TN", lambda: a.t() @ b)):
        out[lay] = round(gemm_ops / time_us(fn, stream, 10) / 1e6, 1)
    return out


def autograd_step(i8, inputs, rounding, seed, stream):
    """The layer step (forward + backward) through the autograd op against
    torch's bf16 nn.Linear at the same shape."""
    import torch
    from int8_mixed_precision_rowwise_amd.training import Int8MixedPrecisionConfig, Int8MixedPrecisionLinear
    X0, W0, dY0 = inputs
    K, N = X0.shape[1], W0.shape[0]
    lin8 = Int8MixedPrecisionLinear(K, N, Int8MixedPrecisionConfig(stochastic_rounding=rounding == "sr", seed=seed),
                                    device=X0.device)
    lin16 = torch.nn.Linear(K, N, bias=False, device=X0.device, dtype=torch.bfloat16)
    with torch.no_grad():
        lin8.weight.copy_(W0)
        lin16.weight.copy_(W0)
    xg = X0.clone().requires_grad_()

    def layer_step(lin):
        xg.grad = None
        lin.weight.grad = None
        lin(xg).backward(dY0)

    # 50 steps: the host enqueues a step of the autograd op in ~185 us against
    # ~250 us of GPU work, so short runs time the host's head start as well
    res = {tag: round(time_us(lambda: layer_step(lin), stream, 50, warm=10) / 1e3, 4)
           for tag, lin in (("int8", lin8), ("bf16", lin16))}
    res["speedup_vs_bf16"] = round(res["bf16"] / res["int8"], 3)
    return res


def fp8_step(i8, sets, M, N, K, stream, gemm_ops):
    """The same step with FP8 (E4M3) codes in place of INT8: the library's FP8
    chains with the column maxima handed from forward to backward (paired
    quantize launches, maxima folded in the GEMMs, as the INT8 step), outputs
    and workspaces allocated once."""
    import torch
    dev = sets[0][0].device
    wsf = torch.empty(i8.linear_workspace_bytes(M, N, K, False), dtype=torch.uint8, device=dev)
    wsb = torch.empty(i8.linear_workspace_bytes(M, N, K, True), dtype=torch.uint8, device=dev)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    k = [0]

    def step():
        k[0] += 1
        X, W, dY = sets[k[0] % len(sets)]
        _, cx, cw = i8.linear_fwd_fp8_colmax(X, W, out=Y, workspace=wsf)
        i8.linear_bwd_fp8(dY, X, W, workspace=wsb, dX=dX, dW=dW, colmax_x=cx, colmax_w=cw)

    ms = time_us(step, stream, 20, warm=5) / 1e3
    out = {"ms_per_step": round(ms, 4), "tops": round(3 * gemm_ops / (ms * 1e-3) / 1e12, 1),
           "note": "linear_fwd_fp8_colmax + linear_bwd_fp8 with the maxima, same inputs"}
    # the forward GEMM alone against hipBLASLt's FP8 GEMM on the same E4M3 codes
    # with the same row-wise scales (torch._scaled_mm, scale_a [M, 1], scale_b [1, N])
    X, W, _ = sets[0]
    qx, sx = i8.quantize_rowwise_fp8(X)
    qw, sw = i8.quantize_rowwise_fp8(W)
    ours = time_us(lambda: i8.fp8_scaled_mm("NT", qx, sx, qw, sw, out=Y), stream, 20)
    gemm = {"ours_us": round(ours, 2), "ours_tops": round(gemm_ops / (ours * 1e-6) / 1e12, 1)}
    try:
        a, b = qx.view(torch.float8_e4m3fn), qw.view(torch.float8_e4m3fn)
        f = lambda: torch._scaled_mm(a, b.t(), scale_a=sx.view(-1, 1), scale_b=sw.view(1, -1),  # noqa: E731
                                     out_dtype=torch.bfloat16)
        f()
        torch.cuda.synchronize()
        theirs = time_us(f, stream, 20)
        gemm.update(hipblaslt_rowwise_us=round(theirs, 2),
                    hipblaslt_rowwise_tops=round(gemm_ops / (theirs * 1e-6) / 1e12, 1))
    except (RuntimeError, TypeError) as e:  # not offered by this torch build
        gemm["hipblaslt_rowwise"] = f"unavailable: {str(e)[:80]}"
    out["gemm_NT_vs_hipblaslt"] = gemm
    return out


def single_linear_ctx(i8, stream, records):
    """The single small linear X [256, 512] @ W [512, 512].T (round to nearest
    even): forward alone and forward + backward through the chains.  Launch
    bound at this size."""
    import torch
    from workloads import linear_inputs, single_linear
    s = single_linear()
    t = linear_inputs(s, seed=0, device="cuda")
    X, W, dY = t["X"], t["W"], t["dY"]
    Y = torch.empty((s.M, s.N), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((s.M, s.K), dtype=torch.bfloat16, device="cuda")
    dW = torch.empty((s.N, s.K), dtype=torch.bfloat16, device="cuda")
    wf = torch.empty(i8.linear_workspace_bytes(s.M, s.N, s.K, False), dtype=torch.uint8, device="cuda")
    wb = torch.empty(i8.linear_workspace_bytes(s.M, s.N, s.K, True), dtype=torch.uint8, device="cuda")
    ops = 2.0 * s.M * s.N * s.K
    fwd = time_us(lambda: i8.linear_fwd(X, W, out=Y, workspace=wf), stream, 50)

    def step():
        _, cx, cw = i8.linear_fwd_colmax(X, W, out=Y, workspace=wf)
        i8.linear_bwd(dY, X, W, dX=dX, dW=dW, workspace=wb, colmax_x=cx, colmax_w=cw)

    both = time_us(step, stream, 50)
    fb16 = time_us(lambda: torch.matmul(X, W.t(), out=Y), stream, 50)
    records.append({"config": "single_linear", "shape": [s.M, s.N, s.K], "layout": "NT", "kernel": "linear_fwd",
                    "us": round(fwd, 2), "tops": round(ops / fwd / 1e6, 2)})
    records.append({"config": "single_linear", "shape": [s.M, s.N, s.K], "layout": None,
                    "kernel": "linear_fwd_colmax+linear_bwd", "us": round(both, 2), "tops": round(3 * ops / both / 1e6, 2)})
    return {"fwd_us": round(fwd, 2), "fwd_bwd_us": round(both, 2), "torch_bf16_fwd_matmul_us": round(fb16, 2)}


def context_square_sweep(i8, dev, stream, records):
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
        it = 50 if n < 4096 else 20
        row = {}
        for lay in ("NT", "NN", "TN"):
            qa, sa = i8.quantize_rowwise(a) if lay != "TN" else i8.quantize_colwise(a)
            qb, sb = i8.quantize_rowwise(b) if lay == "NT" else i8.quantize_colwise(b)
            t8 = time_us(lambda: i8.int8_scaled_mm(lay, qa, sa, qb, sb, y), stream, it)
            f16 = {"NT": lambda: torch.matmul(a, b.t(), out=y), "NN": lambda: torch.matmul(a, b, out=y),
                   "TN": lambda: torch.matmul(a.t(), b, out=y)}[lay]
            t16 = time_us(f16, stream, it)
            row[lay] = {**gemm_entry(t8, n, n, n), "bf16_us": round(t16, 2), "speedup": round(t16 / t8, 3)}
            records.append({"config": "square_gemm_sweep", "shape": [n, n, n], "layout": lay,
                            "kernel": "int8_scaled_mm", **gemm_entry(t8, n, n, n), "torch_bf16_us": round(t16, 2)})
        out[str(n)] = row
    return out


def context_quantize_large(i8, dev, stream, records):
    """The quantize passes at the Llama-1B activation sizes (X 32768 x 2048,
    dY 32768 x 5632), in algorithmic GB/s (3 bytes per element + 4 per scale)
    against the 8 TB/s HBM peak, with a torch bf16 copy of the same tensor
    (4 bytes per element moved) for scale.  Inputs rotate over more bytes than
    the 256 MB MALL, so every pass reads HBM."""
    import torch
    from workloads import gaussian_bf16
    L = i8.lib
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = Abi.p
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

        passes = {
            "row": lambda: Abi.ok(L.i8mp_quantize_rowwise(P(nxt()), R, C, C, P(q), C, P(srow), 0, 0, 0, sp), "row"),
            "row_with_colmax": lambda: Abi.ok(L.i8mp_quantize_rowwise_colmax(
                P(nxt()), R, C, C, P(q), C, P(srow), P(cm), 0, 0, 0, P(ws), ws.numel(), sp), "row+colmax"),
            "col_given_colmax": lambda: Abi.ok(L.i8mp_quantize_colwise_given_colmax(
                P(nxt()), R, C, C, P(cm), P(q), C, P(scol), 0, 0, 0, sp), "col given"),
        }
        row = {}
        for pn, fn in passes.items():
            us = time_us(fn, stream, 20)
            row[pn] = quant_entry(us, R, C, R if pn.startswith("row") else C)
            records.append({"config": "quantize_llama1b_sizes", "shape": [R, C], "layout": None,
                            "kernel": pn, **row[pn]})
        us = time_us(lambda: y.copy_(nxt()), stream, 20)
        row["torch_bf16_copy"] = {"us": round(us, 1), "gbs": round(4.0 * R * C / us / 1e3, 1)}
        out[name] = row
        del xs, q, y, ws
    torch.cuda.empty_cache()
    return out


def layer_steps(i8, dev, stream, shapes, prefix, iters, rounding, records, config):
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
            _, cx, cw = i8.linear_fwd_colmax(X, W, rounding, 7, 0, out=Y, workspace=wsf)
            i8.linear_bwd(dY, X, W, rounding, 7, 0, dX=dX, dW=dW, workspace=wsb, colmax_x=cx, colmax_w=cw)

        def step16():
            torch.matmul(X, W.t(), out=Y)
            torch.matmul(dY, W, out=dX)
            torch.matmul(dY.t(), X, out=dW)

        t8 = time_us(step8, stream, iters)
        t16 = time_us(step16, stream, iters) if rounding == "rne" else None
        nm = shape.name.replace(prefix, "")
        per[nm] = {"int8_us": round(t8, 1)}
        if t16 is not None:
            per[nm]["bf16_us"] = round(t16, 1)
            tot16 += t16
        o = 3 * 2.0 * M * N * K
        records.append({"config": config, "layer": nm, "shape": [M, N, K], "layout": None,
                        "kernel": "linear_fwd_colmax+linear_bwd", "rounding": rounding, "us": round(t8, 1),
                        "tops": round(o / t8 / 1e6, 1)})
        tot8 += t8
        ops += o
        del t, X, W, dY, Y, dX, dW, wsf, wsb
    torch.cuda.empty_cache()
    res = {"int8_us": round(tot8, 1), "int8_tops": round(ops / tot8 / 1e6, 1), "per_linear": per,
           "rounding": rounding}
    if tot16:
        res.update(bf16_gemms_us=round(tot16, 1), speedup_vs_bf16=round(tot16 / tot8, 3))
    res["note"] = f"tokens {shapes[0].M}; int8 includes all quantize passes, bf16 is the GEMMs alone"
    return res, tot16


def context_layers_both(i8, dev, stream, records):
    """The seven Llama-1B decoder linears at 16 x 2048 = 32768 tokens, each
    training step through the chains, with round to nearest even and with
    stochastic rounding in all six quantize passes."""
    from workloads import llama_1b_layers
    rne, t16 = layer_steps(i8, dev, stream, llama_1b_layers(), "llama1b_", 10, "rne", records, "llama1b_layers_rne")
    sr, _ = layer_steps(i8, dev, stream, llama_1b_layers(), "llama1b_", 10, "sr", records, "llama1b_layers_sr")
    sr["speedup_vs_bf16"] = round(t16 / sr["int8_us"], 3)
    sr["time_vs_rne"] = round(sr["int8_us"] / rne["int8_us"], 3)
    return {"rne": rne, "sr": sr}


def context_ablation(i8, dev, stream, records):
    """The pages' per-GEMM ablation (forward, grad-input, grad-weight in INT8
    or BF16, stochastic rounding on or off) at the Llama-1B linear shapes,
    through the autograd op and its toggles (a GEMM left in BF16 is torch's
    bf16 matmul): the seven linears' forward + backward time per
    configuration, and its speed-up over all-BF16."""
    import torch
    from int8_mixed_precision_rowwise_amd.training import Int8MixedPrecisionConfig, Int8MixedPrecisionLinear
    from workloads import linear_inputs, llama_1b_layers
    rows = [("bf16", None)]
    for fwd, gi, gw in ((True, False, False), (True, True, False), (True, True, True)):
        for sr in (False, True):
            tag = "int8_" + "+".join(n for n, on in (("fwd", fwd), ("dgrad", gi), ("wgrad", gw)) if on)
            rows.append((tag + ("_sr" if sr else "_rne"), Int8MixedPrecisionConfig(fwd, gi, gw, sr, seed=3)))
    tot = {tag: 0.0 for tag, _ in rows}
    for shape in llama_1b_layers():
        t = linear_inputs(shape, seed=0, device=dev)
        X, W, dY = t["X"], t["W"], t["dY"]
        xg = X.clone().requires_grad_()
        for tag, cfg in rows:
            if cfg is None:
                lin = torch.nn.Linear(shape.K, shape.N, bias=False, device=dev, dtype=torch.bfloat16)
            else:
                lin = Int8MixedPrecisionLinear(shape.K, shape.N, cfg, device=dev)
            with torch.no_grad():
                lin.weight.copy_(W)

            def step():
                xg.grad = None
                lin.weight.grad = None
                lin(xg).backward(dY)

            us = time_us(step, stream, 5, warm=2)
            tot[tag] += us
            records.append({"config": f"llama1b_ablation_{tag}", "layer": shape.name.replace("llama1b_", ""),
                            "shape": [shape.M, shape.N, shape.K], "layout": None,
                            "kernel": "autograd_linear_fwd_bwd", "us": round(us, 1)})
            del lin
        del t, X, W, dY, xg
        torch.cuda.empty_cache()
    base = tot["bf16"]
    return {"per_config_us": {k: round(v, 1) for k, v in tot.items()},
            "speedup_vs_bf16": {k: round(base / v, 3) for k, v in tot.items() if k != "bf16"},
            "note": "seven Llama-1B linears at 32768 tokens, forward + backward through the autograd op "
                    "(int8_* names the INT8 GEMMs; the others run as bf16 torch matmuls); the pages' table "
                    "reports whole-model tok/s on a 4070Ti SUPER"}


def context_llama3_8b_layers(i8, dev, stream, records):
    """The seven Llama-3-8B decoder linears and the LM head [4096 -> 128256]
    at 8192 tokens, with round to nearest even, and the same steps with
    stochastic rounding (rows of 14336 and 128256 elements take the two-read
    kernels there)."""
    from workloads import llama3_8b_layers
    res, t16 = layer_steps(i8, dev, stream, llama3_8b_layers(), "llama3_8b_", 5, "rne", records,
                           "llama3_8b_layers_rne")
    sr, _ = layer_steps(i8, dev, stream, llama3_8b_layers(), "llama3_8b_", 5, "sr", records, "llama3_8b_layers_sr")
    res["sr"] = {"int8_us": sr["int8_us"], "int8_tops": sr["int8_tops"], "time_vs_rne": round(sr["int8_us"] / res["int8_us"], 3),
                 "speedup_vs_bf16": round(t16 / sr["int8_us"], 3),
                 "per_linear_us": {k: v["int8_us"] for k, v in sr["per_linear"].items()}}
    return res


# --------------------------------------------------------------------------- CPU baseline


def cpu_baseline(tokens: int, N: int, K: int, rounding: str):
    """The CPU oracle, as it is, on the same layer step with `tokens` of the
    tokens (X [tokens, K], dY [tokens, N], W [N, K] in full): once on one core,
    then as one such sample per core on all the host's cores at once (each a
    different band of tokens; the oracle's C calls release the GIL)."""
    import oracle
    from workloads import LinearShape, bf16_bits, linear_inputs

    cores = min(16, len(os.sched_getaffinity(0)))
    t = linear_inputs(LinearShape("cpu_sample", tokens * cores, N, K), seed=0)
    X, W, dY = (bf16_bits(t[k]) for k in ("X", "W", "dY"))
    r = oracle.RNE if rounding == "rne" else oracle.SR

    def sample(i):
        band = slice(i * tokens, (i + 1) * tokens)
        oracle.linear_fwd(X[band], W, r, 1234, 0)
        oracle.linear_bwd(dY[band], X[band], W, r, 1234, 0)

    ops = 3 * 2.0 * tokens * N * K
    t0 = time.perf_counter()
    sample(0)
    one = time.perf_counter() - t0
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(cores) as ex:
        list(ex.map(sample, range(cores)))
    allc = time.perf_counter() - t0
    return {"value": round(cores * ops / allc / 1e12, 6), "unit": "TOPS", "cores": cores, "kind": "oracle",
            "seconds": round(allc, 2), "single_core_value": round(ops / one / 1e12, 6),
            "single_core_seconds": round(one, 2),
            "sample": f"oracle linear fwd+bwd (6 quantize passes + NT/NN/TN) at {tokens} tokens: X [{tokens},{K}], "
                      f"W [{N},{K}], dY [{tokens},{N}]; one sample on one core, then {cores} samples (token bands "
                      f"of one seeded draw) on {cores} threads at once"}


if __name__ == "__main__":
    main()
