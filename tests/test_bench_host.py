"""bench.py's host-side contract, without a GPU: the one-GPU rule, argument
checks that run before any device work, the digest gate on committed counter
summaries, and the algorithmic byte and operation counts it reports."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_unknown_context_is_rejected_before_device_work():
    with pytest.raises(SystemExit):
        bench.parse(["--context", "llama1b,nonsense"])
    a = bench.parse(["--context", "llama1b,fp8"])
    assert a.context == "llama1b,fp8" and a.gpus == 1
    d = bench.parse([])
    assert (d.steps, d.warmup, d.size, d.rounding, d.context) == (50, 10, 4096, "rne", None)


def test_counter_summary_is_read_only_on_matching_sources(tmp_path):
    files = ("gemm.hip", "internal.h")
    good = tmp_path / "good.txt"
    good.write_text(f"# comment: ignored\nkernel_source_sha256_16: {bench.source_digest(files)}\n"
                    "hbm_bytes_per_dispatch_gemm_NN_dgrad: 1234\n")
    f = bench.read_summary(str(good), files)
    assert f["hbm_bytes_per_dispatch_gemm_NN_dgrad"] == "1234"
    stale = tmp_path / "stale.txt"
    stale.write_text("kernel_source_sha256_16: 0000000000000000\nhbm_bytes_per_dispatch_gemm_NN_dgrad: 1\n")
    assert bench.read_summary(str(stale), files) is None
    assert bench.read_summary(str(tmp_path / "missing.txt"), files) is None


def test_algorithmic_counts():
    # a quantize pass: 2 bytes read and 1 written per element, 4 per scale
    assert bench.quant_bytes(4096, 4096, 4096) == 3 * 4096 * 4096 + 4 * 4096
    e = bench.quant_entry(10.0, 4096, 4096, 4096)
    assert e["gbs"] == pytest.approx(bench.quant_bytes(4096, 4096, 4096) / 10e-6 / 1e9, rel=1e-4)
    g = bench.gemm_entry(50.0, 4096, 4096, 4096)
    assert g["tops"] == pytest.approx(2 * 4096 ** 3 / 50e-6 / 1e12, rel=1e-3)
    assert g["frac_int8_peak"] == pytest.approx(g["tops"] / bench.PEAK_INT8_TOPS, abs=1e-4)
    assert bench.PEAK_VALU_LANE_OPS == pytest.approx(256 * 4 * 16 * 2.4e9)
