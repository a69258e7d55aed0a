"""Build step for libi8mp.so (gfx950 only), in-tree.

Each source is compiled by hipcc to an object (in parallel), then linked into
``int8_mixed_precision_rowwise_amd/libi8mp.so``.  Flags:

* ``--offload-arch=gfx950``: CDNA4 only.
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed fp32 VALU ops.
* ``-ffp-contract=off -fno-fast-math``: every float operation is one IEEE
  operation unless a kernel asks for an FMA explicitly.
* ``-fno-gpu-flush-denormals-to-zero``: bf16 subnormals are legal inputs.
* ``-fhip-fp32-correctly-rounded-divide-sqrt``: ``a / b`` is the IEEE quotient.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libi8mp.so")
SOURCES = ["i8mp_api.cpp", "quantize.hip", "gemm.hip"]
HEADERS = ["internal.h", "philox.h", os.path.join("..", "..", "include", "i8mp.h")]

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-Wall",
]


def hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _compile(src: str, obj: str) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *HIP_FLAGS, *lang, "-I", os.path.join(ROOT, "include"), "-c",
           os.path.join(CSRC, src), "-o", obj]
    subprocess.run(cmd, check=True)


def build(verbose: bool = False) -> str:
    """Compile every source and link the library; returns its path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.rsplit(".", 1)[0] + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(_compile, SOURCES, objs))
    tmp = LIB_PATH + ".tmp"
    subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                   check=True)
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(LIB_PATH)
    return LIB_PATH


def stale() -> bool:
    """True when the library is missing or older than any of its sources."""
    if not os.path.exists(LIB_PATH):
        return True
    t = os.path.getmtime(LIB_PATH)
    files = [os.path.join(CSRC, f) for f in SOURCES + HEADERS]
    return any(os.path.getmtime(f) > t for f in files if os.path.exists(f))


if __name__ == "__main__":
    build(verbose=True)
