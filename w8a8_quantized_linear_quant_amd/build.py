"""Build the gfx950 HIP library libw8a8.so in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only and linked into one
shared library exporting the C ABI of include/w8a8.h.  Usable as a script
(`python -m w8a8_quantized_linear_quant_amd.build`) or via build_library().
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw8a8.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["act_quant.hip", "weight_quant.hip", "gemm.hip", "svdq.hip", "q8_0.hip", "gguf_a8.hip", "svd_prep.hip", "hadamard.hip", "probe.hip",
           "status.cpp"]
HEADERS = ["common.hpp", "internal.hpp", "act_quant.hpp"]  # shared by the sources above

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++20", "-fPIC", "--offload-arch=gfx950",
    # packed-f32 instructions stay off: hipcc would otherwise form them from
    # ordinary float code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(src):
    obj = os.path.join(OBJDIR, src + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-O2", "-std=c++17", "-fPIC", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj, err


def build_library(verbose=False, jobs=None):
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    for (obj, err) in results:
        if verbose and err.strip():
            print(err)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
