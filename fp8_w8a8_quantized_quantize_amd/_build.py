"""Build libfp8w8a8.so (the C-ABI library and its gfx950 kernels) in place."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp8w8a8.so")
SOURCES = ["abi.cpp", "quantize.hip", "calibrate.hip", "kv_cache.hip", "block_scale.hip", "gemm_skinny.hip", "gemm_tiled.hip", "gemm_mfma.hip", "stream_read.hip", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def hipcc_flags():
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        # IEEE fp32: correctly rounded division, denormals kept, no fast-math
        "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
        # no packed-fp32 instructions in generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-result",
        "-I" + os.path.join(ROOT, "include"),
    ]


def build(verbose: bool = False) -> str:
    srcs = []
    for s in SOURCES:
        p = os.path.join(CSRC, s)
        srcs += (["-x", "hip", p] if s.endswith(".hip") else ["-x", "hip", p])
    cmd = [HIPCC] + hipcc_flags() + srcs + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libfp8w8a8.so")
    if verbose and (r.stdout or r.stderr):
        print((r.stdout + r.stderr)[-4000:])
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
