"""Build libfp8fg.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Flags: -O3, no fast-math, no FP contraction (every FMA in the kernels is written explicitly),
packed-FP32 instructions disabled, IEEE fp32 division (HIP's default correctly rounded divide).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp8fg.so")
SOURCES = ["api.hip", "quant.hip", "gemm.hip", "per_tensor.hip", "e5m6.hip", "limited_accum.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def flags():
    return ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False, extra=()) -> str:
    objs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, src.replace(".hip", ".o"))
        cmd = [HIPCC, *flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            sys.stderr.write(err + "\n")
            raise RuntimeError(f"hipcc failed on {src}")
        if err.strip() and verbose:
            sys.stderr.write(err + "\n")
        objs.append(obj)
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    # The library must load with every symbol resolved: a kernel missing from the host object (its launch
    # stub not emitted) shows up only here, as an undefined symbol.
    r = subprocess.run([sys.executable, "-c", "import ctypes, sys; ctypes.CDLL(sys.argv[1], mode=ctypes.RTLD_LOCAL)",
                        LIB + ".tmp"], capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stderr + "\n")
        raise RuntimeError("the built library does not load: " + r.stderr.strip().splitlines()[-1])
    os.replace(LIB + ".tmp", LIB)
    return LIB


C_CONSUMER = os.path.join(ROOT, "tests", "c_consumer")


def build_c_consumer(verbose: bool = False) -> str:
    """tests/c_consumer: a C++ program that calls the library through include/fp8fg.h only (the GPU test
    tests/test_gpu_c_consumer.py runs it); linked against libfp8fg.so in this package directory."""
    cmd = [HIPCC, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_consumer.cpp"),
           "-L", HERE, "-lfp8fg", "-Wl,-rpath,$ORIGIN/../fp8_fine_grained_amax_amd", "-o", C_CONSUMER + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stderr + "\n")
        raise RuntimeError("hipcc failed on tests/c_consumer.cpp")
    os.replace(C_CONSUMER + ".tmp", C_CONSUMER)
    return C_CONSUMER


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
