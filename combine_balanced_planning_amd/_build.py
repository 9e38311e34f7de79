"""Build step for libmoon.so (hipcc, gfx950), in-tree next to this file."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SO = os.path.join(HERE, "libmoon.so")
SOURCES = ["moon_api.hip", "moon_plan.hip", "moon_dispatch.hip", "moon_combine.hip",
           "moon_weights.hip"]

# -ffp-contract=off keeps combine's multiply and add separate (no fused
# multiply-add), so its rounding is the one the accumulation order defines.
# Packed fp32 instructions are switched off for all HIP code.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


# Reference kernels of the benchmark (memory-system ceilings for the access
# patterns of dispatch and combine); a library of their own, not part of
# libmoon.
CEILING_SO = os.path.join(HERE, "libmoon_ceiling.so")
CEILING_SOURCES = ["moon_ceiling.hip"]


def _hipcc_shared(sources, so, verbose):
    srcs = [os.path.join(HERE, "csrc", s) for s in sources]
    tmp = so + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-shared", "-I", os.path.join(ROOT, "include"), *srcs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, so)
    return so


def build(verbose=False):
    _hipcc_shared(CEILING_SOURCES, CEILING_SO, verbose)
    return _hipcc_shared(SOURCES, SO, verbose)


# A C11 program that uses libmoon.so through include/moon.h only (hipMalloc'd
# pointers, no Python); the GPU tests run it.  Host code, built with gcc.
C_EXAMPLE_SRC = os.path.join(ROOT, "tests", "c_abi_example.c")
C_EXAMPLE_BIN = os.path.join(ROOT, "tests", "c_abi_example.bin")


def build_c_example(verbose=False):
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           C_EXAMPLE_SRC, "-o", C_EXAMPLE_BIN + ".tmp", "-L", HERE, "-lmoon",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../combine_balanced_planning_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(C_EXAMPLE_BIN + ".tmp", C_EXAMPLE_BIN)
    return C_EXAMPLE_BIN


if __name__ == "__main__":
    build(verbose=True)
    build_c_example(verbose=True)
