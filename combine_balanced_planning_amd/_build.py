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


def build(verbose=False):
    srcs = [os.path.join(HERE, "csrc", s) for s in SOURCES]
    tmp = SO + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-shared", "-I", os.path.join(ROOT, "include"), *srcs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    build(verbose=True)
