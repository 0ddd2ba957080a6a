"""Builds libdevapi_user.so: a caller's kernel that includes only the public
include/ directory of libarx (arx_device.h), for the GPU test of the public
device-side barrier. Same code-generation flags as libarx."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "devapi_user.hip")
LIB = os.path.join(HERE, "libdevapi_user.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
           "-I", os.path.join(ROOT, "include"), SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
