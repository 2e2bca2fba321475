"""Compile the HIP library ``libzero_dp.so`` (gfx950) in-tree.

Device code is built with IEEE fp32 semantics: no fp-contraction, correctly
rounded fp32 division and square root, denormals kept, packed-fp32
instructions disabled.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libzero_dp.so")
BUILD_DIR = os.path.join(HERE, "_build")

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]
DEVICE = [f"--offload-arch={ARCH}", "-ffp-contract=off", "-fno-fast-math",
          "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
SOURCES = [("api.cpp", False), ("kernels.hip", True), ("static_scratch.hip", True), ("copy_probe.hip", True)]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose=False, extra_device_flags=()):
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for name, device in SOURCES:
        src = os.path.join(CSRC, name)
        obj = os.path.join(BUILD_DIR, name + ".o")
        if device:
            cmd = [hipcc(), *COMMON, *DEVICE, *extra_device_flags, "-x", "hip", "-c", src, "-o", obj]
        else:
            cmd = [hipcc(), *COMMON, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                   "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
