"""Compile ``step_demo``, a plain C program that drives the library through
its C ABI alone (no torch, no Python), against the in-tree libzero_dp.so."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "zero_dp_partitioned_amd")
EXE = os.path.join(HERE, "step_demo")


def build(verbose=False):
    src = os.path.join(HERE, "step_demo.c")
    tmp = EXE + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", src,
           "-L", PKG, "-lzero_dp", "-L", "/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../zero_dp_partitioned_amd", "-Wl,-rpath,/opt/rocm/lib", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
