"""Compile libmk.so (host planner/pool + gfx950 megakernel) in place."""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
HOST_SRC = ["mk_common.cpp", "mk_plan.cpp"]
HIP_SRC = ["megakernel.hip"]
ARCH = "gfx950"
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]
INC = ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def build(verbose=False, extra=()):
    out_dir = os.path.join(CSRC, "_build")
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in HOST_SRC:
        o = os.path.join(out_dir, src + ".o")
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-c", os.path.join(CSRC, src),
               "-o", o, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"] + INC
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True)
        objs.append(o)
    for src in HIP_SRC:
        o = os.path.join(out_dir, src + ".o")
        cmd = ["hipcc"] + HIP_FLAGS + list(extra) + INC + ["-c", os.path.join(CSRC, src), "-o", o]
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True)
        objs.append(o)
    lib = os.path.join(PKG, "libmk.so")
    cmd = ["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", lib] + objs
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return lib


if __name__ == "__main__":
    build(verbose=True)
