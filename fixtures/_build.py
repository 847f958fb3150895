"""Compile the fixture libraries in place (host: gcc; device: hipcc, gfx950)."""
import os
import subprocess

DIR = os.path.dirname(os.path.abspath(__file__))
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose=False):
    host_cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                "-o", os.path.join(DIR, "libfx.so"), os.path.join(DIR, "fx_host.c")]
    gpu_cmd = ["hipcc"] + HIP_FLAGS + ["-o", os.path.join(DIR, "libfx_gpu.so"),
                                      os.path.join(DIR, "fx_gpu.hip")]
    for cmd in (host_cmd, gpu_cmd):
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True, cwd=DIR)
