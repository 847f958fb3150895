"""Seeded synthetic inputs shared by the oracle and the GPU path.

This package holds no arithmetic of the decode step: it draws weights, KV,
tokens, contexts and page orders from one counter-based generator (fx.h)
and writes them into plain storage formats. The host library (libfx.so) is
the definition; the device library (libfx_gpu.so) reproduces it bit for bit.
"""
from . import host  # noqa: F401
from .workloads import WORKLOADS, SIGMA_W, SIGMA_KV, NORM_GAIN_BITS, workload, resolve  # noqa: F401
from .hostmodel import HostWeights, HostKV  # noqa: F401
