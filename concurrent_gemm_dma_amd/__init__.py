"""MI355X-native C3 hot path: a bf16 MFMA GEMM running concurrently with a collective-shaped
HBM copy (all-gather local share or all-to-all block transpose) moved by a CU kernel or by the
SDMA engines, under the C3 controls of issue order and CU partitioning.

The compute path is libc3.so (HIP kernels for gfx950 + ROCr SDMA + a C ABI, include/c3.h);
``concurrent_gemm_dma_amd._c3`` is its ctypes binding. ``workloads`` holds the seeded synthetic
inputs.
"""
from . import _c3  # noqa: F401
from ._c3 import *  # noqa: F401,F403
