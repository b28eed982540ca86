"""MI355X-native fused Conv2d + folded BatchNorm + SiLU (FP32 / INT8).

The compute path is libcbs.so (hand-written HIP for gfx950, C ABI in
include/cbs.h); ``convolution_implicit_gemm_02_amd.cbs`` is its thin ctypes
binding and ``workloads`` the seeded synthetic inputs.  Importing the binding
fails loudly when libcbs.so has not been built.
"""
import importlib

__all__ = ["cbs", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
