"""MI355X-native NVFP4 hot path: block quantizer (absmax / MSE), dequantizer,
W4A16 decode GEMV and W4A4 GEMM as hand-written gfx950 HIP kernels behind a
C ABI (include/nvfp4.h).

`dit_quantization_amd.inputs` holds the seeded synthetic workloads.  The
native entry points live in `dit_quantization_amd.nvfp4` and load
libnvfp4.so on first use; a missing library is an error, never a fallback.
"""
__all__ = ["inputs", "nvfp4"]


def __getattr__(name):
    if name == "nvfp4":
        import importlib
        return importlib.import_module(__name__ + ".nvfp4")
    raise AttributeError(name)
