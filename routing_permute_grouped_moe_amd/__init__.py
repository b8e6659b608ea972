"""MI355X-native MoE expert layer: routing, permute, grouped SwiGLU GEMM,
unpermute/combine and their backward, as hand-written HIP kernels behind a
C ABI (``include/moe.h``).  ``abi`` is the ctypes binding; ``layer`` strings
the calls together for one layer."""

__all__ = ["abi", "layer"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
