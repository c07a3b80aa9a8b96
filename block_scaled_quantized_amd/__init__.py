"""block_scaled_quantized_amd: block-scaled (MX) quantized GEMM and dequant matvec for MI355X.

The compute lives in ``libmxgemm.so`` (hand-written gfx950 HIP kernels behind a C ABI declared in
``include/mxgemm.h``). ``api`` is a thin ctypes binding with the same entry-point names; it only
marshals arguments. ``synth`` draws seeded synthetic inputs.
"""
from . import synth  # noqa: F401

__all__ = ["synth", "api"]


def __getattr__(name):
    if name == "api":
        import importlib
        return importlib.import_module(__name__ + ".api")
    raise AttributeError(name)
