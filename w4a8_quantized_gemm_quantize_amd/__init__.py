"""Block-scaled int8 activation quantization + W4A8 grouped GEMM on MI355X (gfx950).

The compute lives in the HIP library ``libw4a8.so`` (C ABI, ``include/w4a8.h``).
``binding`` marshals torch tensors to that ABI; importing it loads the library
and raises if it is missing.  ``inputs`` holds the seeded input generators.
"""
import importlib

__all__ = ["binding", "inputs"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
