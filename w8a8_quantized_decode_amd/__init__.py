"""A8W8 decode linears on MI355X (gfx950): HIP kernels behind a C-ABI library.

``w8a8_quantized_decode_amd.binding`` holds the ctypes binding of ``liba8w8.so``;
it is imported on first use so that the seeded input generators in ``synth`` can be
used without loading the library.
"""

import importlib

__all__ = ["binding", "synth"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
