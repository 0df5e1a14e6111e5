"""MI355X-native sparse MoE fine-tuning hot path (USAF-style), HIP for gfx950.

The product is the C-ABI library libusaf.so (include/usaf.h).  This package
holds its HIP sources (csrc/), the in-tree build (build.py), a ctypes binding
(capi.py) and a thin layer object that sequences the calls of one step
(layer.py).  Importing `capi` fails loudly when libusaf.so is not built.
"""
__all__ = ["capi", "layer", "build"]
