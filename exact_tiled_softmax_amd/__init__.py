"""Exact tiled-softmax attention for MI355X (gfx950).

The computation lives in libattn.so (C ABI in include/attn.h, HIP kernels in
csrc/).  `exact_tiled_softmax_amd.attn` is the ctypes binding; importing this
package does not load the library, so the input generators in `.inputs` stay
usable on machines without it.
"""
__all__ = ["attn", "inputs", "build"]
