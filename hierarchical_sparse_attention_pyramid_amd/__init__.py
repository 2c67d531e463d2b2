"""Lighthouse attention layer for AMD Instinct MI355X (gfx950).

The compute path is the HIP library liblighthouse.so (C ABI in
include/lighthouse.h); `binding` is its ctypes marshalling layer.
"""
from . import binding  # noqa: F401
from .binding import backward, forward  # noqa: F401
