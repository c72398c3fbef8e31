"""Dual-AR (Fish Audio S2) per-frame decode on AMD Instinct MI355X (gfx950).

The compute lives in libdualar.so (hand-written HIP kernels behind the C ABI
of include/dualar.h); `binding` marshals arguments to it with ctypes.
"""
from . import reporting  # noqa: F401
from .binding import DualAR, DualARError, load_library  # noqa: F401
