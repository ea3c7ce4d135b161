"""quantized_gemv_kv_amd — the quantized speech-token decode step on MI355X (gfx950).

The compute lives in libtsd.so (hand-written HIP kernels behind a C ABI, include/tsd.h); the
Python side (binding.py) only marshals arguments.  Importing the package does not load the
library; the first call does, and raises if it has not been built.
"""
from . import binding, roofline, synth  # noqa: F401
from .binding import Model, TsdError, lib  # noqa: F401
