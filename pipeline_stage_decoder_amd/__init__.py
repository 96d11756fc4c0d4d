"""One pipeline stage of a decoder-only transformer on MI355X (gfx950): HIP kernels behind a C ABI.

The C ABI is ``include/stage.h``; ``stage.py`` is its ctypes binding; ``accounting.py`` holds the
algorithmic byte and flop counts used to report throughput against the HBM and MFMA rooflines.
"""
from .stage import Stage, StageError, lib, plan  # noqa: F401
