"""sink_short_window_amd: frame-sink + short-window KV-cache attention on MI355X.

The compute path lives in a C-ABI shared library (``lib/libll.so``, HIP kernels
for gfx950) declared in ``include/ll.h``; :mod:`sink_short_window_amd.ll` is the
thin ctypes binding with the same function names.  Importing the package does
not load the library; the binding loads it on first use and raises if it is
missing.
"""

__all__ = ["ll", "synth"]
