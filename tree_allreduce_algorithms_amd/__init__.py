"""MI355X-native ring / tree collectives over N rank buffers on one GPU.

The collectives live in a C-ABI shared library (``libar.so``, HIP kernels for
gfx950) and this package is a thin ctypes binding with the same names.  The
library is loaded on first use; if it has not been built the call raises.
"""
