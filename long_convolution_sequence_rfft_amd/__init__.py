"""MI355X-native Hyena long-convolution chain (causal 1D and non-causal 2D).

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``libhyena_mi355x.so``); ``hyena`` is its thin ctypes binding.  Import
of this package does not load the library; the binding loads it on first use
and raises if it is missing.
"""
