"""MI355X-native exact tiled attention (online softmax) for gfx950.

The compute path is a C-ABI shared library of hand-written HIP kernels
(``lib/libfa.so``, declared in ``include/fa.h``); ``exact_io_aware_34_amd.fa``
is its thin Python binding and raises on import when the library is missing.
``exact_io_aware_34_amd.workloads`` draws the seeded synthetic inputs.
"""
