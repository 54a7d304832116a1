"""MI355X-native CSA2 (Compressed Sparse Attention 2) decode/prefill hot path.

The compute lives in ``libcsa2.so`` (HIP kernels for gfx950 behind a C ABI,
declared in ``include/csa2.h``); ``csa2`` is a thin ctypes binding with the
same entry-point names.  ``synth`` draws the seeded synthetic workloads.
"""
