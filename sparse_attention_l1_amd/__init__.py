"""MI355X-native HSA (Heterogeneous Step Allocation) denoise-iteration path.

The compute lives in ``libhsastep.so`` (hand-written HIP kernels for gfx950 behind
a C ABI, declared in ``include/hsastep.h``).  ``sparse_attention_l1_amd.hsastep``
is the thin ctypes binding; importing it fails loudly when the library is absent.
``sparse_attention_l1_amd.synth`` holds the seeded synthetic workloads.
"""
