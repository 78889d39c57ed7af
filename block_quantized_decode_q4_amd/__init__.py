"""MI355X-native Q4_K fused dequantize-and-multiply GEMV.

The compute lives in ``libq4k.so`` (hand-written HIP for gfx950 behind a C
ABI, declared in include/q4k.h).  ``block_quantized_decode_q4_amd.q4k`` is the
thin ctypes binding with the same entry-point names; ``synth`` holds the seeded
synthetic workload generator.
"""
