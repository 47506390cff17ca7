"""MI355X-native block-sparse decode attention (Elastic Threshold Attention).

``binding``  ctypes binding of libeta.so (HIP kernels for gfx950, C ABI in
             include/eta.h); fails loudly when the library is not built.
``synth``    seeded synthetic workloads (inputs only).
``build``    in-tree build of libeta.so with hipcc.
"""
__all__ = ["binding", "synth", "build"]
