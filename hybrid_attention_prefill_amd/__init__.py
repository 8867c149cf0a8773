"""HYPIC linear-attention position-independent caching: the data-parallel hot
path (segment build, compose, seam advance) as gfx950 HIP kernels behind the C
ABI in include/hypic.h.

    from hybrid_attention_prefill_amd import binding   # ctypes binding of libhypic.so
    from hybrid_attention_prefill_amd import workloads # seeded synthetic inputs

The binding loads the library on first use and raises if it is missing.
"""
__all__ = ["binding", "workloads"]
