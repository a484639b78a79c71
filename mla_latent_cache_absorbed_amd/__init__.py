"""Absorbed-weight Multi-head Latent Attention decode for MI355X (gfx950).

The compute lives in ``libmla_decode.so`` (hand-written HIP kernels behind a
C ABI declared in ``include/mla_decode.h``).  ``binding`` marshals torch
tensors into that ABI and nothing else; ``inputs`` draws seeded synthetic
workloads.  Importing the package does not load the library: the first call
into ``binding`` does, and fails loudly when it is missing.
"""

__all__ = ["binding", "inputs"]
