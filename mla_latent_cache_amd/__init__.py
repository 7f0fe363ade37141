"""Absorbed Multi-head Latent Attention decode for MI355X (gfx950).

The computation lives in ``libmla_latent.so`` (hand-written HIP kernels behind
the C ABI of ``include/mla_latent.h``); this package is its thin Python
binding.  ``ops`` wraps the five calls on torch tensors; ``step.DecodeStep``
chains them into one decode step.
"""
from ._lib import LIB_PATH, MlaError, load  # noqa: F401

__all__ = ["LIB_PATH", "MlaError", "load"]
