"""Seeded synthetic inputs for absorbed-MLA decode.

This module is shared by the tests, the benchmark and the smoke check.  It
holds random draws, bf16 rounding, page tables and position bookkeeping, and
none of the attention arithmetic: it neither rotates, projects nor softmaxes.
Both the CPU oracle and the GPU path receive exactly the tensors built here.

Semantics of the tensors (the meaning, not a computation done here):

* A cache row is ``[c_t | kr_t]`` with ``d_c + d_rope`` numbers: the shared
  content latent and the decoupled rotary key, stored as one row (the MLA
  tutorial page, "Count the Cache That Is Actually Stored").
* ``kr_t`` is stored *already rotated* at its stored position.  A Gaussian
  pair rotated by any angle is still a standard Gaussian pair, so the stored
  rotary keys are drawn directly as N(0, 1).
* A segment's ``shift[b]`` is the amount that must be added to a stored
  position to obtain the true position in request ``b`` (nonzero only for a
  document cached at canonical position 0, the RedKnot-MLA abstract).
"""
from .configs import WORKLOADS, Spec, SegSpec, spec_for, mini_spec
from .gen import MlaInputs, Segment, make_inputs, make

__all__ = [
    "WORKLOADS", "Spec", "SegSpec", "spec_for", "mini_spec",
    "MlaInputs", "Segment", "make_inputs", "make",
]
