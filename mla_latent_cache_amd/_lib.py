"""ctypes binding of ``libmla_latent.so`` (the C ABI in ``include/mla_latent.h``).

Marshalling only: every step of the decode path runs in the library's HIP
kernels.  Importing this module fails loudly if the library has not been
built; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int, c_int64, c_void_p

# The in-tree build; MLA_LATENT_LIB names another build of the same sources
# (the host-sanitizer build of the C ABI that the CPU tests load).
LIB_PATH = os.environ.get("MLA_LATENT_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                            "libmla_latent.so")

MLA_F32 = 0
MLA_BF16 = 1
MLA_I8 = 2  # cache format: int8 latent codes + bf16 rotary entries per row, fp32 scale per row
MLA_I4 = 3  # cache format: 4-bit latent and rotary codes per row, two fp32 scales per row
MLA_BF16X2 = 4  # query format: bf16 hi and lo planes of fp32 values, [..][2][d]

STATUS = {0: "MLA_OK", 1: "MLA_ERR_NULL", 2: "MLA_ERR_SHAPE", 3: "MLA_ERR_DTYPE", 4: "MLA_ERR_ALIGN",
          5: "MLA_ERR_UNSUPPORTED", 6: "MLA_ERR_WORKSPACE", 7: "MLA_ERR_HIP"}


class MlaSegment(ctypes.Structure):
    """Mirror of ``mla_segment``."""
    _fields_ = [
        ("cache", c_void_p),
        ("block_table", c_void_p),
        ("seq_lens", c_void_p),
        ("q_rot", c_void_p),
        ("max_rows", c_int64),
        ("page_size", c_int),
        ("max_pages", c_int),
        ("n_pages", c_int),
        ("head_begin", c_int),
        ("head_count", c_int),
        ("causal", c_int),
        ("part_begin", c_int),
        ("n_split", c_int),
        ("row_rinv", c_void_p),
        ("row_scale", c_void_p),
    ]


# name -> (restype, argtypes), exactly the declarations of include/mla_latent.h
SIGNATURES = {
    "rope_relocate_q": (c_int, [c_void_p, c_int, c_void_p, c_int, c_void_p, c_void_p, c_int, c_int, c_int,
                                c_double, c_void_p]),
    "mla_absorb_q": (c_int, [c_void_p, c_void_p, c_int, c_void_p, c_int, c_int, c_int, c_int, c_int,
                             c_void_p]),
    "mla_decode_splitkv": (c_int, [POINTER(MlaSegment), c_int, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                   c_int, c_int, c_float, c_void_p, c_int, c_void_p, c_int, c_int, c_void_p]),
    "mla_combine_lse": (c_int, [c_void_p, c_int, c_void_p, c_int, c_int, c_int, c_void_p, c_int, c_void_p,
                                c_void_p]),
    "mla_out_uv": (c_int, [c_void_p, c_int, c_void_p, c_int, c_void_p, c_int, c_int, c_int, c_int, c_int,
                           c_void_p]),
    "mla_out_proj": (c_int, [c_void_p, c_int, c_void_p, c_int, c_void_p, c_int, c_int, c_int, c_int,
                             c_void_p]),
    "mla_combine_out_uv": (c_int, [c_void_p, c_int, c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_int, c_int,
                                   c_void_p, c_void_p, c_void_p, c_int, c_void_p]),
    "mla_prepare_q": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_int, c_void_p, c_int, POINTER(c_void_p),
                              POINTER(c_void_p), c_int, c_int, c_void_p, c_int, c_int, c_int, c_int, c_int,
                              c_double, c_void_p]),
    "mla_prepare_q_qknorm": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_float, c_void_p, c_void_p, c_int,
                                     c_void_p, c_int, POINTER(c_void_p), POINTER(c_void_p), c_int, c_int, c_void_p,
                                     c_int, c_int, c_int, c_int, c_int, c_double, c_void_p]),
    "mla_quantize_latent_i8": (c_int, [c_void_p, c_int, c_int64, c_int, c_int, c_void_p, c_void_p, c_void_p]),
    "mla_quantize_latent_i4": (c_int, [c_void_p, c_int, c_int64, c_int, c_int, c_void_p, c_void_p, c_void_p]),
    "mla_qknorm_query": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_int, c_int, c_int, c_double, c_void_p,
                                 c_void_p]),
    "mla_qknorm_key_gram": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_void_p]),
    "mla_qknorm_key_rinv": (c_int, [c_void_p, c_int, c_int64, c_int, c_void_p, c_int, c_int, c_int, c_double,
                                    c_void_p, c_void_p]),
    "mla_status_string": (ctypes.c_char_p, [c_int]),
    "mla_last_error": (ctypes.c_char_p, []),
    "mla_version": (c_int, []),
    "mla_device_cu_count": (c_int, []),
    "mla_decode_shares": (c_int, [c_int, c_int, c_int]),
}

_lib = None


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


def load() -> ctypes.CDLL:
    """Load the library (once).  Raises if it is missing: build it first with
    ``python -m mla_latent_cache_amd.build``."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"MLA HIP library not built: {LIB_PATH} is missing "
                           "(run `python -m mla_latent_cache_amd.build`)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def call(name: str, *args) -> None:
    """Call an entry point returning mla_status; raise MlaError on failure."""
    lib = load()
    st = getattr(lib, name)(*args)
    if st != 0:
        raise MlaError(name, st, lib.mla_last_error().decode())
