"""Workload shapes: the five decode configurations and scaled-down variants.

Each ``Spec`` fixes dimensions, dtype, softmax scale, RoPE base and a list of
KV segments.  Nothing here computes; ``gen.make_inputs`` draws the tensors.

Position bookkeeping per segment and request ``b`` (``o_b`` is the request's
relocation offset, zero unless the spec draws offsets):

* stored position of row ``j``  = ``(o_b if base_offset else 0) + base_extra
  + (T_b of segment base_after, if set) + j``
* true position of row ``j``    = stored position + ``shift_b``
* ``shift_b`` = ``o_b`` if ``shift_offset`` else 0

The query tokens of request ``b`` are the last ``s_q`` rows of the segment
flagged ``online`` (the newest tokens), so query ``s`` sits at the true
position of that segment's row ``T_b - s_q + s``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class SegSpec:
    name: str
    # Either a fixed length for every request or a uniform integer range.
    length: Optional[int] = None
    length_range: Optional[Tuple[int, int]] = None   # inclusive
    lengths: Optional[Tuple[int, ...]] = None         # explicit per-request
    layout: str = "contiguous"                        # "contiguous" | "paged"
    page_size: int = 64
    spare_pages: int = 0                              # unused pool pages (poisoned in parity runs)
    head_begin: int = 0
    head_count: Optional[int] = None                  # None => all heads
    causal: bool = False
    base_offset: bool = False
    base_extra: int = 0
    base_after: Optional[str] = None                  # add this segment's length to the base
    shift_offset: bool = False
    online: bool = False


@dataclass(frozen=True)
class Spec:
    name: str
    batch: int
    heads: int
    d_c: int
    d_nope: int
    d_rope: int
    d_v: int
    s_q: int
    dtype: str                    # "f32" | "bf16"
    segments: Tuple[SegSpec, ...]
    rope_base: float = 10000.0
    scale: Optional[float] = None  # None => 1/sqrt(d_nope + d_rope)
    offset_range: Optional[Tuple[int, int]] = None  # o_b ~ U{lo..hi}, inclusive
    qk_norm: bool = False          # RMSNorm of the content query and key (weights g_q, g_k drawn)
    qk_eps: float = 1e-6
    quant: Optional[str] = None    # "int8" / "int4": the cache holds per-row low-bit codes (each side quantizes
                                   # the drawn bf16 rows itself; nothing extra is drawn)
    description: str = ""

    @property
    def softmax_scale(self) -> float:
        if self.scale is not None:
            return self.scale
        return 1.0 / math.sqrt(self.d_nope + self.d_rope)

    @property
    def row_width(self) -> int:
        return self.d_c + self.d_rope

    @property
    def n_tok(self) -> int:
        return self.batch * self.s_q


def _dsv3_dims():
    return dict(d_c=512, d_nope=128, d_rope=64, d_v=128)


# The five decode configurations, in the order the benchmark description lists them.
WORKLOADS = {
    "toy": Spec(
        name="toy", batch=1, heads=2, d_c=4, d_nope=4, d_rope=2, d_v=4, s_q=1, dtype="f32",
        segments=(SegSpec("kv", length=16, online=True),),
        description="toy fp32: B=1, H=2, d_c=4, d_nope=4, d_rope=2, d_v=4, T=16, positions 0..15",
    ),
    "small": Spec(
        name="small", batch=4, heads=16, s_q=1, dtype="bf16", **_dsv3_dims(),
        segments=(SegSpec("kv", length=4096, online=True),),
        description="small bf16: B=4, H=16, T=4096 contiguous, 1 query token",
    ),
    "dsv3": Spec(
        name="dsv3", batch=64, heads=128, s_q=1, dtype="bf16", **_dsv3_dims(),
        segments=(SegSpec("kv", length_range=(1024, 32768), layout="paged", page_size=64,
                          online=True),),
        description="DeepSeek-V3-style: B=64, H=128, T~U[1024,32768], 64-row pages, shuffled block table",
    ),
    "long": Spec(
        name="long", batch=4, heads=64, s_q=1, dtype="bf16", **_dsv3_dims(),
        segments=(SegSpec("kv", length=262144, online=True),),
        description="long-context: B=4, H=64, T=262144 contiguous, split-KV <= 256 chunks",
    ),
    "merge": Spec(
        name="merge", batch=16, heads=64, s_q=4, dtype="bf16", **_dsv3_dims(),
        offset_range=(0, 200000),
        segments=(
            # document cached once at canonical position 0, read by the Local heads
            SegSpec("doc_off", length=16384, head_begin=0, head_count=56, shift_offset=True),
            # the same document recomputed in context (true positions), read by the Global heads
            SegSpec("doc_on", length=16384, head_begin=56, head_count=8, base_offset=True),
            # the online tokens after the document, read by every head, causal
            SegSpec("online", length=2048, causal=True, base_offset=True, base_after="doc_on",
                    online=True),
        ),
        description="offline/online segment merge: B=16, H=64 (56 Local / 8 Global), S_q=4, "
                    "16384-row document + 2048-row online segment, offsets U[0,200000]",
    ),
}

# A multi-token query chunk over the merge layout (RedKnot-MLA abstract: the
# online path recomputes in context, in chunks): the same relocated document
# and online segments, read by a 64-token chunk, so every segment serves
# 64 x heads query rows and the pass is bound by the MFMA units, not HBM.
WORKLOADS["prefill"] = replace(
    WORKLOADS["merge"], name="prefill", batch=4, s_q=64,
    description="chunked prefill over relocated segments: B=4, H=64 (56 Local / 8 Global), a 64-token query "
                "chunk, 16384-row document + 2048-row online segment, offsets U[0,200000]")

# The small configuration with QK-Norm (QK-Norm MLA page, abstract): the
# content query and key RMS-normalised after their projections.
WORKLOADS["qknorm"] = replace(
    WORKLOADS["small"], name="qknorm", qk_norm=True,
    description="small bf16 with QK-Norm: B=4, H=16, T=4096 contiguous, 1 query token, RMSNorm of the "
                "content query and key")

# The long-context configuration read from an int8 latent cache (QuantMLA
# abstract: low-bit latent caching; here per-row symmetric int8 codes, the
# rotary key kept 16-bit).  The drawn rows are the same bf16 rows; each side
# quantizes them itself.
WORKLOADS["int8"] = replace(
    WORKLOADS["long"], name="int8", quant="int8",
    description="long context from an int8 latent cache: B=4, H=64, T=262144 contiguous, 1 query token; "
                "per-row int8 latent codes + bf16 rotary key (640 B + a 4 B scale per row)")

# The long-context configuration read from an int4 cache (QuantMLA abstract:
# joint INT4 caching of the content and rotary caches; here per-row
# symmetric 4-bit codes for both parts, each with its own scale).  Again each
# side quantizes the drawn bf16 rows itself.
WORKLOADS["int4"] = replace(
    WORKLOADS["long"], name="int4", quant="int4",
    description="long context from an int4 cache: B=4, H=64, T=262144 contiguous, 1 query token; "
                "per-row 4-bit latent and rotary codes (288 B + two 4 B scales per row)")

# The DeepSeek-V3-style batch with QK-Norm (QK-Norm MLA abstract): 128 heads
# per request, so the row factors ride on the 128-row groups of the decode.
WORKLOADS["qknorm_dsv3"] = replace(
    WORKLOADS["dsv3"], name="qknorm_dsv3", qk_norm=True,
    description="DeepSeek-V3-style with QK-Norm: B=64, H=128, T~U[1024,32768], 64-row pages, shuffled block "
                "table, RMSNorm of the content query and key")

# Order of the configurations as listed by the benchmark description.
WORKLOAD_ORDER = ("toy", "small", "dsv3", "long", "merge")
# Further workloads (beyond the five configurations)
EXTRA_WORKLOADS = ("prefill", "qknorm", "int8", "int4", "qknorm_dsv3")


def spec_for(name: str) -> Spec:
    return WORKLOADS[name]


def mini_spec(name: str) -> Spec:
    """Scaled-down variant of a configuration that the fp64 oracle finishes in
    seconds, keeping the head count, dims, layout and segment structure and
    leaving several 32/64-row tiles plus ragged tails in every request."""
    s = WORKLOADS[name]
    if name == "toy":
        return s
    if name == "small":
        return replace(s, name="small-mini", batch=3,
                       segments=(SegSpec("kv", lengths=(1, 129, 777), online=True),))
    if name == "dsv3":
        return replace(s, name="dsv3-mini", batch=5,
                       segments=(SegSpec("kv", lengths=(700, 64, 1, 333, 1000), layout="paged",
                                         page_size=64, spare_pages=3, online=True),))
    if name == "long":
        return replace(s, name="long-mini", batch=2,
                       segments=(SegSpec("kv", lengths=(3000, 2113), online=True),))
    if name == "merge":
        segs = (
            replace(s.segments[0], length=None, lengths=(300, 97, 129)),
            replace(s.segments[1], length=None, lengths=(300, 97, 129)),
            replace(s.segments[2], length=None, lengths=(70, 4, 65)),
        )
        return replace(s, name="merge-mini", batch=3, segments=segs)
    if name == "qknorm_dsv3":
        return replace(s, name="qknorm_dsv3-mini", batch=5,
                       segments=(SegSpec("kv", lengths=(700, 64, 1, 333, 1000), layout="paged",
                                         page_size=64, spare_pages=3, online=True),))
    if name == "qknorm":
        return replace(s, name="qknorm-mini", batch=3,
                       segments=(SegSpec("kv", lengths=(1, 129, 777), online=True),))
    if name == "int8":
        return replace(s, name="int8-mini", batch=3,
                       segments=(SegSpec("kv", lengths=(1, 777, 2113), layout="paged", page_size=64,
                                         spare_pages=2, online=True),))
    if name == "int4":
        return replace(s, name="int4-mini", batch=3,
                       segments=(SegSpec("kv", lengths=(1, 777, 2113), layout="paged", page_size=64,
                                         spare_pages=2, online=True),))
    if name == "prefill":
        segs = (
            replace(s.segments[0], length=None, lengths=(300, 97)),
            replace(s.segments[1], length=None, lengths=(300, 97)),
            replace(s.segments[2], length=None, lengths=(70, 64)),   # >= s_q: the chunk is the newest rows
        )
        return replace(s, name="prefill-mini", batch=2, segments=segs)
    raise KeyError(name)
