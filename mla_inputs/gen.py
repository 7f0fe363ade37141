"""Seeded draws for the decode workloads (torch CPU generator, fixed draw order).

Draw order for ``make_inputs(spec, seed)``, all from one
``torch.Generator('cpu').manual_seed(seed)``:

1. relocation offsets ``o_b`` (if the spec has ``offset_range``);
2. per segment, in spec order: the per-request lengths (if drawn), then the
   physical page permutation (paged layout);
3. per segment, in spec order: the cache storage, N(0, 1), in fixed chunks;
4. ``q_nope`` then ``q_pe``, N(0, 1);
5. ``w_uk`` then ``w_uv``, N(0, 1) / sqrt(d_c)  (fan-in of both is ``d_c``);
6. with ``qk_norm``: the RMSNorm weights ``g_q`` then ``g_k`` [H, d_nope],
   1 + 0.1 N(0, 1), kept in fp32.

Floating tensors are then rounded to the spec dtype (bf16 rounds to nearest
even, as ``Tensor.to(torch.bfloat16)`` does).  With ``poison=True`` every
stored row that no request may read (rows past ``T_b`` in a contiguous
cache, the tail of a request's last page, spare pool pages) is set to NaN so
that a kernel which lets such a row enter its arithmetic is caught.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import torch

from .configs import Spec, SegSpec, WORKLOADS, mini_spec

_CHUNK = 1 << 24  # elements per randn call; fixed so the stream is reproducible


def _dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _randn_into(out: torch.Tensor, g: torch.Generator, mul: float = 1.0) -> None:
    flat = out.view(-1)
    n = flat.numel()
    for i in range(0, n, _CHUNK):
        m = min(_CHUNK, n - i)
        x = torch.randn(m, generator=g, dtype=torch.float32)
        if mul != 1.0:
            x.mul_(mul)
        flat[i:i + m].copy_(x.to(out.dtype))


@dataclass
class Segment:
    """One KV segment: a cache of rows ``[c_t | kr_t]`` plus its read rule."""
    name: str
    cache: torch.Tensor                 # contiguous [B, T_max, R] or paged pool [P, page, R]
    block_table: Optional[torch.Tensor]  # int32 [B, max_pages], -1 padded; None => contiguous
    seq_lens: torch.Tensor              # int32 [B]
    shift: torch.Tensor                 # int64 [B]: true position = stored position + shift
    stored_base: torch.Tensor           # int64 [B]: stored position of row 0
    head_begin: int
    head_count: int
    causal: bool
    page_size: int

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    def rows(self, b: int) -> torch.Tensor:
        """The ``T_b`` logical rows of request ``b`` in order, as stored."""
        t = int(self.seq_lens[b])
        if not self.paged:
            return self.cache[b, :t]
        ps = self.page_size
        n_pages = (t + ps - 1) // ps
        if n_pages == 0:
            return self.cache.new_empty((0, self.cache.shape[-1]))
        ids = self.block_table[b, :n_pages].long()
        return self.cache[ids].reshape(n_pages * ps, -1)[:t]


@dataclass
class MlaInputs:
    spec: Spec
    seed: int
    q_nope: torch.Tensor      # [n_tok, H, d_nope]
    q_pe: torch.Tensor        # [n_tok, H, d_rope]   unrotated
    q_pos: torch.Tensor       # int64 [n_tok]          true position of each query token
    w_uk: torch.Tensor        # [H, d_nope, d_c]
    w_uv: torch.Tensor        # [H, d_v, d_c]
    segments: List[Segment]
    offsets: torch.Tensor     # int64 [B]
    g_q: Optional[torch.Tensor] = None   # fp32 [H, d_nope]: QK-Norm query weight (spec.qk_norm)
    g_k: Optional[torch.Tensor] = None   # fp32 [H, d_nope]: QK-Norm key weight

    @property
    def scale(self) -> float:
        return self.spec.softmax_scale

    @property
    def rope_base(self) -> float:
        return self.spec.rope_base

    def token_shift(self, seg: Segment) -> torch.Tensor:
        """int64 [n_tok]: the segment's shift for each query token's request."""
        return seg.shift.repeat_interleave(self.spec.s_q)

    def cache_bytes(self) -> int:
        """Bytes of cache rows a decode step must read: every visible row once."""
        el = self.segments[0].cache.element_size()
        return sum(int(s.seq_lens.sum()) for s in self.segments) * self.spec.row_width * el


def _lengths(seg: SegSpec, batch: int, g: torch.Generator) -> torch.Tensor:
    if seg.lengths is not None:
        assert len(seg.lengths) == batch
        return torch.tensor(seg.lengths, dtype=torch.int64)
    if seg.length is not None:
        return torch.full((batch,), seg.length, dtype=torch.int64)
    lo, hi = seg.length_range
    return torch.randint(lo, hi + 1, (batch,), generator=g, dtype=torch.int64)


def make_inputs(spec: Spec, seed: int, poison: bool = False) -> MlaInputs:
    g = torch.Generator(device="cpu").manual_seed(seed)
    B, H = spec.batch, spec.heads
    dt = _dtype(spec.dtype)
    R = spec.row_width

    if spec.offset_range is not None:
        lo, hi = spec.offset_range
        offsets = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64)
    else:
        offsets = torch.zeros(B, dtype=torch.int64)

    # step 2: structure
    plans = []
    for ss in spec.segments:
        lens = _lengths(ss, B, g)
        if ss.layout == "paged":
            ps = ss.page_size
            pages = (lens + ps - 1) // ps
            total = int(pages.sum()) + ss.spare_pages
            perm = torch.randperm(total, generator=g).to(torch.int32)
            max_pages = max(1, int(pages.max()))
            bt = torch.full((B, max_pages), -1, dtype=torch.int32)
            cur = 0
            for b in range(B):
                n = int(pages[b])
                bt[b, :n] = perm[cur:cur + n]
                cur += n
            plans.append((ss, lens, bt, total))
        elif ss.layout == "contiguous":
            plans.append((ss, lens, None, None))
        else:
            raise ValueError(ss.layout)

    # step 3: caches
    segments: List[Segment] = []
    by_name = {}
    for ss, lens, bt, total in plans:
        if bt is not None:
            cache = torch.empty((total, ss.page_size, R), dtype=dt)
        else:
            cache = torch.empty((B, max(1, int(lens.max())), R), dtype=dt)
        _randn_into(cache, g)
        hc = H - ss.head_begin if ss.head_count is None else ss.head_count
        base = torch.full((B,), ss.base_extra, dtype=torch.int64)
        if ss.base_offset:
            base += offsets
        shift = offsets.clone() if ss.shift_offset else torch.zeros(B, dtype=torch.int64)
        seg = Segment(name=ss.name, cache=cache, block_table=bt, seq_lens=lens.to(torch.int32),
                      shift=shift, stored_base=base, head_begin=ss.head_begin, head_count=hc,
                      causal=ss.causal, page_size=ss.page_size)
        segments.append(seg)
        by_name[ss.name] = (ss, seg)
    for ss, seg in zip(spec.segments, segments):
        if ss.base_after is not None:
            seg.stored_base += by_name[ss.base_after][1].seq_lens.to(torch.int64)

    # step 4: queries
    n_tok = spec.n_tok
    q_nope = torch.empty((n_tok, H, spec.d_nope), dtype=dt)
    _randn_into(q_nope, g)
    q_pe = torch.empty((n_tok, H, spec.d_rope), dtype=dt)
    _randn_into(q_pe, g)

    # step 5: weights, N(0, 1/fan_in) with fan_in = d_c
    w_uk = torch.empty((H, spec.d_nope, spec.d_c), dtype=dt)
    _randn_into(w_uk, g, mul=spec.d_c ** -0.5)
    w_uv = torch.empty((H, spec.d_v, spec.d_c), dtype=dt)
    _randn_into(w_uv, g, mul=spec.d_c ** -0.5)

    # step 6: QK-Norm weights
    g_q = g_k = None
    if spec.qk_norm:
        g_q = torch.empty((H, spec.d_nope), dtype=torch.float32)
        _randn_into(g_q, g, mul=0.1)
        g_q += 1.0
        g_k = torch.empty((H, spec.d_nope), dtype=torch.float32)
        _randn_into(g_k, g, mul=0.1)
        g_k += 1.0

    # query positions: the last s_q rows of the online segment
    online = [seg for ss, seg in zip(spec.segments, segments) if ss.online]
    assert len(online) == 1, "exactly one segment holds the newest tokens"
    on = online[0]
    q_pos = torch.empty(n_tok, dtype=torch.int64)
    for b in range(B):
        for s in range(spec.s_q):
            j = int(on.seq_lens[b]) - spec.s_q + s
            q_pos[b * spec.s_q + s] = on.stored_base[b] + on.shift[b] + j

    if poison:
        for seg in segments:
            _poison(seg)

    return MlaInputs(spec=spec, seed=seed, q_nope=q_nope, q_pe=q_pe, q_pos=q_pos,
                     w_uk=w_uk, w_uv=w_uv, segments=segments, offsets=offsets, g_q=g_q, g_k=g_k)


def _poison(seg: Segment) -> None:
    if not seg.cache.dtype.is_floating_point:
        return
    nan = float("nan")
    B = seg.seq_lens.numel()
    if not seg.paged:
        for b in range(B):
            seg.cache[b, int(seg.seq_lens[b]):] = nan
        return
    used = torch.zeros(seg.cache.shape[0], dtype=torch.bool)
    ps = seg.page_size
    for b in range(B):
        t = int(seg.seq_lens[b])
        n = (t + ps - 1) // ps
        ids = seg.block_table[b, :n].long()
        used[ids] = True
        if n and t % ps:
            seg.cache[ids[-1], t % ps:] = nan
    seg.cache[~used] = nan


def make(name: str, seed: int, mini: bool = False, poison: bool = False) -> MlaInputs:
    spec = mini_spec(name) if mini else WORKLOADS[name]
    return make_inputs(spec, seed, poison=poison)
