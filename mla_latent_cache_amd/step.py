"""One decode step of one attention layer: the five calls, with buffers.

``DecodeStep`` owns the device buffers of the chain

    rope_relocate_q (once per distinct segment shift) -> mla_absorb_q
    -> mla_decode_splitkv (all segments) -> mla_combine_lse -> mla_out_uv

(the first two as one mla_prepare_q launch for up to 8 distinct shifts),
and lays out the partial-state slots: segments with disjoint head ranges that
follow each other share a slot range (e.g. a document read by the Local heads
at a relocated position and its recomputed copy read by the Global heads),
later ranges stack after it, so each head's slots tile [0, n_part).

With QK-Norm (``qk_norm=(g_q, g_k, eps)``) the content query is normalised
and weighted first.  For few query rows (n_tok * n_heads <= 512, the MFMA
shape) that happens inside the same launch (mla_prepare_q_qknorm); otherwise
mla_qknorm_query writes the query in fp32 and mla_prepare_q absorbs it
against the bf16 U_K (hi + lo parts of the query on MFMA; other shapes use
an fp32 copy of U_K).  Each segment carries the inverse RMS of its rows'
content keys, computed once here from the cache (mla_qknorm_key_gram and
mla_qknorm_key_rinv: the cache writer's share of the work).  With an int8 or
int4 cache (``quant="int8"`` / ``"int4"``) each segment's bf16 rows are
quantized here by mla_quantize_latent_i8 / _i4 (again the cache writer's
part) and the decode reads the packed rows and their scales.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

from . import ops

# query rows (tokens x heads) up to which the QK-Norm query normalisation runs
# inside the prepare launch
QK_FUSED_ROWS = 512


@dataclass
class StepSegment:
    cache: torch.Tensor                 # device
    seq_lens: torch.Tensor              # device int32 [B]
    seq_lens_host: Sequence[int]
    shift: torch.Tensor                 # device int64 [n_tok]
    shift_host: Sequence[int]
    block_table: Optional[torch.Tensor] = None
    head_begin: int = 0
    head_count: int = 0
    causal: bool = False


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


class DecodeStep:
    def __init__(self, q_nope, q_pe, q_pos, w_uk, w_uv, segments: List[StepSegment], batch: int, s_q: int,
                 scale: float, rope_base: float = 10000.0, n_wg: int = 0,
                 n_split: Optional[Sequence[int]] = None, fuse_post: Optional[bool] = None,
                 qk_norm: Optional[tuple] = None, quant: Optional[str] = None,
                 split_query: Optional[bool] = None):
        self.q_nope, self.q_pe, self.q_pos = q_nope, q_pe, q_pos
        self.w_uk, self.w_uv = w_uk, w_uv
        self.batch, self.s_q, self.scale, self.rope_base, self.n_wg = batch, s_q, scale, rope_base, n_wg
        dev, dt = q_nope.device, q_nope.dtype
        n_tok, H, _ = q_nope.shape
        d_c = w_uk.shape[2]
        d_v = w_uv.shape[1]
        self.bf16 = dt == torch.bfloat16

        # The query enters the decode in fp32 (q_lat and the rotated q_rot):
        # the kernel splits it into bf16 hi + lo parts, so the scores are not
        # limited by a bf16-rounded query.
        q_dt = torch.float32
        # one rotated query per distinct shift
        self.q_rots = []
        keys = {}
        self.seg_rot = []
        for s in segments:
            key = tuple(int(v) for v in s.shift_host)
            if key not in keys:
                keys[key] = len(self.q_rots)
                self.q_rots.append((s.shift, torch.empty_like(q_pe, dtype=q_dt)))
            self.seg_rot.append(keys[key])

        # split counts
        if n_split is None:
            n_split = [self._auto_split(s) for s in segments]
        # slot layout: runs of head-disjoint segments share one slot range
        layers, cur, used = [], [], set()
        for i, s in enumerate(segments):
            hs = set(range(s.head_begin, s.head_begin + s.head_count))
            if cur and (hs & used):
                layers.append(cur)
                cur, used = [], set()
            cur.append(i)
            used |= hs
        layers.append(cur)
        self.n_split = list(n_split)
        part_begin = [0] * len(segments)
        pb = 0
        for layer in layers:
            m = max(self.n_split[i] for i in layer)
            for i in layer:
                self.n_split[i] = m
                part_begin[i] = pb
            pb += m
        self.n_part = pb
        # QK-Norm: static weights and key statistics
        self.qk_norm = qk_norm is not None
        rinvs = [None] * len(segments)
        if self.qk_norm:
            g_q, g_k, eps = qk_norm
            self.g_q = g_q.to(device=dev, dtype=torch.float32).contiguous()
            self.g_k = g_k.to(device=dev, dtype=torch.float32).contiguous()
            self.qk_eps = float(eps)
            # the MFMA prepare takes the fp32 query with the bf16 weights;
            # elsewhere the absorption needs weights of the query's dtype
            mfma_shape = w_uk.dtype == torch.bfloat16 and w_uk.shape[1] == 128 and d_c == 512
            self.w_uk_q = w_uk if mfma_shape else w_uk.to(torch.float32).contiguous()
            self.q_norm = torch.empty(q_nope.shape, dtype=torch.float32, device=dev)
            self.gram = ops.qknorm_key_gram(w_uk)
            d_nope = w_uk.shape[1]
            rinvs = [ops.qknorm_key_rinv(s.cache, self.gram, H, d_nope, self.qk_eps) for s in segments]
        # int8 cache: the cache writer's quantization of each segment's rows
        caches = [s.cache for s in segments]
        scales = [None] * len(segments)
        if quant is not None:
            if quant not in ("int8", "int4"):
                raise ValueError(f"unknown cache quantization {quant!r}")
            quantize = ops.quantize_latent_i8 if quant == "int8" else ops.quantize_latent_i4
            qs = [quantize(s.cache, d_c) for s in segments]
            caches = [c for c, _ in qs]
            scales = [sc for _, sc in qs]
        self.segments = [
            ops.Segment(cache=caches[i], seq_lens=s.seq_lens, q_rot=self.q_rots[self.seg_rot[i]][1],
                        block_table=s.block_table, head_begin=s.head_begin, head_count=s.head_count,
                        causal=s.causal, part_begin=part_begin[i], n_split=self.n_split[i], row_rinv=rinvs[i],
                        row_scale=scales[i])
            for i, s in enumerate(segments)
        ]
        # The row-owning kernel reads the latent query as bf16 hi and lo
        # planes written by the fused query kernel (half the bytes per read
        # of an fp32 query): on that kernel's calls (several segments, more
        # than 32 query rows, a low-bit cache), where the fused kernel has its
        # MFMA shape (with QK-Norm too: the query is normalised first).
        rows = max(s_q * s.head_count for s in segments)
        rows_kernel = quant is not None or len(segments) > 1 or rows > 32
        mfma_shape = w_uk.dtype == torch.bfloat16 and w_uk.shape[1] == 128 and d_c == 512
        can_split = (self.bf16 and rows_kernel and mfma_shape and len(self.q_rots) <= 8
                     and q_nope.data_ptr() % 16 == 0 and w_uk.data_ptr() % 16 == 0)
        if split_query and not can_split:
            raise ValueError("a split query needs the row-owning kernel's calls and the fused query kernel")
        self.q_split = can_split if split_query is None else bool(split_query)
        self.q_lat = (ops.split_query(n_tok, H, d_c, dev) if self.q_split
                      else torch.empty((n_tok, H, d_c), dtype=q_dt, device=dev))
        # partial outputs in bf16 beside a bf16 cache (half the bytes written
        # and merged), fp32 on the fp32 path
        part_dt = torch.float32 if segments[0].cache.dtype == torch.float32 else torch.bfloat16
        self.o_part = torch.empty((n_tok, H, self.n_part, d_c), dtype=part_dt, device=dev)
        self.lse_part = torch.empty((n_tok, H, self.n_part), dtype=torch.float32, device=dev)
        self.o_lat = torch.empty((n_tok, H, d_c), dtype=dt, device=dev)
        self.lse = torch.empty((n_tok, H), dtype=torch.float32, device=dev)
        self.out = torch.empty((n_tok, H, d_v), dtype=dt, device=dev)
        # merge and U_V in one launch (mla_combine_out_uv) for few query
        # tokens: each of its workgroups reads one head's U_V
        if fuse_post is None:
            fuse_post = n_tok <= 8
        self.fuse_post = bool(fuse_post) and d_c <= 512 and d_v <= 128

    def _auto_split(self, s: StepSegment) -> int:
        lens = [int(x) for x in s.seq_lens_host]
        tmax = max(lens) if lens else 0
        tsum = sum(lens)
        if not self.bf16:
            return 2 if tmax >= 2 else 1
        if tsum == 0:
            return 1
        shares = ops.decode_shares(self.s_q, s.head_count, self.n_wg)
        share = 32 * _ceil_div(_ceil_div(tsum, shares), 32)
        return _ceil_div(tmax, share) + 1

    def rope(self):
        for shift, q_rot in self.q_rots:
            ops.rope_relocate_q(self.q_pe, self.q_pos, shift, self.rope_base, out=q_rot)

    def absorb(self):
        if self.qk_norm:
            ops.qknorm_query(self.q_nope, self.g_q, self.g_k, self.qk_eps, out=self.q_norm)
            if self.w_uk_q.dtype == torch.float32:
                ops.absorb_q(self.q_norm, self.w_uk_q, out=self.q_lat)
            else:  # fp32 query against bf16 weights: only the fused prepare path offers it
                from . import _lib
                _lib.call("mla_prepare_q", *ops.prepare_args(self.q_norm, self.q_pe, self.w_uk_q, self.q_lat, [],
                                                              [], self.q_pos, self.rope_base, ops._stream()))
        else:
            ops.absorb_q(self.q_nope, self.w_uk, out=self.q_lat)

    def decode(self):
        ops.decode_splitkv(self.segments, self.q_lat, self.batch, self.s_q, self.scale, self.o_part,
                           self.lse_part, self.n_wg)

    def combine(self):
        ops.combine_lse(self.o_part, self.lse_part, self.o_lat.dtype, o_lat=self.o_lat, lse=self.lse)

    def expand(self):
        ops.out_uv(self.o_lat, self.w_uv, out=self.out)

    def _fused_prepare(self) -> bool:
        """rope (all shifts) and absorb in one mla_prepare_q launch?"""
        return len(self.q_rots) <= 8 and (not self.qk_norm or self.w_uk_q.dtype == torch.bfloat16)

    def _qk_fused(self) -> bool:
        """QK-Norm of the query inside that launch too (mla_prepare_q_qknorm:
        few query rows, the MFMA shape)?"""
        n_tok, H, _ = self.q_nope.shape
        return (self.qk_norm and self._fused_prepare() and n_tok * H <= QK_FUSED_ROWS
                and self.q_nope.data_ptr() % 16 == 0 and self.w_uk_q.data_ptr() % 16 == 0)

    def _prepare_args(self, stream: int):
        rots, shifts = [r for _, r in self.q_rots], [s for s, _ in self.q_rots]
        if self._qk_fused():
            return ops.prepare_qknorm_args(self.q_nope, self.g_q, self.g_k, self.qk_eps, self.q_pe, self.w_uk_q,
                                           self.q_lat, rots, shifts, self.q_pos, self.rope_base, stream)
        q, w = (self.q_norm, self.w_uk_q) if self.qk_norm else (self.q_nope, self.w_uk)
        return ops.prepare_args(q, self.q_pe, w, self.q_lat, rots, shifts, self.q_pos, self.rope_base, stream)

    def prepare(self):
        """rope (all shifts) and absorb, in one launch (mla_prepare_q) where it
        can; with QK-Norm the query normalisation runs first."""
        if not self._fused_prepare():
            self.rope()
            self.absorb()
            return
        from . import _lib
        if self._qk_fused():
            _lib.call("mla_prepare_q_qknorm", *self._prepare_args(ops._stream()))
            return
        if self.qk_norm:
            ops.qknorm_query(self.q_nope, self.g_q, self.g_k, self.qk_eps, out=self.q_norm)
        _lib.call("mla_prepare_q", *self._prepare_args(ops._stream()))

    def combine_expand(self):
        ops.combine_out_uv(self.o_part, self.lse_part, self.w_uv, self.out.dtype, out=self.out, o_lat=self.o_lat,
                           lse=self.lse)

    def run(self):
        self.prepare()
        self.decode()
        if self.fuse_post:
            self.combine_expand()
        else:
            self.combine()
            self.expand()
        return self.out, self.o_lat, self.lse

    # -- low-overhead replay: ctypes arguments built once for a fixed stream --
    def bind(self, stream: Optional[torch.cuda.Stream] = None):
        """Precompute the C calls of one step on ``stream`` (default: current).
        Returns (pre, decode, post): lists of (function, args) to run in order."""
        from . import _lib
        lib = _lib.load()
        st = (stream or torch.cuda.current_stream()).cuda_stream
        dt = ops._dt
        n_tok, H, d_nope = self.q_nope.shape
        d_c = self.w_uk.shape[2]
        d_r = self.q_pe.shape[2]
        if self._qk_fused():  # QK-Norm, rope (all shifts) and absorb in one launch
            self._prep_args = self._prepare_args(st)
            pre = [(lib.mla_prepare_q_qknorm, self._prep_args)]
        elif self._fused_prepare():  # one launch for rope (all shifts) and absorb
            pre = []
            if self.qk_norm:
                pre.append((lib.mla_qknorm_query, (self.q_nope.data_ptr(), dt(self.q_nope), self.g_q.data_ptr(),
                                                   self.g_k.data_ptr(), n_tok, H, d_nope, self.qk_eps,
                                                   self.q_norm.data_ptr(), st)))
            self._prep_args = self._prepare_args(st)
            pre.append((lib.mla_prepare_q, self._prep_args))
        else:
            pre = [(lib.rope_relocate_q, (self.q_pe.data_ptr(), dt(self.q_pe), q_rot.data_ptr(), dt(q_rot),
                                          self.q_pos.data_ptr(), shift.data_ptr(), n_tok, H, d_r,
                                          float(self.rope_base), st))
                   for shift, q_rot in self.q_rots]
            if self.qk_norm:
                pre.append((lib.mla_qknorm_query, (self.q_nope.data_ptr(), dt(self.q_nope), self.g_q.data_ptr(),
                                                   self.g_k.data_ptr(), n_tok, H, d_nope, self.qk_eps,
                                                   self.q_norm.data_ptr(), st)))
                if self.w_uk_q.dtype == torch.float32:
                    pre.append((lib.mla_absorb_q, (self.q_norm.data_ptr(), self.w_uk_q.data_ptr(), dt(self.q_norm),
                                                   self.q_lat.data_ptr(), dt(self.q_lat), n_tok, H, d_nope, d_c, st)))
                else:
                    self._absorb_args = ops.prepare_args(self.q_norm, self.q_pe, self.w_uk_q, self.q_lat, [], [],
                                                         self.q_pos, self.rope_base, st)
                    pre.append((lib.mla_prepare_q, self._absorb_args))
            else:
                pre.append((lib.mla_absorb_q, (self.q_nope.data_ptr(), self.w_uk.data_ptr(), dt(self.q_nope),
                                               self.q_lat.data_ptr(), dt(self.q_lat), n_tok, H, d_nope, d_c, st)))
        self._seg_arr = (_lib.MlaSegment * len(self.segments))(*[sg.to_c() for sg in self.segments])
        dec = [(lib.mla_decode_splitkv, (self._seg_arr, len(self.segments), self.q_lat.data_ptr(),
                                         ops._lat_dt(self.q_lat),
                                         ops._cache_dt(self.segments[0].cache, self.segments[0].row_scale),
                                         self.batch, self.s_q, H, d_c, d_r,
                                         float(self.scale), self.o_part.data_ptr(), dt(self.o_part),
                                         self.lse_part.data_ptr(),
                                         self.n_part, self.n_wg, st))]
        if self.fuse_post:
            post = [(lib.mla_combine_out_uv, (self.o_part.data_ptr(), dt(self.o_part), self.lse_part.data_ptr(), n_tok,
                                              H, self.n_part,
                                              d_c, self.w_uv.data_ptr(), dt(self.w_uv), self.w_uv.shape[1],
                                              self.o_lat.data_ptr(), self.lse.data_ptr(), self.out.data_ptr(),
                                              dt(self.out), st))]
        else:
            post = [(lib.mla_combine_lse, (self.o_part.data_ptr(), dt(self.o_part), self.lse_part.data_ptr(), n_tok * H,
                                           self.n_part,
                                           d_c, self.o_lat.data_ptr(), dt(self.o_lat), self.lse.data_ptr(), st)),
                    (lib.mla_out_uv, (self.o_lat.data_ptr(), dt(self.o_lat), self.w_uv.data_ptr(), dt(self.w_uv),
                                      self.out.data_ptr(), dt(self.out), n_tok, H, d_c, self.w_uv.shape[1], st))]
        return pre, dec, post


def run_calls(calls) -> None:
    """Run bound calls; raise on the first failing status."""
    from . import _lib
    for fn, args in calls:
        st = fn(*args)
        if st != 0:
            raise _lib.MlaError(fn.__name__, st, _lib.load().mla_last_error().decode())


def step_from_inputs(x, device="cuda", n_wg: int = 0, n_split=None, fuse_post=None,
                     split_query=None) -> DecodeStep:
    """Upload a seeded input set (``mla_inputs.MlaInputs``) and build its step."""
    d = torch.device(device)
    segs = []
    for s in x.segments:
        shift_tok = x.token_shift(s)
        segs.append(StepSegment(
            cache=s.cache.to(d), seq_lens=s.seq_lens.to(d), seq_lens_host=s.seq_lens.tolist(),
            shift=shift_tok.to(d), shift_host=shift_tok.tolist(),
            block_table=None if s.block_table is None else s.block_table.to(d),
            head_begin=s.head_begin, head_count=s.head_count, causal=s.causal))
    qk = None
    if getattr(x, "g_q", None) is not None:
        qk = (x.g_q.to(d), x.g_k.to(d), x.spec.qk_eps)
    return DecodeStep(x.q_nope.to(d), x.q_pe.to(d), x.q_pos.to(d), x.w_uk.to(d), x.w_uv.to(d), segs,
                      x.spec.batch, x.spec.s_q, x.scale, x.rope_base, n_wg=n_wg, n_split=n_split,
                      fuse_post=fuse_post, qk_norm=qk, quant=getattr(x.spec, "quant", None),
                      split_query=split_query)
