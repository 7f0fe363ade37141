"""Torch-tensor wrappers of the five decode calls (argument marshalling only).

Tensors must be contiguous and on the current HIP device; work is enqueued on
torch's current stream.  Shapes and meaning: ``include/mla_latent.h``.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

from . import _lib
from ._lib import MLA_BF16, MLA_BF16X2, MLA_F32, MLA_I4, MLA_I8, MlaSegment

_DT = {torch.float32: MLA_F32, torch.bfloat16: MLA_BF16}


def _cache_dt(cache: torch.Tensor, row_scale: Optional[torch.Tensor] = None) -> int:
    """Cache format: fp32 / bf16 rows, or packed rows held as uint8 bytes: int8
    (one scale per row) or int4 (a (latent, rotary) scale pair per row)."""
    if cache.dtype != torch.uint8:
        return _dt(cache)
    return MLA_I4 if row_scale is not None and row_scale.dim() == cache.dim() else MLA_I8


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def is_split_query(q_lat: torch.Tensor) -> bool:
    """A query held as bf16 hi and lo planes: bf16 [n_tok, n_heads, 2, d_c]."""
    return q_lat.dtype == torch.bfloat16 and q_lat.dim() == 4 and q_lat.shape[2] == 2


def _lat_dt(q_lat: torch.Tensor) -> int:
    """dtype code of a q_lat tensor (MLA_BF16X2 for the split form)."""
    return MLA_BF16X2 if is_split_query(q_lat) else _dt(q_lat)


def split_query(n_tok: int, n_heads: int, d_c: int, device) -> torch.Tensor:
    """An empty split query (mla_prepare_q writes it with lat_dtype MLA_BF16X2)."""
    return torch.empty((n_tok, n_heads, 2, d_c), dtype=torch.bfloat16, device=device)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def rope_relocate_q(q_pe: torch.Tensor, pos: torch.Tensor, shift: Optional[torch.Tensor] = None,
                    base: float = 10000.0, out: Optional[torch.Tensor] = None,
                    out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    n_tok, n_heads, d_rope = q_pe.shape
    if out is None:
        out = torch.empty_like(q_pe, dtype=out_dtype or q_pe.dtype)
    _lib.call("rope_relocate_q", _ptr(q_pe), _dt(q_pe), _ptr(out), _dt(out), _ptr(pos), _ptr(shift), n_tok,
              n_heads, d_rope, float(base), _stream())
    return out


def absorb_q(q_nope: torch.Tensor, w_uk: torch.Tensor, out: Optional[torch.Tensor] = None,
             out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    n_tok, n_heads, d_nope = q_nope.shape
    d_c = w_uk.shape[2]
    if w_uk.shape != (n_heads, d_nope, d_c) or w_uk.dtype != q_nope.dtype:
        raise ValueError("w_uk must be [n_heads, d_nope, d_c] of q_nope's dtype")
    if out is None:
        out = torch.empty((n_tok, n_heads, d_c), dtype=out_dtype or q_nope.dtype, device=q_nope.device)
    _lib.call("mla_absorb_q", _ptr(q_nope), _ptr(w_uk), _dt(q_nope), _ptr(out), _dt(out), n_tok, n_heads,
              d_nope, d_c, _stream())
    return out


def prepare_args(q_nope: torch.Tensor, q_pe: torch.Tensor, w_uk: torch.Tensor, q_lat: torch.Tensor,
                 q_rots: Sequence[torch.Tensor], shifts: Sequence[Optional[torch.Tensor]], pos: torch.Tensor,
                 base: float, stream: int):
    """Argument tuple of mla_prepare_q (the two pointer arrays are part of it
    and must stay alive while the tuple is used)."""
    import ctypes
    n_tok, n_heads, d_nope = q_nope.shape
    d_rope = q_pe.shape[2]
    d_c = w_uk.shape[2]
    n = len(q_rots)
    rot_arr = (ctypes.c_void_p * max(1, n))(*[r.data_ptr() for r in q_rots])
    sh_arr = (ctypes.c_void_p * max(1, n))(*[_ptr(s) for s in shifts])
    rot_dt = _dt(q_rots[0]) if n else 0
    return (_ptr(q_nope), _dt(q_nope), _ptr(q_pe), _ptr(w_uk), _dt(w_uk), _ptr(q_lat), _lat_dt(q_lat), rot_arr, sh_arr, n,
            rot_dt, _ptr(pos), n_tok, n_heads, d_nope, d_rope, d_c, float(base), stream)


def prepare_qknorm_args(q_nope: torch.Tensor, g_q: torch.Tensor, g_k: torch.Tensor, eps: float,
                        q_pe: torch.Tensor, w_uk: torch.Tensor, q_lat: torch.Tensor,
                        q_rots: Sequence[torch.Tensor], shifts: Sequence[Optional[torch.Tensor]], pos: torch.Tensor,
                        base: float, stream: int):
    """Argument tuple of mla_prepare_q_qknorm (its pointer arrays must stay
    alive while the tuple is used)."""
    a = prepare_args(q_nope, q_pe, w_uk, q_lat, q_rots, shifts, pos, base, stream)
    for g in (g_q, g_k):
        if g.dtype != torch.float32 or not g.is_contiguous() or g.shape != q_nope.shape[1:]:
            raise ValueError("g_q, g_k must be contiguous fp32 [n_heads, d_nope]")
    return a[:2] + (g_q.data_ptr(), g_k.data_ptr(), float(eps)) + a[2:]


def prepare_q_qknorm(q_nope: torch.Tensor, g_q: torch.Tensor, g_k: torch.Tensor, eps: float, q_pe: torch.Tensor,
                     w_uk: torch.Tensor, pos: torch.Tensor, shifts: Sequence[Optional[torch.Tensor]],
                     base: float = 10000.0, lat_dtype: Optional[torch.dtype] = None,
                     rot_dtype: Optional[torch.dtype] = None):
    """mla_prepare_q_qknorm: the QK-Norm query absorbed, and the rotary query
    per shift, in one launch."""
    n_tok, n_heads, _ = q_nope.shape
    q_lat = torch.empty((n_tok, n_heads, w_uk.shape[2]), dtype=lat_dtype or torch.float32, device=q_nope.device)
    q_rots = [torch.empty_like(q_pe, dtype=rot_dtype or q_pe.dtype) for _ in shifts]
    _lib.call("mla_prepare_q_qknorm", *prepare_qknorm_args(q_nope, g_q, g_k, eps, q_pe, w_uk, q_lat, q_rots, shifts,
                                                           pos, base, _stream()))
    return q_lat, q_rots


def prepare_q(q_nope: torch.Tensor, q_pe: torch.Tensor, w_uk: torch.Tensor, pos: torch.Tensor,
              shifts: Sequence[Optional[torch.Tensor]], base: float = 10000.0,
              lat_dtype: Optional[torch.dtype] = None, rot_dtype: Optional[torch.dtype] = None,
              split: bool = False):
    """mla_prepare_q: (q_lat, [q_rot per shift]) in one launch.  split: q_lat
    as bf16 hi and lo planes [n_tok, n_heads, 2, d_c] (MLA_BF16X2)."""
    n_tok, n_heads, _ = q_nope.shape
    if split:
        q_lat = split_query(n_tok, n_heads, w_uk.shape[2], q_nope.device)
    else:
        q_lat = torch.empty((n_tok, n_heads, w_uk.shape[2]), dtype=lat_dtype or q_nope.dtype, device=q_nope.device)
    q_rots = [torch.empty_like(q_pe, dtype=rot_dtype or q_pe.dtype) for _ in shifts]
    _lib.call("mla_prepare_q", *prepare_args(q_nope, q_pe, w_uk, q_lat, q_rots, shifts, pos, base, _stream()))
    return q_lat, q_rots


def out_uv(o_lat: torch.Tensor, w_uv: torch.Tensor, out: Optional[torch.Tensor] = None,
           out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    n_tok, n_heads, d_c = o_lat.shape
    d_v = w_uv.shape[1]
    if w_uv.shape != (n_heads, d_v, d_c):
        raise ValueError("w_uv must be [n_heads, d_v, d_c]")
    if out is None:
        out = torch.empty((n_tok, n_heads, d_v), dtype=out_dtype or w_uv.dtype, device=o_lat.device)
    _lib.call("mla_out_uv", _ptr(o_lat), _dt(o_lat), _ptr(w_uv), _dt(w_uv), _ptr(out), _dt(out), n_tok,
              n_heads, d_c, d_v, _stream())
    return out


def out_proj(x: torch.Tensor, w_o: torch.Tensor, out: Optional[torch.Tensor] = None,
             out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """x [n_tok, ...] (flattened to [n_tok, k_in]), w_o [d_model, k_in] -> out [n_tok, d_model]."""
    n_tok = x.shape[0]
    k_in = x[0].numel() if n_tok else w_o.shape[1]
    d_model = w_o.shape[0]
    if w_o.dim() != 2 or w_o.shape[1] != k_in:
        raise ValueError("w_o must be [d_model, k_in] with k_in = the product of x's trailing dims")
    if not x.is_contiguous() or not w_o.is_contiguous():
        raise ValueError("x and w_o must be contiguous")
    if out is None:
        out = torch.empty((n_tok, d_model), dtype=out_dtype or w_o.dtype, device=x.device)
    _lib.call("mla_out_proj", _ptr(x), _dt(x), _ptr(w_o), _dt(w_o), _ptr(out), _dt(out), n_tok, k_in, d_model,
              _stream())
    return out


def combine_lse(o_part: torch.Tensor, lse_part: torch.Tensor, out_dtype: torch.dtype,
                o_lat: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """o_part [..., n_part, d_c] fp32 or bf16, lse_part [..., n_part] -> (o_lat [..., d_c], lse [...])."""
    lead = o_part.shape[:-2]
    n_part, d_c = o_part.shape[-2:]
    n_rows = 1
    for x in lead:
        n_rows *= x
    if o_lat is None:
        o_lat = torch.empty(tuple(lead) + (d_c,), dtype=out_dtype, device=o_part.device)
    if lse is None:
        lse = torch.empty(tuple(lead), dtype=torch.float32, device=o_part.device)
    _lib.call("mla_combine_lse", _ptr(o_part), _dt(o_part), _ptr(lse_part), n_rows, n_part, d_c, _ptr(o_lat),
              _DT[out_dtype], _ptr(lse), _stream())
    return o_lat, lse


def combine_out_uv(o_part: torch.Tensor, lse_part: torch.Tensor, w_uv: torch.Tensor, out_dtype: torch.dtype,
                   out: Optional[torch.Tensor] = None, o_lat: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, want_o_lat: bool = True, want_lse: bool = True):
    """o_part [n_tok, H, n_part, d_c] fp32 or bf16, lse_part [n_tok, H, n_part], w_uv [H, d_v, d_c]
    -> (out [n_tok, H, d_v], o_lat [n_tok, H, d_c] or None, lse [n_tok, H] or None)."""
    n_tok, H, n_part, d_c = o_part.shape
    d_v = w_uv.shape[1]
    dev = o_part.device
    if out is None:
        out = torch.empty((n_tok, H, d_v), dtype=out_dtype, device=dev)
    if o_lat is None and want_o_lat:
        o_lat = torch.empty((n_tok, H, d_c), dtype=out_dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((n_tok, H), dtype=torch.float32, device=dev)
    _lib.call("mla_combine_out_uv", _ptr(o_part), _dt(o_part), _ptr(lse_part), n_tok, H, n_part, d_c, _ptr(w_uv),
              _DT[w_uv.dtype], d_v, _ptr(o_lat), _ptr(lse), _ptr(out), _DT[out_dtype], _stream())
    return out, o_lat, lse


def quantize_latent_i8(rows: torch.Tensor, d_c: int, out: Optional[torch.Tensor] = None,
                       scales: Optional[torch.Tensor] = None):
    """Int8 latent cache from bf16 rows [..., d_c + d_rope]: (packed rows uint8
    [..., d_c + 2 d_rope], scales fp32 [...])."""
    width = rows.shape[-1]
    d_rope = width - d_c
    n_rows = rows.numel() // width
    if out is None:
        out = torch.empty(rows.shape[:-1] + (d_c + 2 * d_rope,), dtype=torch.uint8, device=rows.device)
    if scales is None:
        scales = torch.empty(rows.shape[:-1], dtype=torch.float32, device=rows.device)
    _lib.call("mla_quantize_latent_i8", _ptr(rows), _dt(rows), n_rows, d_c, d_rope, _ptr(out), _ptr(scales),
              _stream())
    return out, scales


def quantize_latent_i4(rows: torch.Tensor, d_c: int, out: Optional[torch.Tensor] = None,
                       scales: Optional[torch.Tensor] = None):
    """Int4 cache from bf16 rows [..., d_c + d_rope]: (packed rows uint8
    [..., (d_c + d_rope) / 2], scales fp32 [..., 2] = (latent, rotary))."""
    width = rows.shape[-1]
    d_rope = width - d_c
    n_rows = rows.numel() // width
    if out is None:
        out = torch.empty(rows.shape[:-1] + (width // 2,), dtype=torch.uint8, device=rows.device)
    if scales is None:
        scales = torch.empty(rows.shape[:-1] + (2,), dtype=torch.float32, device=rows.device)
    _lib.call("mla_quantize_latent_i4", _ptr(rows), _dt(rows), n_rows, d_c, d_rope, _ptr(out), _ptr(scales),
              _stream())
    return out, scales


def qknorm_query(q_nope: torch.Tensor, g_q: torch.Tensor, g_k: torch.Tensor, eps: float,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """QK-Norm of the content query with both static weights folded in:
    [n_tok, H, d_nope] -> fp32 [n_tok, H, d_nope]."""
    n_tok, n_heads, d_nope = q_nope.shape
    if g_q.shape != (n_heads, d_nope) or g_k.shape != (n_heads, d_nope):
        raise ValueError("g_q and g_k must be [n_heads, d_nope]")
    if out is None:
        out = torch.empty((n_tok, n_heads, d_nope), dtype=torch.float32, device=q_nope.device)
    _lib.call("mla_qknorm_query", _ptr(q_nope), _dt(q_nope), _ptr(g_q), _ptr(g_k), n_tok, n_heads, d_nope,
              float(eps), _ptr(out), _stream())
    return out


def qknorm_key_gram(w_uk: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """G = sum_h U_K[h]^T U_K[h]: [H, d_nope, d_c] -> fp32 [d_c, d_c]."""
    n_heads, d_nope, d_c = w_uk.shape
    if out is None:
        out = torch.empty((d_c, d_c), dtype=torch.float32, device=w_uk.device)
    _lib.call("mla_qknorm_key_gram", _ptr(w_uk), _dt(w_uk), n_heads, d_nope, d_c, _ptr(out), _stream())
    return out


def qknorm_key_rinv(rows: torch.Tensor, gram: torch.Tensor, n_heads: int, d_nope: int, eps: float,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Inverse RMS of each stored row's content key.  ``rows``: a cache or page
    pool [..., row_width] (latent first); result fp32 of shape rows.shape[:-1]."""
    d_c = gram.shape[0]
    row_width = rows.shape[-1]
    n_rows = rows.numel() // row_width
    if out is None:
        out = torch.empty(rows.shape[:-1], dtype=torch.float32, device=rows.device)
    _lib.call("mla_qknorm_key_rinv", _ptr(rows), _dt(rows), n_rows, row_width, _ptr(gram), d_c, n_heads,
              d_nope, float(eps), _ptr(out), _stream())
    return out


@dataclass
class Segment:
    """Device tensors of one KV segment (see ``mla_segment``)."""
    cache: torch.Tensor                   # [B, max_rows, R] or pool [P, page, R]
    seq_lens: torch.Tensor                # int32 [B]
    q_rot: torch.Tensor                   # [n_tok, H, d_rope]
    block_table: Optional[torch.Tensor] = None   # int32 [B, max_pages]
    head_begin: int = 0
    head_count: int = 0
    causal: bool = False
    part_begin: int = 0
    n_split: int = 1
    row_rinv: Optional[torch.Tensor] = None      # fp32, cache.shape[:2] (QK-Norm)
    row_scale: Optional[torch.Tensor] = None     # fp32, cache.shape[:2] (int8) or + (2,) (int4); uint8 rows

    def to_c(self) -> MlaSegment:
        s = MlaSegment()
        s.cache = _ptr(self.cache)
        s.block_table = _ptr(self.block_table)
        s.seq_lens = _ptr(self.seq_lens)
        s.q_rot = _ptr(self.q_rot)
        if self.block_table is None:
            s.max_rows = self.cache.shape[1]
            s.page_size = s.max_pages = s.n_pages = 0
        else:
            s.max_rows = 0
            s.page_size = self.cache.shape[1]
            s.max_pages = self.block_table.shape[1]
            s.n_pages = self.cache.shape[0]
        s.head_begin = self.head_begin
        s.head_count = self.head_count
        s.causal = int(self.causal)
        s.part_begin = self.part_begin
        s.n_split = self.n_split
        s.row_rinv = _ptr(self.row_rinv)
        s.row_scale = _ptr(self.row_scale)
        return s


def decode_splitkv(segments: Sequence[Segment], q_lat: torch.Tensor, batch: int, s_q: int, scale: float,
                   o_part: torch.Tensor, lse_part: torch.Tensor, n_wg: int = 0) -> None:
    """o_part [n_tok, H, n_part, d_c] (fp32 or bf16) and lse_part [n_tok, H, n_part] are written.
    q_lat: [n_tok, H, d_c], or a split query [n_tok, H, 2, d_c] (then q_rot is fp32)."""
    split = is_split_query(q_lat)
    n_tok, n_heads = q_lat.shape[:2]
    d_c = q_lat.shape[-1]
    d_rope = segments[0].q_rot.shape[2]
    n_part = o_part.shape[2]
    cache_dt = _cache_dt(segments[0].cache, segments[0].row_scale)
    rot_dt = torch.float32 if split else q_lat.dtype
    for s in segments:
        if _cache_dt(s.cache, s.row_scale) != cache_dt or s.q_rot.dtype != rot_dt:
            raise ValueError("segments must share the cache dtype; q_rot must have q_lat's dtype (fp32 beside a "
                             "split query)")
    arr = (MlaSegment * len(segments))(*[s.to_c() for s in segments])
    _lib.call("mla_decode_splitkv", arr, len(segments), _ptr(q_lat), _lat_dt(q_lat), cache_dt, batch, s_q, n_heads,
              d_c, d_rope, float(scale), _ptr(o_part), _dt(o_part), _ptr(lse_part), n_part, n_wg, _stream())


def cu_count() -> int:
    return _lib.load().mla_device_cu_count()


def decode_shares(s_q: int, head_count: int, n_wg: int = 0) -> int:
    return _lib.load().mla_decode_shares(s_q, head_count, n_wg)
