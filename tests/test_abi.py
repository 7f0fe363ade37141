"""The C ABI on the CPU: the library loads, exports every function the header
declares with the argument count the binding uses, and rejects bad arguments
before touching the GPU."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_latent.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    decls = {}
    for m in re.finditer(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(([^)]*)\)\s*;", src, flags=re.M):
        name, args = m.group(1), m.group(2).strip()
        n = 0 if args in ("", "void") else args.count(",") + 1
        decls[name] = n
    return decls


@pytest.fixture(scope="module")
def lib():
    from mla_latent_cache_amd import _lib
    return _lib.load()


def test_header_declares_the_five_calls():
    d = _declared()
    for name in ("rope_relocate_q", "mla_absorb_q", "mla_decode_splitkv", "mla_combine_lse", "mla_out_uv"):
        assert name in d


def test_every_declared_symbol_is_exported_and_bound(lib):
    from mla_latent_cache_amd._lib import SIGNATURES
    decls = _declared()
    assert set(decls) == set(SIGNATURES), (set(decls) ^ set(SIGNATURES))
    for name, nargs in decls.items():
        assert hasattr(lib, name), name
        assert len(SIGNATURES[name][1]) == nargs, (name, nargs)


def test_segment_struct_layout(tmp_path):
    """ctypes' mirror of mla_segment has the C compiler's size and offsets."""
    import subprocess
    from mla_latent_cache_amd._lib import MlaSegment
    fields = [f for f, _ in MlaSegment._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "mla_latent.h"\nint main(void){\n'
                   'printf("%zu\\n", sizeof(mla_segment));\n'
                   + "".join(f'printf("%zu\\n", offsetof(mla_segment, {f}));\n' for f in fields)
                   + "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(MlaSegment)
    assert vals[1:] == [getattr(MlaSegment, f).offset for f in fields]


def test_status_strings(lib):
    assert lib.mla_status_string(0) == b"ok"
    assert lib.mla_status_string(7) == b"HIP runtime error"
    assert lib.mla_version() == 100


def _st(lib, name, *args):
    return getattr(lib, name)(*args)


def test_null_and_shape_errors_before_any_gpu_call(lib):
    from mla_latent_cache_amd._lib import MlaSegment
    P = 16  # fake, aligned, non-null address: validation fails before it is used
    assert _st(lib, "rope_relocate_q", None, 1, P, 0, P, None, 1, 1, 64, 1e4, None) == 1
    assert _st(lib, "rope_relocate_q", P, 1, P, 0, P, None, 1, 1, 63, 1e4, None) == 2
    assert _st(lib, "rope_relocate_q", P, 5, P, 0, P, None, 1, 1, 64, 1e4, None) == 3
    assert _st(lib, "rope_relocate_q", P, 1, P, 0, P, None, 1, 1, 64, 0.5, None) == 2
    assert b"base" in lib.mla_last_error()
    assert _st(lib, "mla_absorb_q", P, None, 1, P, 0, 1, 1, 128, 512, None) == 1
    assert _st(lib, "mla_absorb_q", P, P, 1, P, 9, 1, 1, 128, 512, None) == 3
    assert _st(lib, "mla_absorb_q", P, P, 1, P, 0, 1, 0, 128, 512, None) == 2
    assert _st(lib, "mla_out_uv", P, 1, P, 1, P, 1, -1, 1, 512, 128, None) == 2
    assert _st(lib, "mla_combine_lse", P, 0, P, 1, 0, 512, P, 1, None, None) == 2
    assert _st(lib, "mla_combine_lse", P, 7, P, 1, 4, 512, P, 1, None, None) == 3
    # mla_out_proj(x, x_dtype, w_o, w_dtype, out, out_dtype, n_tok, k_in, d_model)
    assert _st(lib, "mla_out_proj", None, 1, P, 1, P, 1, 1, 256, 64, None) == 1
    assert _st(lib, "mla_out_proj", P, 1, P, 7, P, 1, 1, 256, 64, None) == 3
    assert _st(lib, "mla_out_proj", P, 1, P, 1, P, 1, -1, 256, 64, None) == 2
    assert _st(lib, "mla_out_proj", P, 1, P, 1, P, 1, 1, 0, 64, None) == 2
    assert _st(lib, "mla_out_proj", P, 1, P, 1, P, 1, 1, 256, 0, None) == 2
    assert _st(lib, "mla_out_proj", P, 1, P, 1, P, 1, 1, (1 << 20) + 1, 64, None) == 2
    assert _st(lib, "mla_out_proj", P, 1, P, 1, P, 1, 1, 256, (1 << 20) + 1, None) == 2
    assert _st(lib, "mla_out_proj", P, 1, P, 1, P, 1, 0, 256, 64, None) == 0  # nothing to do: no launch
    assert _st(lib, "mla_combine_lse", P, 1, None, 1, 1, 512, P, 1, None, None) == 1
    # mla_combine_out_uv(o_part, part_dtype, lse_part, n_tok, n_heads, n_part, d_c, w_uv, w_dtype, d_v, o_lat,
    #                    lse, out, dt)
    assert _st(lib, "mla_combine_out_uv", P, 5, P, 1, 1, 4, 512, P, 1, 128, None, None, P, 1, None) == 3
    assert _st(lib, "mla_combine_out_uv", P, 1, P, 1, 1, 4, 512, None, 1, 128, None, None, P, 1, None) == 1
    assert _st(lib, "mla_combine_out_uv", P, 1, P, 1, 1, 4, 512, P, 4, 128, None, None, P, 1, None) == 3
    assert _st(lib, "mla_combine_out_uv", P, 1, P, 1, 1, 4, 1024, P, 1, 128, None, None, P, 1, None) == 2
    assert _st(lib, "mla_combine_out_uv", P, 1, P, 1, 1, 4, 512, P, 1, 129, None, None, P, 1, None) == 2
    assert _st(lib, "mla_combine_out_uv", P, 1, P, 1, 1, 4, 510, P, 1, 128, None, None, P, 1, None) == 2
    assert _st(lib, "mla_combine_out_uv", P + 4, 1, P, 1, 1, 4, 512, P, 1, 128, None, None, P, 1, None) == 2
    assert _st(lib, "mla_combine_out_uv", P, 1, P, 0, 1, 4, 512, P, 1, 128, None, None, P, 1, None) == 0
    assert _st(lib, "mla_combine_out_uv", P, 1, P, 65535, 65535, 4, 512, P, 1, 128, None, None, P, 1, None) == 2
    assert _st(lib, "mla_combine_out_uv", P, 1, P, 2048, 1025, 4, 512, P, 1, 128, None, None, P, 1, None) == 2
    assert _st(lib, "mla_combine_lse", P, 1, P, 1 << 24, 4, 512, P, 1, None, None) == 2
    # mla_qknorm_query(q_nope, in_dtype, g_q, g_k, n_tok, n_heads, d_nope, eps, q_out, stream)
    assert _st(lib, "mla_qknorm_query", P, 1, P, None, 1, 16, 128, 1e-6, P, None) == 1
    assert _st(lib, "mla_qknorm_query", P, 3, P, P, 1, 16, 128, 1e-6, P, None) == 3
    assert _st(lib, "mla_qknorm_query", P, 1, P, P, 1, 16, 128, -1.0, P, None) == 2
    assert _st(lib, "mla_qknorm_query", P, 1, P, P, 1, 16, 128, float("inf"), P, None) == 2
    assert _st(lib, "mla_qknorm_query", P, 1, P, P, 1, 0, 128, 1e-6, P, None) == 2
    assert _st(lib, "mla_qknorm_query", P, 1, P, P, 0, 16, 128, 1e-6, P, None) == 0
    # mla_qknorm_key_gram(w_uk, w_dtype, n_heads, d_nope, d_c, gram, stream)
    assert _st(lib, "mla_qknorm_key_gram", None, 1, 16, 128, 512, P, None) == 1
    assert _st(lib, "mla_qknorm_key_gram", P, 1, 16, 128, 1024, P, None) == 2
    assert _st(lib, "mla_qknorm_key_gram", P, 2, 16, 128, 512, P, None) == 3
    # mla_qknorm_key_rinv(rows, dtype, n_rows, row_width, gram, d_c, n_heads, d_nope, eps, rinv, stream)
    assert _st(lib, "mla_qknorm_key_rinv", P, 1, 10, 500, P, 512, 16, 128, 1e-6, P, None) == 2
    assert _st(lib, "mla_qknorm_key_rinv", P, 1, 10, 576, P, 512, 16, 128, float("nan"), P, None) == 2
    assert _st(lib, "mla_qknorm_key_rinv", P, 1, 10, 576, None, 512, 16, 128, 1e-6, P, None) == 1
    assert _st(lib, "mla_qknorm_key_rinv", P, 1, 0, 576, P, 512, 16, 128, 1e-6, P, None) == 0
    # mla_prepare_q(q_nope, q_dtype, q_pe, w_uk, in_dtype, q_lat, lat_dtype, q_rots, shifts, n_shift, rot_dtype,
    #               pos, n_tok, n_heads, d_nope, d_rope, d_c, base, stream): an fp32 query with bf16 weights
    # needs the MFMA shape; a bf16 query with fp32 weights is not offered
    assert _st(lib, "mla_prepare_q", P, 0, P, P, 1, P, 0, None, None, 0, 0, P, 1, 4, 64, 64, 512, 1e4, None) == 5
    assert _st(lib, "mla_prepare_q", P, 1, P, P, 0, P, 0, None, None, 0, 0, P, 1, 4, 128, 64, 512, 1e4, None) == 5
    assert _st(lib, "mla_prepare_q", P, 0, P, P + 8, 1, P, 0, None, None, 0, 0, P, 1, 4, 128, 64, 512, 1e4,
               None) == 5
    assert _st(lib, "mla_prepare_q", P, 4, P, P, 1, P, 0, None, None, 0, 0, P, 1, 4, 128, 64, 512, 1e4, None) == 3
    # a split q_lat (lat_dtype 4) only on the MFMA path (bf16 weights, 128 x 512, aligned)
    assert _st(lib, "mla_prepare_q", P, 0, P, P, 0, P, 4, None, None, 0, 0, P, 1, 4, 128, 64, 512, 1e4, None) == 5
    assert _st(lib, "mla_prepare_q", P, 1, P, P + 8, 1, P, 4, None, None, 0, 0, P, 1, 4, 128, 64, 512, 1e4,
               None) == 5
    assert _st(lib, "mla_prepare_q", P, 1, P, P, 1, P, 5, None, None, 0, 0, P, 1, 4, 128, 64, 512, 1e4, None) == 3
    # mla_prepare_q_qknorm(q_nope, q_dtype, g_q, g_k, eps, q_pe, w_uk, in_dtype, q_lat, lat_dtype, q_rots,
    #                      shifts, n_shift, rot_dtype, pos, n_tok, n_heads, d_nope, d_rope, d_c, base, stream)
    qk = lambda q_dt, gq, eps, in_dt, n_tok, H, d_nope: _st(  # noqa: E731
        lib, "mla_prepare_q_qknorm", P, q_dt, gq, P, eps, P, P, in_dt, P, 0, None, None, 0, 0, P, n_tok, H, d_nope,
        64, 512, 1e4, None)
    assert qk(0, None, 1e-6, 1, 4, 16, 128) == 1       # g_q NULL
    assert qk(4, P, 1e-6, 1, 4, 16, 128) == 3          # unknown q dtype
    assert qk(0, P, -1.0, 1, 4, 16, 128) == 2          # eps < 0
    assert qk(0, P, float("nan"), 1, 4, 16, 128) == 2
    assert qk(0, P, 1e-6, 0, 4, 16, 128) == 5          # fp32 weights: not the MFMA path
    assert qk(0, P, 1e-6, 1, 4, 16, 64) == 5           # d_nope 64
    assert _st(lib, "mla_prepare_q_qknorm", P + 8, 0, P, P, 1e-6, P, P, 1, P, 0, None, None, 0, 0, P, 4, 16, 128,
               64, 512, 1e4, None) == 5                 # q_nope not 16-byte aligned
    assert qk(0, P, 1e-6, 1, 33, 16, 128) == 5         # 528 query rows > 512
    assert qk(0, P, 1e-6, 1, 0, 16, 128) == 0          # no tokens: nothing enqueued
    # mla_quantize_latent_i8(rows, row_dtype, n_rows, d_c, d_rope, out_rows, scales, stream)
    assert _st(lib, "mla_quantize_latent_i8", P, 1, 10, 512, 64, None, P, None) == 1
    assert _st(lib, "mla_quantize_latent_i8", P, 0, 10, 512, 64, P, P, None) == 3
    assert _st(lib, "mla_quantize_latent_i8", P, 1, 10, 1024, 64, P, P, None) == 2
    assert _st(lib, "mla_quantize_latent_i8", P, 1, 10, 500, 64, P, P, None) == 2
    assert _st(lib, "mla_quantize_latent_i8", P, 1, 10, 512, 66, P, P, None) == 2
    assert _st(lib, "mla_quantize_latent_i8", P + 4, 1, 10, 512, 64, P, P, None) == 4
    assert _st(lib, "mla_quantize_latent_i8", P, 1, 0, 512, 64, P, P, None) == 0
    assert _st(lib, "mla_quantize_latent_i8", P, 1, (1 << 32) + 1, 512, 64, P, P, None) == 2
    # mla_quantize_latent_i4(rows, row_dtype, n_rows, d_c, d_rope, out_rows, scales, stream)
    assert _st(lib, "mla_quantize_latent_i4", P, 1, 10, 512, 64, P, None, None) == 1
    assert _st(lib, "mla_quantize_latent_i4", P, 0, 10, 512, 64, P, P, None) == 3
    assert _st(lib, "mla_quantize_latent_i4", P, 1, 10, 1024, 64, P, P, None) == 2
    assert _st(lib, "mla_quantize_latent_i4", P, 1, 10, 512, 60, P, P, None) == 2
    assert _st(lib, "mla_quantize_latent_i4", P, 1, 10, 512, 0, P, P, None) == 2
    assert _st(lib, "mla_quantize_latent_i4", P, 1, 10, 512, 64, P + 2, P, None) == 4
    assert _st(lib, "mla_quantize_latent_i4", P, 1, 10, 512, 64, P, P + 4, None) == 4
    assert _st(lib, "mla_quantize_latent_i4", P, 1, 0, 512, 64, P, P, None) == 0
    # zero-size calls succeed without launching anything
    assert _st(lib, "mla_absorb_q", P, P, 1, P, 0, 0, 1, 128, 512, None) == 0

    def seg(**kw):
        s = MlaSegment()
        s.cache, s.seq_lens, s.q_rot = P, P, P
        s.max_rows, s.head_begin, s.head_count, s.part_begin, s.n_split = 64, 0, 4, 0, 2
        for k, v in kw.items():
            setattr(s, k, v)
        return s

    def dec(segs, n_heads=4, n_part=2, dtype=1, d_c=512, d_r=64, q=P, o=P, q_dtype=0, part_dtype=0, batch=2):
        # batch 0: every argument is checked, then nothing is launched (0 = accepted)
        arr = (MlaSegment * len(segs))(*segs)
        return _st(lib, "mla_decode_splitkv", arr, len(segs), q, q_dtype, dtype, batch, 1, n_heads, d_c, d_r,
                   0.1, o, part_dtype, P, n_part, 0, None)

    assert dec([seg()], q=None) == 1
    assert dec([seg(cache=None)]) == 1
    assert dec([seg()], d_c=256) == 5                     # bf16 needs d_c 512
    assert dec([seg()], q=P + 8) == 4                     # misaligned q_lat
    assert dec([seg(head_count=5)]) == 2                  # heads out of range
    assert dec([seg(n_split=3)]) == 2                     # slots past n_part
    assert dec([seg(n_split=1)]) == 2                     # slot 1 uncovered
    assert b"covered" in lib.mla_last_error()
    assert dec([seg(), seg()]) == 2                       # slots covered twice
    assert dec([seg(block_table=P, page_size=32, max_pages=4, n_pages=8)]) == 5  # bf16 page 64 only
    assert dec([seg(causal=2)]) == 2
    assert dec([seg(head_count=4)], n_heads=4, dtype=7) == 3
    assert dec([seg()], dtype=0, q_dtype=1) == 5          # fp32 cache needs an fp32 query
    assert dec([seg()], dtype=0, part_dtype=1) == 5       # and writes fp32 partials
    assert dec([seg()], part_dtype=3) == 3                # partials are fp32 or bf16
    assert dec([seg(row_rinv=P)], q_dtype=1) == 5         # QK-Norm factors need an fp32 or split query
    # row factors on every segment of a call or on none
    assert dec([seg(row_rinv=P, n_split=1), seg(part_begin=1, n_split=1)]) == 5
    assert dec([seg(n_split=1), seg(row_rinv=P, part_begin=1, n_split=1)]) == 5
    assert dec([seg(row_rinv=P, n_split=1), seg(row_rinv=P, part_begin=1, n_split=1)], batch=0) == 0
    # int8 cache (cache_dtype 2): fp32 or split query, row_scale on every segment, no QK-Norm
    assert dec([seg()], dtype=2) == 1                     # row_scale missing
    assert dec([seg(row_scale=P)], dtype=2, q_dtype=1) == 5
    assert dec([seg(row_scale=P, row_rinv=P)], dtype=2) == 5
    assert dec([seg(row_scale=P)], dtype=1) == 5          # row_scale only with a low-bit cache
    # int4 cache (cache_dtype 3): the same rules
    assert dec([seg()], dtype=3) == 1
    assert dec([seg(row_scale=P)], dtype=3, q_dtype=1) == 5
    assert dec([seg(row_scale=P, row_rinv=P)], dtype=3) == 5
    assert dec([seg(row_scale=P)], dtype=4) == 3
    # split query (q_dtype 4, bf16 hi and lo planes): bf16, int8 or int4 cache; QK-Norm with bf16 only
    assert dec([seg()], dtype=0, q_dtype=4) == 5
    assert dec([seg(row_scale=P)], dtype=2, q_dtype=4, batch=0) == 0
    assert dec([seg(row_scale=P)], dtype=3, q_dtype=4, batch=0) == 0
    assert dec([seg(row_rinv=P)], q_dtype=4, batch=0) == 0
    assert dec([seg()], q_dtype=5) == 3


def test_size_limits_refused(lib):
    """Sizes past the 32-bit index arithmetic of the kernels are refused on
    the host: split counts beyond the 15-bit slot field, segments holding more
    than 2^30 rows in all, and more than 2^20 query tokens per call."""
    from mla_latent_cache_amd._lib import MlaSegment
    P = 16

    def seg(**kw):
        s = MlaSegment()
        s.cache, s.seq_lens, s.q_rot = P, P, P
        s.max_rows, s.head_begin, s.head_count, s.part_begin, s.n_split = 64, 0, 4, 0, 2
        for k, v in kw.items():
            setattr(s, k, v)
        return s

    def dec(segs, n_part, batch=2):
        arr = (MlaSegment * len(segs))(*segs)
        return lib.mla_decode_splitkv(arr, len(segs), P, 0, 1, batch, 1, 4, 512, 64, 0.1, P, 0, P, n_part, 0, None)

    assert dec([seg(n_split=32768)], 32768) == 5
    assert b"n_split" in lib.mla_last_error()
    assert dec([seg(max_rows=1 << 29)], 2, batch=3) == 5           # 3 * 2^29 rows
    assert dec([seg(block_table=P, page_size=64, max_pages=1 << 25, n_pages=8)], 2) == 5
    assert dec([seg(max_rows=1 << 29)], 2, batch=0) == 0             # nothing to launch: accepted
    n = (1 << 20) + 1
    assert lib.rope_relocate_q(P, 1, P, 0, P, None, n, 1, 64, 1e4, None) == 2
    assert lib.mla_absorb_q(P, P, 1, P, 0, n, 1, 128, 512, None) == 2
    assert lib.mla_out_uv(P, 1, P, 1, P, 1, n, 1, 512, 128, None) == 2
    assert lib.mla_out_proj(P, 1, P, 1, P, 1, n, 256, 64, None) == 2
    assert lib.mla_prepare_q(P, 1, P, P, 1, P, 0, None, None, 0, 0, P, n, 4, 128, 64, 512, 1e4, None) == 2
