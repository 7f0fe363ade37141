"""Low-bit latent cache: plain per-row symmetric int8 and int4 quantizers, fp32 rules.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this file; it is used by the tests, by the smoke check and by the benchmark's
CPU-baseline leg.  It shares no code with the HIP library.

Source: the QuantMLA abstract (low-bit caching of the MLA content latent and
the rotary key, dequantized inside the attention kernel).  The page gives no
format and its transforms are learned, so this is the plainest quantizer its
description admits; the readings, also listed in the design notes:

* only the content latent c_t is quantized, to int8, with one scale per stored
  row; the rotary key stays in the cache's 16-bit form;
* symmetric, no zero point: amax = max_i |c_i|, scale = amax / 127, code_i =
  round_half_even(c_i / scale) clamped to [-127, 127]; a zero row has scale 0
  and codes 0;
* the decisions are taken in fp32 (the quotient amax / 127 and each c_i / scale
  rounded to fp32, then to the nearest integer, ties to even), so that the
  codes are one exact function of the stored bf16 latent;
* the latent the attention sees is the dequantized value scale * code; the
  decode then is the ordinary direct form (``mla_direct``) on those rows.

The int4 cache (the abstract's joint INT4 caching of the content and rotary
caches) applies the same rule with 4-bit codes to both parts of a row, each
with its own scale:

* content c_t and rotary key k^R_t are quantized separately: scale = amax / 7,
  code = round_half_even(x / scale) clamped to [-7, 7] (fp32 decisions, a
  zero part has scale 0 and codes 0);
* codes are stored two per byte, entry 2j in the low nibble and entry 2j + 1
  in the high nibble of byte j, as 4-bit two's complement;
* a stored row is [d_c / 2 content bytes | d_rope / 2 rotary bytes] and its
  two scales (content, rotary) are kept beside the cache.
"""
from __future__ import annotations

import numpy as np

QMAX = 127


def quantize_latent_i8(c: np.ndarray):
    """c [n, d_c] (values of the stored latent, any float dtype holding them
    exactly in fp32) -> (codes int8 [n, d_c], scales float32 [n])."""
    c32 = np.asarray(c, dtype=np.float32)
    amax = np.max(np.abs(c32), axis=1) if c32.shape[1] else np.zeros(c32.shape[0], np.float32)
    scales = (amax / np.float32(QMAX)).astype(np.float32)          # fp32 quotient, nearest
    codes = np.zeros(c32.shape, dtype=np.int8)
    nz = scales > 0
    q = c32[nz] / scales[nz][:, None]                               # fp32 quotient per entry
    codes[nz] = np.clip(np.rint(q), -QMAX, QMAX).astype(np.int8)    # nearest, ties to even
    return codes, scales


def dequantize_latent_i8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """scale * code in fp64: [n, d_c]."""
    return np.asarray(scales, np.float64)[:, None] * np.asarray(codes, np.float64)


def quantized_rows(rows: np.ndarray, d_c: int) -> np.ndarray:
    """Stored rows [n, d_c + d_rope] -> the rows attention reads from an int8
    cache: dequantized latent, rotary key unchanged (fp64)."""
    rows = np.asarray(rows)
    codes, scales = quantize_latent_i8(rows[:, :d_c])
    out = np.array(rows, dtype=np.float64)
    out[:, :d_c] = dequantize_latent_i8(codes, scales)
    return out


def cache_row_bytes_i8(d_c: int, d_rope: int, rope_bytes: int = 2, scale_bytes: int = 4) -> int:
    """Bytes per stored row: d_c one-byte codes, the rotary key, one scale."""
    return d_c + d_rope * rope_bytes + scale_bytes


# --------------------------------------------------------------------------
# int4: content and rotary key, one scale each per row
# --------------------------------------------------------------------------
QMAX4 = 7


def quantize_i4(x: np.ndarray):
    """x [n, d] -> (codes int8 in [-7, 7] [n, d], scales float32 [n]): the
    int8 rule with 7 in place of 127."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=1) if x32.shape[1] else np.zeros(x32.shape[0], np.float32)
    scales = (amax / np.float32(QMAX4)).astype(np.float32)
    codes = np.zeros(x32.shape, dtype=np.int8)
    nz = scales > 0
    q = x32[nz] / scales[nz][:, None]
    codes[nz] = np.clip(np.rint(q), -QMAX4, QMAX4).astype(np.int8)
    return codes, scales


def pack_i4(codes: np.ndarray) -> np.ndarray:
    """[n, d] codes (d even) -> uint8 [n, d / 2]: entry 2j in the low nibble of
    byte j, entry 2j + 1 in the high nibble, 4-bit two's complement."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_i4(packed: np.ndarray) -> np.ndarray:
    """uint8 [n, m] -> codes int8 [n, 2 m] (sign-extended nibbles)."""
    b = np.asarray(packed, dtype=np.int64)
    out = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.int64)
    out[:, 0::2] = b & 0xF
    out[:, 1::2] = (b >> 4) & 0xF
    return np.where(out >= 8, out - 16, out).astype(np.int8)


def quantize_cache_i4(rows: np.ndarray, d_c: int):
    """Stored rows [n, d_c + d_rope] -> (packed uint8 [n, (d_c + d_rope) / 2],
    scales float32 [n, 2] = (content, rotary))."""
    rows = np.asarray(rows)
    cc, sc = quantize_i4(rows[:, :d_c])
    cr, sr = quantize_i4(rows[:, d_c:])
    return np.concatenate([pack_i4(cc), pack_i4(cr)], axis=1), np.stack([sc, sr], axis=1)


def quantized_rows_i4(rows: np.ndarray, d_c: int) -> np.ndarray:
    """Stored rows -> the rows attention reads from an int4 cache: both parts
    dequantized (scale * code, fp64)."""
    packed, scales = quantize_cache_i4(rows, d_c)
    codes = unpack_i4(packed).astype(np.float64)
    out = np.empty(codes.shape, dtype=np.float64)
    out[:, :d_c] = np.asarray(scales[:, 0], np.float64)[:, None] * codes[:, :d_c]
    out[:, d_c:] = np.asarray(scales[:, 1], np.float64)[:, None] * codes[:, d_c:]
    return out


def cache_row_bytes_i4(d_c: int, d_rope: int, scale_bytes: int = 4) -> int:
    """Bytes per stored row: half a byte per entry, two scales."""
    return (d_c + d_rope) // 2 + 2 * scale_bytes
