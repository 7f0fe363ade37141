"""Low-bit latent cache: a plain per-row symmetric int8 quantizer, fp32 rules.

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
