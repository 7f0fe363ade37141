"""Pins of the int8 latent quantizer in the oracle (``oracle/mla_quant.py``),
and planted mistakes in a copy of it that some pin must catch.

The quantizer follows the plainest reading of the QuantMLA abstract (per-row
symmetric int8 content codes, fp32 decisions); the pins fix what that reading
and the mathematics determine: exact codes where the scale is exactly 1 (ties
to even), the rounding bound, range and argmax codes, sign symmetry, exact
power-of-two scaling, the zero row, and a lossless case in which decoding the
quantized rows must equal decoding the original rows bit for bit.
"""
import sys
import types

import numpy as np
import pytest

import oracle.mla_direct as O
import oracle.mla_quant as Q

SRC = open(Q.__file__).read()


def pin_quant_exact_unit_scale(Q):
    """amax = 127 gives scale exactly 1, so the codes are the entries rounded
    to the nearest integer, ties to even."""
    c = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -126.5, 3.0, 126.5, -2.5]], np.float32)
    codes, scales = Q.quantize_latent_i8(c)
    assert scales.dtype == np.float32 and float(scales[0]) == 1.0, scales
    assert codes.dtype == np.int8
    assert codes[0].tolist() == [127, 0, 2, 2, 0, -2, -126, 3, 126, -2], codes[0].tolist()
    assert np.array_equal(Q.dequantize_latent_i8(codes, scales), codes.astype(np.float64))


def pin_quant_bound_and_range(Q):
    """Random rows of very different magnitudes: every code in [-127, 127],
    the largest entry at +-127, scale the fp32 quotient amax / 127 (within
    one unit in the last place of an fp64 division), and |c - s q| <= s / 2
    up to the fp32 rounding of the quotient c / s."""
    g = np.random.default_rng(5)
    c = (g.standard_normal((64, 512)) * np.exp(g.uniform(-12, 12, (64, 1)))).astype(np.float32)
    codes, scales = Q.quantize_latent_i8(c)
    assert codes.shape == c.shape and scales.shape == (64,)
    assert np.all(np.abs(codes.astype(np.int32)) <= 127)
    amax = np.max(np.abs(c.astype(np.float64)), axis=1)
    assert np.all(np.abs(scales.astype(np.float64) - amax / 127) <= amax / 127 * 2.0 ** -23)
    arg = np.argmax(np.abs(c), axis=1)
    assert np.array_equal(np.abs(codes[np.arange(64), arg].astype(np.int32)), np.full(64, 127))
    assert np.array_equal(np.sign(codes[np.arange(64), arg]), np.sign(c[np.arange(64), arg]).astype(np.int8))
    s = scales.astype(np.float64)[:, None]
    err = np.abs(c.astype(np.float64) - Q.dequantize_latent_i8(codes, scales))
    assert np.all(err <= s * (0.5 + 2.0 ** -16)), float(np.max(err / s))


def pin_quant_symmetry_and_scaling(Q):
    """quantize(-c) = (-codes, s); quantize(2^k c) = (codes, 2^k s) exactly
    (power-of-two scaling is exact in fp32 away from under/overflow)."""
    g = np.random.default_rng(6)
    c = g.standard_normal((8, 96)).astype(np.float32)
    codes, scales = Q.quantize_latent_i8(c)
    cn, sn = Q.quantize_latent_i8(-c)
    assert np.array_equal(cn, -codes) and np.array_equal(sn, scales)
    for k in (-9, -1, 3, 11):
        ck, sk = Q.quantize_latent_i8(c * np.float32(2.0 ** k))
        assert np.array_equal(ck, codes), k
        assert np.array_equal(sk, scales * np.float32(2.0 ** k)), k


def pin_quant_zero_and_per_row(Q):
    """A zero row: scale 0, codes 0.  Rows are independent: a row's codes do
    not change when another row is scaled."""
    c = np.zeros((3, 16), np.float32)
    c[1] = np.arange(16) - 7.5
    c[2] = np.linspace(-3, 5, 16)
    codes, scales = Q.quantize_latent_i8(c)
    assert float(scales[0]) == 0.0 and not np.any(codes[0])
    c2 = c.copy()
    c2[2] *= np.float32(1000.0)
    codes2, scales2 = Q.quantize_latent_i8(c2)
    assert np.array_equal(codes2[:2], codes[:2]) and np.array_equal(scales2[:2], scales[:2])


def pin_quant_lossless_decode(Q):
    """Latents that are integers with amax 127 in every row quantize without
    loss, so the decode over quantized rows equals the decode over the stored
    rows exactly; the rotary part passes through untouched."""
    g = np.random.default_rng(7)
    d_c, d_r, H, T = 8, 4, 2, 9
    c = g.integers(-126, 127, (T, d_c)).astype(np.float64)
    c[np.arange(T), g.integers(0, d_c, T)] = 127.0 * np.where(g.random(T) < 0.5, -1, 1)
    kr = g.standard_normal((T, d_r))
    rows = np.concatenate([c, kr], axis=1)
    qrows = Q.quantized_rows(rows, d_c)
    assert np.array_equal(qrows, rows)
    q_nope = g.standard_normal((1, H, 6))
    q_pe = g.standard_normal((1, H, d_r))
    w_uk = g.standard_normal((H, 6, d_c)) / 3
    w_uv = g.standard_normal((H, 5, d_c)) / 3
    seg = lambda f: [O.OracleSegment(rows=lambda b: f, shift=[0], head_begin=0, head_count=H, causal=False)]
    a = O.direct_mla_decode(q_nope, q_pe, np.array([T - 1]), w_uk, w_uv, seg(rows), 0.3, 10000.0, 1)
    b = O.direct_mla_decode(q_nope, q_pe, np.array([T - 1]), w_uk, w_uv, seg(qrows), 0.3, 10000.0, 1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def pin_quant_row_bytes(Q):
    """Stored bytes per row of the int8 cache: 512 codes, the 64-entry 16-bit
    rotary key and a 4-byte scale, against 1152 for the bf16 row."""
    assert Q.cache_row_bytes_i8(512, 64) == 644
    assert O.cache_bytes(1, 1, 1, 512, 64, 2) == 1152


def pin_i4_exact_unit_scale_and_packing(Q):
    """amax = 7 gives scale exactly 1: codes are the entries rounded to the
    nearest integer, ties to even; the packed bytes, written out by hand:
    (7, 0) -> 0x07, (2, 2) -> 0x22, (0, -2) -> 0xE0, (-6, 6) -> 0x6A,
    (-7, 3) -> 0x39."""
    c = np.array([[7.0, 0.5, 1.5, 2.5, -0.5, -1.5, -6.5, 6.5, -7.0, 3.0]], np.float32)
    codes, scales = Q.quantize_i4(c)
    assert float(scales[0]) == 1.0 and codes[0].tolist() == [7, 0, 2, 2, 0, -2, -6, 6, -7, 3], codes[0].tolist()
    packed = Q.pack_i4(codes)
    assert packed.dtype == np.uint8 and packed[0].tolist() == [0x07, 0x22, 0xE0, 0x6A, 0x39], packed[0].tolist()
    assert np.array_equal(Q.unpack_i4(packed), codes)


def pin_i4_brute_force(Q):
    """Against a pure-Python quantizer on small rows: content and rotary
    parts each with their own scale, every nibble checked one by one."""
    g = np.random.default_rng(8)
    d_c, d_r = 8, 4
    rows = (g.standard_normal((6, d_c + d_r)) * np.exp(g.uniform(-5, 5, (6, 1)))).astype(np.float32)
    rows[2, :d_c] = 0.0
    packed, scales = Q.quantize_cache_i4(rows, d_c)
    assert packed.shape == (6, (d_c + d_r) // 2) and scales.shape == (6, 2) and scales.dtype == np.float32
    for i in range(6):
        for part, (lo, hi) in enumerate([(0, d_c), (d_c, d_c + d_r)]):
            x = [float(v) for v in rows[i, lo:hi]]
            s = float(np.float32(np.float32(max(abs(v) for v in x)) / np.float32(7)))
            assert float(scales[i, part]) == s
            for k, v in enumerate(x):
                e = 0 if s == 0 else max(-7, min(7, int(np.rint(np.float32(np.float32(v) / np.float32(s))))))
                byte = int(packed[i, (lo + k) // 2])
                nib = (byte >> (4 * ((lo + k) % 2))) & 0xF
                assert (nib - 16 if nib >= 8 else nib) == e, (i, lo + k)


def pin_i4_bound_and_decode(Q):
    """|x - s code| <= s / 2 (up to the fp32 quotient) on both parts, the
    largest entry of each part at +-7; integer rows with a 7 in each part
    quantize without loss, so the decode over them is unchanged."""
    g = np.random.default_rng(9)
    d_c, d_r = 32, 8
    rows = (g.standard_normal((40, d_c + d_r)) * np.exp(g.uniform(-8, 8, (40, 1)))).astype(np.float32)
    deq = Q.quantized_rows_i4(rows, d_c)
    packed, scales = Q.quantize_cache_i4(rows, d_c)
    codes = Q.unpack_i4(packed)
    for part, (lo, hi) in enumerate([(0, d_c), (d_c, d_c + d_r)]):
        s = scales[:, part].astype(np.float64)[:, None]
        err = np.abs(rows[:, lo:hi].astype(np.float64) - deq[:, lo:hi])
        assert np.all(err <= s * (0.5 + 2.0 ** -16))
        arg = np.argmax(np.abs(rows[:, lo:hi]), axis=1)
        assert np.array_equal(np.abs(codes[np.arange(40), lo + arg].astype(np.int32)), np.full(40, 7))
    ints = g.integers(-6, 7, (5, d_c + d_r)).astype(np.float64)
    ints[:, 0] = 7.0
    ints[:, d_c] = -7.0
    assert np.array_equal(Q.quantized_rows_i4(ints, d_c), ints)


def pin_i4_row_bytes(Q):
    """An int4 row: 256 content bytes, 32 rotary bytes, two 4-byte scales
    (296 bytes against 1152 for the bf16 row)."""
    assert Q.cache_row_bytes_i4(512, 64) == 296


QUANT_PINS = [pin_quant_exact_unit_scale, pin_quant_bound_and_range, pin_quant_symmetry_and_scaling,
              pin_quant_zero_and_per_row, pin_quant_lossless_decode, pin_quant_row_bytes,
              pin_i4_exact_unit_scale_and_packing, pin_i4_brute_force, pin_i4_bound_and_decode, pin_i4_row_bytes]


@pytest.mark.parametrize("pin", QUANT_PINS, ids=lambda p: p.__name__)
def test_quant_pin(pin):
    pin(Q)


MUTANTS = {
    "i4_scale_8": ("scales = (amax / np.float32(QMAX4)).astype(np.float32)",
                   "scales = (amax / np.float32(8)).astype(np.float32)"),
    "i4_nibbles_swapped": ("return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)",
                           "return (c[:, 1::2] | (c[:, 0::2] << 4)).astype(np.uint8)"),
    "i4_no_sign_extend": ("return np.where(out >= 8, out - 16, out).astype(np.int8)", "return out.astype(np.int8)"),
    "i4_shared_scale": ("cr, sr = quantize_i4(rows[:, d_c:])",
                        "cr, sr = quantize_i4(rows[:, d_c:])\n    sr = sc\n    cr = np.clip(np.rint(np.where(sc[:, None] > 0, "
                        "rows[:, d_c:] / np.where(sc[:, None] > 0, sc[:, None], 1), 0)), -7, 7).astype(np.int8)"),
    "i4_round_half_away": ("codes[nz] = np.clip(np.rint(q), -QMAX4, QMAX4).astype(np.int8)",
                           "codes[nz] = np.clip(np.floor(q + 0.5), -QMAX4, QMAX4).astype(np.int8)"),
    "i4_rotary_scale_from_content": ("out[:, d_c:] = np.asarray(scales[:, 1], np.float64)[:, None] * codes[:, d_c:]",
                                     "out[:, d_c:] = np.asarray(scales[:, 0], np.float64)[:, None] * codes[:, d_c:]"),
    "scale_128": ("scales = (amax / np.float32(QMAX)).astype(np.float32)",
                  "scales = (amax / np.float32(128)).astype(np.float32)"),
    "round_half_away": ("np.clip(np.rint(q), -QMAX, QMAX)", "np.clip(np.floor(q + 0.5), -QMAX, QMAX)"),
    "truncate": ("np.clip(np.rint(q), -QMAX, QMAX)", "np.clip(np.trunc(q), -QMAX, QMAX)"),
    "per_tensor_amax": ("amax = np.max(np.abs(c32), axis=1) if c32.shape[1]",
                        "amax = np.full(c32.shape[0], np.max(np.abs(c32))) if c32.shape[1]"),
    "codes_wrong_sign": ("codes[nz] = np.clip(np.rint(q), -QMAX, QMAX).astype(np.int8)",
                                   "codes[nz] = np.clip(np.rint(-q), -QMAX, QMAX).astype(np.int8)"),
    "dequant_no_scale": ("return np.asarray(scales, np.float64)[:, None] * np.asarray(codes, np.float64)",
                         "return np.asarray(codes, np.float64)"),
    "rotary_quantized": ("out[:, :d_c] = dequantize_latent_i8(codes, scales)",
                         "out[:, :d_c] = dequantize_latent_i8(codes, scales)\n"
                         "    out[:, d_c:] = np.rint(out[:, d_c:] * 8) / 8"),
    "row_bytes_no_scale": ("return d_c + d_rope * rope_bytes + scale_bytes", "return d_c + d_rope * rope_bytes"),
}


def _mutant(old, new):
    assert old in SRC, f"mutation site vanished: {old!r}"
    mod = types.ModuleType("quant_mutant")
    mod.__file__ = Q.__file__
    sys.modules["quant_mutant"] = mod
    try:
        exec(compile(SRC.replace(old, new), "quant_mutant", "exec"), mod.__dict__)
    finally:
        del sys.modules["quant_mutant"]
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_quant_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    caught = []
    for pin in QUANT_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"mutant {name} passed every pin"
