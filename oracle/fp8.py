"""OCP 8-bit float E4M3 ("e4m3fn"), written from the format definition.

TEST INFRASTRUCTURE: see the package docstring.

A code is 1 sign bit, 4 exponent bits (bias 7) and 3 mantissa bits.
  * exponent field e = 0: subnormal, value (m / 8) * 2^-6;
  * e in 1..15: value (1 + m / 8) * 2^(e - 7), except e = 15, m = 7:
    not a number (S.1111.111); there is no infinity, the largest finite
    magnitude is 448 (S.1111.110).
A KV pool in this format stores codes; the value of a key element is
decode(code) * k_scale (values likewise with v_scale), one float32 scale
per pool.  The pages name cache quantization as the complementary way to
fit more tokens ("PagedAttention KV cache memory management" [AITJ],
"PagedAttention vs KV-cache quantization vs prefix caching").

Encoding (how reshape_and_cache quantizes a new token) is a reading, as the
pages give none: the float32 quotient x / scale, computed in float32, is
rounded to the nearest code, ties to the even mantissa; magnitudes at or
beyond 448 saturate to +-448; NaN becomes 0x7F.

Parity: pinned (all 256 codes against torch's float8_e4m3fn decoding and
hand values; encoding against torch's rounding wherever torch keeps a
finite value, the round trip of every code, ties, saturation and NaN).
"""

import numpy as np

MAX = 448.0
NAN_CODE = 0x7F


def e4m3_decode(codes):
    """float64 values of e4m3 codes (uint8 array)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_encode(x):
    """e4m3 codes (uint8) of float32 values: nearest code, ties to even,
    saturating at +-448, NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)   # exact
    a = np.abs(x)
    # subnormal grid below 2^-6: multiples of 2^-9 (8 lands on 2^-6 = code 8)
    q_sub = np.rint(a * 512.0)
    # normal: a = (1 + f) * 2^E with f in [0, 1); 3 mantissa bits
    with np.errstate(divide="ignore", invalid="ignore"):
        mant, exp = np.frexp(a)                                # a = mant * 2^exp, mant in [0.5, 1)
    f8 = np.rint((2.0 * mant - 1.0) * 8.0)
    E = exp - 1 + (f8 == 8)
    f8 = np.where(f8 == 8, 0.0, f8)
    code_norm = (E + 7) * 8 + f8
    code = np.where(a < 2.0 ** -6, q_sub, code_norm)
    code = np.where(a >= MAX, 126.0, code)                     # saturate (inf included)
    code = np.where(np.isnan(x), 0.0, code)
    code = code.astype(np.int64) + np.where(np.signbit(x) & ~np.isnan(x), 128, 0)
    code = np.where(np.isnan(x), NAN_CODE, code)
    return code.astype(np.uint8)


def quantize(values, dtype, scale):
    """Codes of storage-format values divided by a float32 scale, the
    quotient taken in float32 (one rounding), then encoded."""
    from .formats import to_f64
    v = to_f64(values, dtype).astype(np.float32)               # exact for f16/bf16/f32
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = v / np.float32(scale)
    return e4m3_encode(q)
