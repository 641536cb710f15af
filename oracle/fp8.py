"""OCP FP8 E4M3 ("e4m3fn") codec (oracle, test infrastructure only).

The pages fix only that an fp8 KV element takes one byte (page "KV cache &
continuous batching", section "KV cache memory math"; page "LLM Inference
Optimization: KV Cache, Batching, and Speculative Decoding", section "Memory
Bandwidth Optimization").  Which 8-bit float is not on the pages; the reading
taken is the OCP 8-bit floating point specification's E4M3 format:

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field 0 encodes subnormals  (-1)^s * 2^-6 * m/8;
* exponent fields 1..15 encode normals (-1)^s * 2^(e-7) * (1 + m/8);
* S.1111.111 is NaN; there are no infinities; the largest finite value is 448.

Encoding is round-to-nearest, ties to even (the even code), saturating to
+-448 for finite inputs beyond it; NaN stays NaN (code 0x7F or 0xFF).

The cache-write quantization rule (reading of the fp8 variant of the slot
write; the pages give no rule) is:  y = float32(float32(x) * float32(1/scale)),
then saturate to [-448, 448], then encode.  ``quantize`` follows it step by step
in float32 so that a byte-for-byte comparison is meaningful.

Pins: all 256 codes against the closed form above evaluated by hand in the
tests, against ``torch.float8_e4m3fn`` (a library routine), and every midpoint
between neighbouring codes rounding to the even code.
"""

import numpy as np

E4M3_MAX = 448.0


def decode_code(code):
    """Exact value of one E4M3 code as a Python float (NaN for the NaN codes)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (2.0 ** -6) * (m / 8.0)
    return sign * (2.0 ** (e - 7)) * (1.0 + m / 8.0)


# Value of every code, built once from the definition above.
DECODE_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)

# Non-negative finite codes 0x00..0x7E in increasing value order (the code
# order is the value order for a sign-magnitude format).
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = DECODE_TABLE[:0x7F]


def decode(codes):
    """Vectorised decode: uint8 array of codes -> float64 values."""
    codes = np.asarray(codes, dtype=np.uint8)
    return DECODE_TABLE[codes.astype(np.int64)]


def encode(values):
    """Round-to-nearest-even E4M3 encoding of float values (saturating).

    Each finite |x| is placed between its two neighbouring representable
    non-negative values; the nearer one wins and an exact tie goes to the even
    code.  |x| >= 448 gives 448.  The sign bit is copied from x (so -0.0 and
    small negatives that round to zero give 0x80).  NaN gives 0x7F|sign.
    """
    x = np.asarray(values, dtype=np.float64)
    sign = np.where(np.signbit(x), 0x80, 0x00).astype(np.int64)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, np.abs(x))
    sat = a >= E4M3_MAX
    a = np.where(sat, 0.0, a)
    # neighbours: hi = first representable value >= a, lo = the one below it
    hi = np.searchsorted(_POS_VALUES, a, side="left")
    lo = np.maximum(hi - 1, 0)
    exact = _POS_VALUES[hi] == a
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    tie_pick = np.where(lo % 2 == 0, lo, hi)
    code = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, tie_pick))
    code = np.where(exact, hi, code)
    code = np.where(sat, 0x7E, code)
    code = np.where(nan, 0x7F, code)
    return (code | sign).astype(np.uint8)


def quantize(x_f32, scale):
    """Cache-write quantization of float32 inputs with one float32 scale.

    y = f32(x * f32(1/scale)) in float32 arithmetic; saturate to +-448 with
    comparisons that let NaN through; then ``encode``.
    """
    x = np.asarray(x_f32, dtype=np.float32)
    inv = np.float32(1.0) / np.float32(scale)
    y = (x * inv).astype(np.float32)
    y = np.where(y > np.float32(E4M3_MAX), np.float32(E4M3_MAX), y)
    y = np.where(y < np.float32(-E4M3_MAX), np.float32(-E4M3_MAX), y)
    return encode(y.astype(np.float64))
