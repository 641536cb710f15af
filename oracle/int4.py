"""Symmetric int4 KV codec (oracle, test infrastructure only).

The pages name int4 as a half-byte KV-cache element type (page "LLM Inference
Optimization: KV Cache, Batching, and Speculative Decoding", section "Memory
Bandwidth Optimization": KV cache quantisation to int8 or int4 shrinks the
bytes a decode step reads).  They give no encoding; the reading taken is the
plainest symmetric one, the same as for int8 with a 4-bit range:

* a stored code c is a two's-complement nibble in [-7, 7] (the code -8 is
  never written) and stands for c * scale, with a float32 scale per (layer,
  KV head), separately for K and V;
* writing x: y = float32(float32(x) * float32(1/scale)); NaN becomes 0;
  y is rounded to the nearest integer, ties to even, then saturated to
  [-7, 7];
* two codes share a byte, the element with the even nibble index in the low
  half (the nibble layout of the pool is in oracle/pool.py).

Pins (tests/test_oracle_int4.py): hand-worked codes (tests/golden/
int4_codes.txt), ties to even and saturation, torch's round-half-even + clamp
on random values, and the nibble packing against hand-written bytes.
"""

import numpy as np

I4_MAX = 7


def encode(values):
    """float32-representable values -> int4 codes as int8 (round half to even, saturate, NaN -> 0)."""
    y = np.asarray(values, dtype=np.float64)
    y = np.where(np.isnan(y), 0.0, y)
    r = np.rint(y)                         # numpy rounds halves to even
    r = np.clip(r, -I4_MAX, I4_MAX)
    return r.astype(np.int8)


def quantize(x, scale):
    """Codes (int8 in [-7, 7]) of values x (float32 array) for one (layer, head) scale."""
    x = np.asarray(x, dtype=np.float32)
    inv = np.float32(np.float32(1.0) / np.float32(scale))
    y = (x * inv).astype(np.float32)       # one float32 multiply, round to nearest
    return encode(y)


def decode(codes, scale=1.0):
    """int4 codes (any integer array in [-8, 7]) -> exact float64 values code * float32(scale)."""
    c = np.asarray(codes).astype(np.int64).astype(np.float64)
    return c * np.float64(np.float32(scale))


def nibble_of(code):
    """The 4-bit two's-complement pattern of a code."""
    return np.asarray(code).astype(np.int64) & 0xF


def code_of(nibble):
    """Signed value of a 4-bit pattern."""
    n = np.asarray(nibble).astype(np.int64) & 0xF
    return np.where(n >= 8, n - 16, n)
