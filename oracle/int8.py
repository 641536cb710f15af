"""Symmetric int8 KV codec (oracle, test infrastructure only).

The pages name int8 as a one-byte KV-cache element type beside fp8 (page "KV
cache & continuous batching", section "KV cache memory math": "1 for
fp8/int8"; page "LLM Inference Optimization: KV Cache, Batching, and
Speculative Decoding", section "Memory Bandwidth Optimization").  They give no
encoding; the reading taken is the plainest symmetric one:

* a stored code c is a two's-complement byte in [-127, 127] (the code -128 is
  never written) and stands for c * scale, with a float32 scale per (layer,
  KV head), separately for K and V;
* writing x: y = float32(float32(x) * float32(1/scale)); NaN becomes 0;
  y is rounded to the nearest integer, ties to even, then saturated to
  [-127, 127].

Pins (tests/test_oracle_int8.py): hand-worked codes, ties to even, saturation
and NaN, and torch's round-half-even + clamp on random values.
"""

import numpy as np

I8_MAX = 127


def encode(values):
    """float32-representable values -> int8 codes (round half to even, saturate, NaN -> 0)."""
    y = np.asarray(values, dtype=np.float64)
    y = np.where(np.isnan(y), 0.0, y)
    r = np.rint(y)                         # numpy rounds halves to even
    r = np.clip(r, -I8_MAX, I8_MAX)
    return r.astype(np.int8)


def quantize(x, scale):
    """Stored codes of values x (float32 array) for one (layer, head) scale."""
    x = np.asarray(x, dtype=np.float32)
    inv = np.float32(np.float32(1.0) / np.float32(scale))
    y = (x * inv).astype(np.float32)       # one float32 multiply, round to nearest
    return encode(y)


def decode(codes, scale=1.0):
    """int8 codes -> exact float64 values code * float32(scale)."""
    c = np.asarray(codes).astype(np.int8).astype(np.float64)
    return c * np.float64(np.float32(scale))
