"""Pins for the oracle's symmetric int4 KV codec and nibble layout (CPU only)."""

import numpy as np
import torch

from conftest import golden_lines
from oracle import int4


def test_hand_worked_codes():
    rows = golden_lines("int4_codes.txt")
    assert len(rows) >= 15
    for x, scale, code in rows:
        got = int4.quantize(np.array([float(x)], np.float32), float(scale))[0]
        assert int(got) == int(code), (x, scale, code, got)


def test_ties_go_to_even_and_saturation():
    halves = np.arange(-10, 10, dtype=np.float64) + 0.5
    got = int4.encode(halves).astype(np.int64)
    lo = np.floor(halves)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    want = np.clip(want, -7, 7)
    assert np.array_equal(got, want)
    assert int4.encode(np.array([np.inf]))[0] == 7 and int4.encode(np.array([-np.inf]))[0] == -7
    assert (int4.encode(np.linspace(-1e6, 1e6, 1001)) >= -7).all()


def test_against_torch_round_and_clamp():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(20000) * 4).astype(np.float32)
    for scale in (1.0, 0.37, 0.125):
        ours = int4.quantize(x, scale)
        inv = torch.tensor(np.float32(1.0) / np.float32(scale))
        t = torch.from_numpy(x) * inv
        ref = torch.clamp(torch.round(t), -7, 7).to(torch.int8).numpy()
        assert np.array_equal(ours, ref)


def test_nibble_patterns_by_hand():
    # two's complement nibbles written out
    assert [int(int4.nibble_of(c)) for c in (-7, -4, -1, 0, 1, 7)] == [0x9, 0xC, 0xF, 0x0, 0x1, 0x7]
    assert [int(int4.code_of(n)) for n in (0x9, 0xC, 0xF, 0x0, 0x1, 0x7, 0x8)] == [-7, -4, -1, 0, 1, 7, -8]


def test_decode_is_code_times_scale():
    codes = np.arange(-7, 8)
    assert np.array_equal(int4.decode(codes, 0.5), codes.astype(np.float64) * 0.5)
    assert np.array_equal(int4.decode(int4.encode(codes.astype(np.float64))), codes.astype(np.float64))
