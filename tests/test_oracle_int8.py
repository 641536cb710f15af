"""Pins for the oracle's symmetric int8 KV codec (CPU only)."""

import numpy as np
import torch

from conftest import golden_lines
from oracle import int8


def test_hand_worked_codes():
    rows = golden_lines("int8_codes.txt")
    assert len(rows) >= 15
    for x, scale, code in rows:
        got = int8.quantize(np.array([float(x)], np.float32), float(scale))[0]
        assert int(got) == int(code), (x, scale, code, got)


def test_ties_go_to_even_and_saturation():
    halves = np.arange(-130, 130, dtype=np.float64) + 0.5
    got = int8.encode(halves).astype(np.int64)
    lo = np.floor(halves)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    want = np.clip(want, -127, 127)
    assert np.array_equal(got, want)
    assert int8.encode(np.array([np.inf]))[0] == 127 and int8.encode(np.array([-np.inf]))[0] == -127
    assert (int8.encode(np.linspace(-1e6, 1e6, 1001)) >= -127).all()


def test_against_torch_round_and_clamp():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(20000) * 60).astype(np.float32)
    for scale in (1.0, 0.37, 0.03125):
        ours = int8.quantize(x, scale)
        inv = torch.tensor(np.float32(1.0) / np.float32(scale))
        t = torch.from_numpy(x) * inv
        ref = torch.clamp(torch.round(t), -127, 127).to(torch.int8).numpy()
        assert np.array_equal(ours, ref)


def test_decode_is_code_times_scale():
    codes = np.arange(-127, 128).astype(np.int8)
    assert np.array_equal(int8.decode(codes, 0.5), codes.astype(np.float64) * 0.5)
    assert np.array_equal(int8.decode(int8.encode(codes.astype(np.float64))), codes.astype(np.float64))
