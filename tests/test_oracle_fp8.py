"""Pins for the oracle's OCP E4M3 codec and cache-write quantization (CPU only)."""

import math

import numpy as np
import torch

from conftest import golden_lines
from oracle import fp8


def test_hand_worked_codes():
    rows = golden_lines("e4m3_codes.txt")
    assert len(rows) >= 15
    for code, value in rows:
        got = fp8.decode_code(int(code, 16))
        if value == "nan":
            assert math.isnan(got)
        else:
            assert got == float(value)
            assert math.copysign(1.0, got) == math.copysign(1.0, float(value))


def test_all_codes_against_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = fp8.decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert nan.sum() == 2
    assert np.array_equal(ours[~nan], ref[~nan])
    # the value order of non-negative codes is the code order (used by encode)
    assert (np.diff(fp8.DECODE_TABLE[:0x7F]) > 0).all()


def test_encode_is_exact_on_every_code():
    vals = fp8.DECODE_TABLE
    finite = ~np.isnan(vals)
    codes = np.arange(256)[finite]
    assert np.array_equal(fp8.encode(vals[finite]), codes.astype(np.uint8))


def test_midpoints_round_to_even_and_match_torch():
    pos = fp8.DECODE_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2.0
    got = fp8.encode(mids)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(got, expect)
    assert np.array_equal(fp8.encode(-mids), expect | 0x80)
    # torch's float -> e4m3fn conversion is round-to-nearest-even as well
    t = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, t)


def test_random_values_against_torch_after_clamp():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 1e-1, 1, 30, 300)])
    x = np.clip(x, -448, 448).astype(np.float32)
    ours = fp8.encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_saturation_nan_and_signed_zero():
    got = fp8.encode(np.array([449.0, 1e30, -1e30, 464.0, -0.0, -1e-9, float("nan")]))
    assert got[:5].tolist() == [0x7E, 0x7E, 0xFE, 0x7E, 0x80]
    assert got[5] == 0x80
    assert got[6] in (0x7F, 0xFF)


def test_quantize_rule_against_torch():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(50000) * 2.5).astype(np.float32)
    scale = np.float32(0.0093)
    ours = fp8.quantize(x, scale)
    t = torch.from_numpy(x) * torch.tensor(1.0, dtype=torch.float32).div(torch.tensor(scale))
    t = t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, t)
    # values beyond amax saturate instead of overflowing
    assert fp8.quantize(np.array([1e6, -1e6], np.float32), scale).tolist() == [0x7E, 0xFE]
