"""Pins of the FP8 key oracle (oracle/fp8_ref.py).

* hand values: the E4M3 bit patterns of chosen inputs, worked by hand
  (1.0 = 0x38; 448 = 0x7E; 2^-9 = 0x01, the smallest subnormal; ties to the
  even code at 1.0625, 1.1875, 2^-10 and 464; saturation beyond 448);
* torch's own float8_e4m3fn cast (a library routine the oracle does not
  call), on all 48,768 fp16 inputs where the two readings agree
  (|x| < 464: torch returns NaN from 464 up, the oracle saturates);
* every finite E4M3 value encodes to its own code and decodes exactly;
* planted mistakes (ties away from zero, truncation, no saturation, a
  dropped sign) are caught.
"""

import numpy as np
import pytest
import torch

from oracle import fp8_ref as f8

F16 = np.float16

HAND = [(0.0, 0x00), (-0.0, 0x80), (1.0, 0x38), (-1.0, 0xB8), (1.0625, 0x38), (1.1875, 0x3A),
        (1.125, 0x39), (448.0, 0x7E), (464.0, 0x7E), (500.0, 0x7E), (-1000.0, 0xFE),
        (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (2.0 ** -6, 0x08),
        (0.015625 * 1.0625, 0x08), (240.0, 0x77), (256.0, 0x78), (-300.0, 0xF9), (65504.0, 0x7E)]


@pytest.mark.parametrize("x,code", HAND)
def test_hand_values(x, code):
    assert int(f8.encode(np.array([x], dtype=F16))[0]) == code


def _all_fp16():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16).view(F16)


def test_matches_torch_cast_where_both_readings_agree():
    x = _all_fp16()
    finite = np.isfinite(x) & (np.abs(x.astype(np.float64)) < 464.0)
    x = x[finite]
    want = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(f8.encode(x), want)
    assert x.size == 2 * 0x5F40          # both signs of every magnitude below 464 (= 0x5F40)


def test_saturates_beyond_the_largest_value():
    x = _all_fp16()
    big = np.isfinite(x) & (np.abs(x.astype(np.float64)) >= 448.0)
    codes = f8.encode(x[big])
    assert np.all((codes & 0x7F) == 0x7E)
    assert np.array_equal(codes >> 7, np.signbit(x[big]).astype(np.uint8))


def test_every_value_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = f8.decode(codes)
    assert np.array_equal(f8.encode(vals), codes)
    for c, v in zip(codes, vals):
        assert float(v) == f8.e4m3_value(int(c))


def test_encode_is_monotone():
    x = np.sort(_all_fp16()[np.isfinite(_all_fp16())].astype(np.float64)).astype(F16)
    v = f8.decode(f8.encode(x)).astype(np.float64)
    assert np.all(np.diff(v) >= 0)


# planted mistakes -----------------------------------------------------------

def _checks():
    return [lambda: [test_hand_values(x, c) for x, c in HAND],
            test_matches_torch_cast_where_both_readings_agree,
            test_saturates_beyond_the_largest_value]


def _caught():
    for chk in _checks():
        try:
            chk()
        except Exception:
            return True
    return False


def _ties_away(x):
    x = np.asarray(x, dtype=F16)
    a = np.abs(x.astype(np.float64))
    hi = np.clip(np.searchsorted(f8._VALS, a), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    pick_hi = np.abs(f8._VALS[hi] - a) <= np.abs(a - f8._VALS[lo])
    mag = np.where(pick_hi, f8._CODES[hi], f8._CODES[lo]).astype(np.uint8)
    mag = np.where(a >= 448, np.uint8(0x7E), mag)
    return mag | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))


def _truncate(x):
    x = np.asarray(x, dtype=F16)
    a = np.abs(x.astype(np.float64))
    idx = np.clip(np.searchsorted(f8._VALS, a, side="right") - 1, 0, 126)
    return f8._CODES[idx] | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))


def _no_saturation(x, _orig=f8.encode):
    c = _orig(x)
    a = np.abs(np.asarray(x, dtype=F16).astype(np.float64))
    return np.where(a >= 464, c | 0x7F, c).astype(np.uint8)


def _no_sign(x, _orig=f8.encode):
    return _orig(x) & np.uint8(0x7F)


@pytest.mark.parametrize("mutant", [_ties_away, _truncate, _no_saturation, _no_sign])
def test_planted_mistake_is_caught(monkeypatch, mutant):
    assert not _caught()
    monkeypatch.setattr(f8, "encode", mutant)
    assert _caught()
