"""FP8 keys for the k8v4 cache layout -- oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

vLLM ``turboquant/config.py``: the ``turboquant_k8v4`` preset stores keys
with 8 bits and values with 4; its ``TurboQuantConfig`` docstring says 8-bit
keys are FP8 (no rotation, no MSE codebook), and ``key_packed_size`` gives
one byte per element with no overhead, i.e. a plain cast with no scale.
``value_packed_size`` gives ``ceil(D*b/8) + 4`` bytes per value vector: a
uniform code with one fp16 scale and zero per vector, which is the KIVI
value codec with one group spanning the head.

Readings (the page names neither the FP8 variant nor its rounding):

* the OCP E4M3 format ("e4m3fn"): 1 sign, 4 exponent bits (bias 7), 3
  mantissa bits, subnormals, no infinities, NaN only at S.1111.111, largest
  finite magnitude 448;
* round to nearest, ties to the even code (the one with an even last
  mantissa bit), sign kept (so -0 -> 0x80);
* saturating: magnitudes beyond 448 give +-448 (a NaN would poison every
  attention score that reads the key).

The encoder is the definition written out: every finite E4M3 value is
listed, and each input takes the nearest one.
"""

from __future__ import annotations

import numpy as np

F16 = np.float16
MAX_E4M3 = 448.0


def e4m3_value(code: int) -> float:
    """Exact value of an E4M3 code (NaN for S.1111.111)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9                 # subnormal: m/8 * 2^(1-7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def _magnitudes():
    """Codes 0x00 .. 0x7E and their values, ascending (all finite, >= 0)."""
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = np.array([e4m3_value(int(c)) for c in codes], dtype=np.float64)
    assert np.all(np.diff(vals) > 0)
    return codes, vals


_CODES, _VALS = _magnitudes()


def encode(x) -> np.ndarray:
    """fp16 array -> uint8 E4M3 codes (nearest, ties to even code, saturating)."""
    x = np.asarray(x, dtype=F16)
    a = np.abs(x.astype(np.float64))
    neg = np.signbit(x)
    hi = np.clip(np.searchsorted(_VALS, a, side="left"), 0, len(_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(_VALS) - 1)
    d_lo = np.abs(a - _VALS[lo])
    d_hi = np.abs(_VALS[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_CODES[hi] & 1) == 0))
    mag = np.where(pick_hi, _CODES[hi], _CODES[lo]).astype(np.uint8)
    mag = np.where(a >= MAX_E4M3, np.uint8(0x7E), mag)            # saturate
    return (mag | np.where(neg, np.uint8(0x80), np.uint8(0))).astype(np.uint8)


def decode(codes) -> np.ndarray:
    """uint8 E4M3 codes -> fp16 (exact: every E4M3 value is an fp16 value)."""
    table = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)].astype(F16)


def encode_keys(k, n_tokens: int) -> np.ndarray:
    """Keys ``[S, T_alloc, D]`` fp16 -> FP8 codes ``[S, n_tokens, D]``."""
    return encode(np.asarray(k, dtype=F16)[:, :n_tokens, :])
