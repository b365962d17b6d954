"""KIVI grouped KV-cache codec -- exact-rational scalar oracle tier.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Pure Python: every
value is a ``fractions.Fraction``; rounding into binary16 / binary32 is done
by :func:`round_binary`, written here from the IEEE 754 definition of the
formats (round to nearest, ties to even, gradual underflow).  It uses no
floating-point hardware at all, so agreement with :mod:`oracle.kivi_ref`
pins that tier's use of numpy's float32 division, ``rint`` and float16
conversion.

Same method and readings as :mod:`oracle.kivi_ref` (CacheForge README,
"How it works"; CacheSeek PR #4 description): min/max statistics over the
valid elements of a group, ``scale = fp16(fp32(fp32(mx-mn)/(2**b-1)))``,
``zero = mn``, ``q = clamp(rint(fp32(fp32(x-zero)/scale)), 0, 2**b-1)``
(``q = 0`` when ``scale == 0``), LSB-first packing into 32-bit words, and
``xhat = fp16(fp32(q*scale + zero))``.  Meant for tiny inputs only.
"""

from __future__ import annotations

from fractions import Fraction

# (precision p including the hidden bit, minimum normal exponent, maximum exponent)
BINARY16 = (11, -14, 15)
BINARY32 = (24, -126, 127)


class Overflow(ArithmeticError):
    """The rounded magnitude exceeds the format's largest finite value."""


def _floor_log2(x: Fraction) -> int:
    """Largest e with 2**e <= x, for x > 0."""
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    elif Fraction(2) ** (e + 1) <= x:
        e += 1
    return e


def round_half_even(m: Fraction) -> int:
    """Nearest integer to ``m``, ties to the even integer."""
    fl = m.numerator // m.denominator
    r = m - fl
    if r > Fraction(1, 2):
        return fl + 1
    if r < Fraction(1, 2):
        return fl
    return fl + (fl & 1)


def round_binary(x: Fraction, fmt) -> Fraction:
    """Round ``x`` to the binary format ``fmt`` (round to nearest, ties to
    even, subnormals kept).  Raises :class:`Overflow` past the largest
    finite value."""
    p, emin, emax = fmt
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = -x if x < 0 else x
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - (p - 1))
    n = round_half_even(a / quantum)
    r = n * quantum
    if r >= Fraction(2) ** (emax + 1):
        raise Overflow(x)
    return sign * r


def f32(x) -> Fraction:
    return round_binary(Fraction(x), BINARY32)


def f16(x) -> Fraction:
    return round_binary(Fraction(x), BINARY16)


def f16_value(bits: int) -> Fraction:
    """Value of a finite binary16 bit pattern (negative zero maps to 0)."""
    bits &= 0xFFFF
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 10) & 0x1F
    frac = bits & 0x3FF
    if exp == 0x1F:
        raise ValueError("inf/nan is outside the codec's contract")
    if exp == 0:
        return sign * Fraction(frac, 1 << 24)
    return sign * Fraction(1024 + frac, 1024) * Fraction(2) ** (exp - 15)


def f16_bits(value: Fraction) -> int:
    """Bit pattern of a value exactly representable in binary16 (0 -> +0,
    too large -> +/-inf)."""
    value = Fraction(value)
    if value == 0:
        return 0
    sign = 0x8000 if value < 0 else 0
    a = -value if value < 0 else value
    if a >= 65520:          # rounds to infinity
        return sign | 0x7C00
    e = _floor_log2(a)
    if e < -14:
        m = a * (1 << 24)
        assert m.denominator == 1 and m < 1024, value
        return sign | int(m)
    m = a / Fraction(2) ** (e - 10)
    assert m.denominator == 1 and 1024 <= m < 2048, value
    return sign | ((e + 15) << 10) | (int(m) - 1024)


# ---------------------------------------------------------------------------
# one group
# ---------------------------------------------------------------------------

def group_params(xs_bits, bits: int):
    """``(scale_bits, zero_bits)`` of one group given its valid fp16 bit
    patterns."""
    vals = [f16_value(b) for b in xs_bits]
    mn, mx = min(vals), max(vals)
    rng = f32(mx - mn)
    s32 = f32(rng / (2 ** bits - 1))
    scale = f16(s32)
    return f16_bits(scale), f16_bits(mn)


def quantize(x_bits: int, scale_bits: int, zero_bits: int, bits: int) -> int:
    """Code of one fp16 value."""
    s = f16_value(scale_bits)
    if s == 0:
        return 0
    d = f32(f16_value(x_bits) - f16_value(zero_bits))
    quot = f32(d / s)
    q = round_half_even(quot)
    return min(max(q, 0), 2 ** bits - 1)


def dequantize(q: int, scale_bits: int, zero_bits: int) -> int:
    """fp16 bit pattern of the reconstruction of code ``q``."""
    prod = q * f16_value(scale_bits)
    assert f32(prod) == prod          # exact: <= 8-bit code x 11-bit significand
    try:
        y = f32(prod + f16_value(zero_bits))
        return f16_bits(f16(y))
    except Overflow:
        return 0x7C00 if prod + f16_value(zero_bits) > 0 else 0xFC00


def nearest_level(x_bits: int, scale_bits: int, zero_bits: int, bits: int):
    """All codes ``q`` in ``[0, 2**b-1]`` minimising ``|x - (zero + q*scale)|``
    in exact arithmetic (one code, or two at an exact tie)."""
    x, s, z = f16_value(x_bits), f16_value(scale_bits), f16_value(zero_bits)
    errs = [abs(x - (z + q * s)) for q in range(2 ** bits)]
    best = min(errs)
    return [q for q, e in enumerate(errs) if e == best]


def pack(codes, bits: int):
    """LSB-first packing of a code list (length a multiple of 32/bits)."""
    per = 32 // bits
    assert len(codes) % per == 0
    out = []
    for w in range(len(codes) // per):
        word = 0
        for i in range(per):
            c = codes[w * per + i]
            assert 0 <= c < 2 ** bits
            word += c * 2 ** (bits * i)
        out.append(word)
    return out


def unpack(words, bits: int):
    per = 32 // bits
    out = []
    for word in words:
        for i in range(per):
            out.append((word // 2 ** (bits * i)) % 2 ** bits)
    return out


# ---------------------------------------------------------------------------
# whole tensors as nested lists of fp16 bit patterns, [S][T][D]
# ---------------------------------------------------------------------------

def _ceil_div(a, b):
    return -(-a // b)


def encode_k(k_bits16, n_tokens: int, bits: int, group_size: int):
    """Keys: ``k_bits16[s][t][d]`` -> ``(words[s][row][d], scale[s][g][d],
    zero[s][g][d])`` as Python ints (words unsigned)."""
    G = group_size
    S, D = len(k_bits16), len(k_bits16[0][0])
    ng = _ceil_div(n_tokens, G)
    W = G * bits // 32
    words = [[[0] * D for _ in range(ng * W)] for _ in range(S)]
    scale = [[[0] * D for _ in range(ng)] for _ in range(S)]
    zero = [[[0] * D for _ in range(ng)] for _ in range(S)]
    for s in range(S):
        for g in range(ng):
            toks = range(g * G, min((g + 1) * G, n_tokens))
            for d in range(D):
                col = [k_bits16[s][t][d] for t in toks]
                sb, zb = group_params(col, bits)
                scale[s][g][d], zero[s][g][d] = sb, zb
                codes = [quantize(x, sb, zb, bits) for x in col]
                codes += [0] * (G - len(codes))
                for w, word in enumerate(pack(codes, bits)):
                    words[s][g * W + w][d] = word
    return words, scale, zero


def encode_v(v_bits16, n_tokens: int, bits: int, group_size: int):
    """Values: ``v_bits16[s][t][d]`` -> ``(words[s][t][col], scale[s][t][g],
    zero[s][t][g])``."""
    G = group_size
    S, D = len(v_bits16), len(v_bits16[0][0])
    ng = _ceil_div(D, G)
    words = [[None] * n_tokens for _ in range(S)]
    scale = [[[0] * ng for _ in range(n_tokens)] for _ in range(S)]
    zero = [[[0] * ng for _ in range(n_tokens)] for _ in range(S)]
    for s in range(S):
        for t in range(n_tokens):
            row_words = []
            for g in range(ng):
                chans = range(g * G, min((g + 1) * G, D))
                grp = [v_bits16[s][t][c] for c in chans]
                sb, zb = group_params(grp, bits)
                scale[s][t][g], zero[s][t][g] = sb, zb
                codes = [quantize(x, sb, zb, bits) for x in grp]
                codes += [0] * (G - len(codes))
                row_words += pack(codes, bits)
            words[s][t] = row_words
    return words, scale, zero


def decode_k(words, scale, zero, n_tokens: int, bits: int, group_size: int):
    G = group_size
    W = G * bits // 32
    S, D = len(words), len(words[0][0])
    out = [[[0] * D for _ in range(n_tokens)] for _ in range(S)]
    for s in range(S):
        for t in range(n_tokens):
            g, j = divmod(t, G)
            per = 32 // bits
            w, i = divmod(j, per)
            for d in range(D):
                q = unpack([words[s][g * W + w][d]], bits)[i]
                out[s][t][d] = dequantize(q, scale[s][g][d], zero[s][g][d])
    return out


def decode_v(words, scale, zero, n_tokens: int, bits: int, group_size: int, head_dim: int):
    G = group_size
    S = len(words)
    out = [[[0] * head_dim for _ in range(n_tokens)] for _ in range(S)]
    for s in range(S):
        for t in range(n_tokens):
            codes = unpack(words[s][t], bits)
            for d in range(head_dim):
                g = d // G
                out[s][t][d] = dequantize(codes[d], scale[s][t][g], zero[s][t][g])
    return out
