"""The pins in test_oracle_pins.py must catch plausible slips in the oracle.

Each case plants one mistake in the numpy oracle (on the CPU, through
monkeypatching) and runs a selection of the pin checks; at least one of them
must fail.  Nothing here touches a GPU.
"""

import numpy as np
import pytest

from oracle import kivi_ref as ref
import tests.test_oracle_pins as pins

F16, F32 = np.float16, np.float32


def _golden_hand(golden_dir):
    return {c["name"]: c for c in pins._load(golden_dir, "hand_worked_groups.json")["cases"]}


def _checks(golden_dir):
    hand = _golden_hand(golden_dir)
    return [
        lambda: [pins.test_hand_worked_value_groups(hand, n) for n in
                 ("A_values_b4", "B_ties_to_even_b2", "C_representable_grid_b2", "E_constant_group_b4")],
        lambda: pins.test_hand_worked_padded_key_group(hand),
        lambda: [pins.test_exact_tier_matches_numpy_tier(m, b, 32)
                 for m in ("normal", "tiny", "coarse") for b in (2, 4, 8)],
        lambda: pins.test_rounding_is_half_even_not_half_up_or_truncation(),
        lambda: pins.test_subnormal_scale_clamps_codes(),
        lambda: pins.test_signed_zero_is_canonical(),
        lambda: pins.test_key_words_pack_along_tokens_and_value_words_along_channels(),
        lambda: [pins.test_error_bound(b, k) for b in (2, 4) for k in ("k", "v")],
        lambda: [pins.test_exact_tie_quotients_round_to_even(b) for b in (4, 8)],
        lambda: pins.test_scale_is_rounded_twice(),
    ]


def _caught(golden_dir):
    for chk in _checks(golden_dir):
        try:
            chk()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return True
    return False


def _group_params_levels_off_by_one(x, bits):
    x32 = np.asarray(x).astype(F32)
    mn = x32.min(axis=-1) + F32(0)
    mx = x32.max(axis=-1) + F32(0)
    s32 = ((mx - mn) / F32(2 ** bits)).astype(F32)          # 2**b instead of 2**b - 1
    return s32.astype(F16), mn.astype(F16)


def _group_params_no_canonical_zero(x, bits):
    x32 = np.asarray(x).astype(F32)
    mn, mx = x32.min(axis=-1), x32.max(axis=-1)
    s32 = ((mx - mn) / F32(2 ** bits - 1)).astype(F32)
    return s32.astype(F16), mn.astype(F16)


def _group_params_scale_in_fp64(x, bits):
    x64 = np.asarray(x).astype(np.float64)
    mn, mx = x64.min(axis=-1) + 0.0, x64.max(axis=-1) + 0.0
    return ((mx - mn) / (2 ** bits - 1)).astype(F16), mn.astype(F16)


def _quantize_half_up(x, scale, zero, bits):
    x32 = np.asarray(x).astype(F32)
    s32 = np.broadcast_to(np.asarray(scale).astype(F32), x32.shape)
    d = (x32 - np.asarray(zero).astype(F32)).astype(F32)
    q = np.zeros(d.shape, F32)
    np.divide(d, s32, out=q, where=s32 != 0)
    return np.clip(np.floor(q + F32(0.5)), 0, 2 ** bits - 1).astype(np.uint32)


def _quantize_no_clamp(x, scale, zero, bits):
    x32 = np.asarray(x).astype(F32)
    s32 = np.broadcast_to(np.asarray(scale).astype(F32), x32.shape)
    d = (x32 - np.asarray(zero).astype(F32)).astype(F32)
    q = np.zeros(d.shape, F32)
    np.divide(d, s32, out=q, where=s32 != 0)
    return (np.rint(q).astype(np.uint32)) & np.uint32(0xFFFF)


def _quantize_reciprocal(x, scale, zero, bits):
    x32 = np.asarray(x).astype(F32)
    s32 = np.broadcast_to(np.asarray(scale).astype(F32), x32.shape)
    d = (x32 - np.asarray(zero).astype(F32)).astype(F32)
    r = np.zeros(d.shape, F32)
    np.divide(F32(1), s32, out=r, where=s32 != 0)
    q = (d * r).astype(F32)
    return np.clip(np.rint(q), 0, 2 ** bits - 1).astype(np.uint32)


def _pack_msb_first(codes, bits):
    per = 32 // bits
    c = np.asarray(codes).astype(np.uint32)
    c = c.reshape(c.shape[:-1] + (c.shape[-1] // per, per))
    w = np.zeros(c.shape[:-1], np.uint32)
    for i in range(per):
        w |= c[..., i] << np.uint32(bits * (per - 1 - i))
    return w


def _unpack_msb_first(words, bits):
    per = 32 // bits
    w = np.asarray(words).astype(np.uint32)
    out = np.empty(w.shape + (per,), np.uint32)
    for i in range(per):
        out[..., i] = (w >> np.uint32(bits * (per - 1 - i))) & np.uint32(2 ** bits - 1)
    return out.reshape(w.shape[:-1] + (w.shape[-1] * per,))


def _dequantize_fp16_math(codes, scale, zero):
    return (np.asarray(codes).astype(F16) * np.asarray(scale).astype(F16)
            + np.asarray(zero).astype(F16)).astype(F16)


def _encode_k_stats_over_padding(k, n_tokens, bits, group_size):
    k = np.asarray(k, dtype=F16).copy()
    ng = ref.n_groups(n_tokens, group_size)
    kp = np.zeros((k.shape[0], ng * group_size, k.shape[2]), F16)
    kp[:, :n_tokens] = k[:, :n_tokens]
    return _orig_encode_k(kp, ng * group_size, bits, group_size)


_orig_encode_k = ref.encode_k

MUTATIONS = {
    "levels_2b": ("group_params", _group_params_levels_off_by_one),
    "no_canonical_zero": ("group_params", _group_params_no_canonical_zero),
    "scale_in_fp64": ("group_params", _group_params_scale_in_fp64),
    "round_half_up": ("quantize", _quantize_half_up),
    "no_clamp": ("quantize", _quantize_no_clamp),
    "reciprocal_multiply": ("quantize", _quantize_reciprocal),
    "msb_first_packing": ("pack_words", _pack_msb_first),
    "fp16_decode_math": ("dequantize", _dequantize_fp16_math),
    "stats_over_padding": ("encode_k", _encode_k_stats_over_padding),
}


def test_unmutated_oracle_passes_the_checks(golden_dir):
    assert not _caught(golden_dir)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(monkeypatch, golden_dir, name):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(ref, attr, fn)
    if name == "msb_first_packing":
        monkeypatch.setattr(ref, "unpack_words", _unpack_msb_first)
    assert _caught(golden_dir), f"planted mistake {name!r} went unnoticed"
