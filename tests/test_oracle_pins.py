"""Pins of the CPU oracle to facts outside itself.

Each test checks the oracle against something it does not compute: numbers
worked by hand (tests/golden), statements printed on the pages, closed
forms, invariants of min/max affine quantization, brute force in exact
rational arithmetic, and the independent exact-rational tier.  A plausible
slip in the oracle (dropped clamp, wrong rounding mode, transposed packing,
stats taken over padding, swapped scale/zero) fails at least one of them.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import kivi_exact as ex
from oracle import kivi_ref as ref

F16, F32 = np.float16, np.float32


def _bits16(a):
    return np.asarray(a, dtype=F16).view(np.uint16)


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _hex(s):
    return int(s, 16)


# ---------------------------------------------------------------------------
# hand-worked groups
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def hand(golden_dir):
    return {c["name"]: c for c in _load(golden_dir, "hand_worked_groups.json")["cases"]}


@pytest.mark.parametrize("name", ["A_values_b4", "B_ties_to_even_b2",
                                  "C_representable_grid_b2", "E_constant_group_b4"])
def test_hand_worked_value_groups(hand, name):
    c = hand[name]
    b, G = c["bits"], c["group_size"]
    v = np.array(c["x"], dtype=F16).reshape(1, 1, G)
    codes, scale, zero = ref.encode_v(v, 1, b, G)
    assert [int(s) for s in _bits16(scale).ravel()] == [_hex(s) for s in c["scale_bits"]]
    assert [int(z) for z in _bits16(zero).ravel()] == [_hex(z) for z in c["zero_bits"]]
    words = codes.view(np.uint32).ravel().tolist()
    assert words == [_hex(w) for w in c["words"]]
    assert ref.unpack_words(codes.view(np.uint32), b).ravel().tolist() == c["codes"]
    dec = ref.decode_v(codes, scale, zero, 1, b, G, G).astype(np.float64).ravel()
    if "decoded_first8" in c:
        assert dec[:8].tolist() == c["decoded_first8"]
    if "max_abs_error" in c:
        err = np.max(np.abs(dec - np.array(c["x"], dtype=np.float64)))
        assert err == c["max_abs_error"]
        assert err <= float(scale.ravel()[0]) / 2


def test_hand_worked_ties_discriminate_rounding(hand):
    c = hand["B_ties_to_even_b2"]
    v = np.array(c["x"], dtype=F16).reshape(1, 1, 32)
    codes, _, _ = ref.encode_v(v, 1, 2, 32)
    assert int(codes.view(np.uint32)[0, 0, 0]) != _hex(c["half_up_word0"])


def test_hand_worked_padded_key_group(hand):
    c = hand["D_padded_key_group_b2"]
    n, G, b = c["n_tokens"], c["group_size"], c["bits"]
    rng = np.random.default_rng(5)
    k = np.zeros((1, 64, 1), dtype=F16)
    k[0, :32, 0] = rng.uniform(-5, 5, 32).astype(F16)
    k[0, 32:40, 0] = np.array(c["x_tokens_32_to_39"], dtype=F16)
    k[0, 40:, 0] = F16(-100.0)        # beyond n_tokens: must not enter the stats
    codes, scale, zero = ref.encode_k(k, n, b, G)
    assert codes.shape == (1, 4, 1) and scale.shape == (1, 2, 1)
    assert int(_bits16(scale)[0, 1, 0]) == _hex(c["scale_bits"][0])
    assert int(_bits16(zero)[0, 1, 0]) == _hex(c["zero_bits"][0])
    assert codes.view(np.uint32)[0, 2:4, 0].tolist() == [_hex(w) for w in c["words"]]
    dec = ref.decode_k(codes, scale, zero, n, b, G)
    assert dec.shape == (1, 40, 1)
    assert dec[0, 32:40, 0].astype(float).tolist() == c["x_tokens_32_to_39"]


# ---------------------------------------------------------------------------
# facts printed on the pages
# ---------------------------------------------------------------------------

def test_page_defaults_and_levels(golden_dir):
    facts = _load(golden_dir, "page_facts.json")
    d = facts["defaults"]
    assert d["k_bits"] in ref.VALID_BITS and d["v_bits"] in ref.VALID_BITS
    assert d["group_size"] in ref.VALID_GROUPS
    # b bits give 2**b levels: the largest code of a group is 2**b - 1, reached at its max
    for b in ref.VALID_BITS:
        x = np.linspace(-3, 5, 32).astype(F16).reshape(1, 1, 32)
        codes, _, _ = ref.encode_v(x, 1, b, 32)
        q = ref.unpack_words(codes.view(np.uint32), b).ravel()
        assert q.min() == 0 and q.max() == 2 ** b - 1
        assert len(set(q.tolist())) <= 2 ** b
    assert facts["levels"]["bits_to_levels"] == {"3": 2 ** 3, "4": 2 ** 4}


@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("b", [2, 4, 8])
def test_value_bytes_match_page_closed_form(golden_dir, D, b):
    """vLLM ``value_packed_size``: ceil(D*b/8) + 4 bytes per value vector.
    Our value path with one group spanning the head (G = D) stores exactly
    that per token-head."""
    facts = _load(golden_dir, "page_facts.json")["value_packed_size"]
    if D not in ref.VALID_GROUPS:
        pytest.skip("G = D needs D to be a supported group size")
    per_token = 4 * ref.v_code_words(1, D, b, D) + 2 * 2 * ref.v_stat_elems(1, D, D)
    assert per_token == math.ceil(D * b / 8) + facts["extra_bytes"]
    v = np.random.default_rng(0).standard_normal((1, 3, D)).astype(F16)
    c, s, z = ref.encode_v(v, 3, b, D)
    assert c.nbytes + s.nbytes + z.nbytes == 3 * per_token


def test_size_closed_forms_at_workload_shapes():
    # Llama-2-7B shape: S = 32*8*32 slices, 4096 - 128 quantized tokens, D 128, 2-bit, G 32
    S, Tq, D, G = 8192, 3968, 128, 32
    assert S * 4 * ref.k_code_words(Tq, D, 2, G) == 1_040_187_392
    assert S * 2 * ref.k_stat_elems(Tq, D, G) == 520_093_696 // 2
    assert S * 4 * ref.v_code_words(Tq, D, 2, G) == 1_040_187_392
    # Mistral-7B shape, 4-bit values
    S, Tq = 4096, 16256
    assert S * 4 * ref.v_code_words(Tq, D, 4, G) == 4_261_412_864
    # partial groups are padded: 1000 tokens at G 32 -> 32 groups
    assert ref.n_groups(1000, 32) == 32 and ref.n_groups(3077, 128) == 25
    assert ref.n_groups(96, 64) == 2 and ref.n_groups(64, 128) == 1
    assert ref.quantized_tokens(512, 128) == 384 and ref.quantized_tokens(100, 128) == 0


# ---------------------------------------------------------------------------
# the exact-rational tier agrees with the numpy tier
# ---------------------------------------------------------------------------

def _random_fp16(rng, shape, mode):
    if mode == "normal":
        return rng.standard_normal(shape).astype(F16)
    if mode == "bits":     # any finite fp16 (incl. subnormals, +-0, huge)
        b = rng.integers(0, 0x10000, size=shape, dtype=np.uint32).astype(np.uint16)
        b = np.where((b & 0x7C00) == 0x7C00, b & 0x83FF, b).astype(np.uint16)
        return b.view(F16)
    if mode == "tiny":     # subnormal-scale groups
        return (rng.integers(-6, 7, size=shape) * 2.0 ** -24).astype(F16)
    if mode == "coarse":   # many exact ties and repeats
        return (rng.integers(-8, 9, size=shape) * 0.5).astype(F16)
    raise ValueError(mode)


def _to_lists(a16):
    return a16.view(np.uint16).astype(int).tolist()


@pytest.mark.parametrize("mode", ["normal", "bits", "tiny", "coarse"])
@pytest.mark.parametrize("b", [2, 4, 8])
@pytest.mark.parametrize("G", [32, 64])
def test_exact_tier_matches_numpy_tier(mode, b, G):
    rng = np.random.default_rng(hash((mode, b, G)) % 2 ** 32)
    S, T, D = 1, G + 5, 12 if G == 32 else 8
    x = _random_fp16(rng, (S, T, D), mode)
    n = T - 2
    # keys
    kc, ks, kz = ref.encode_k(x, n, b, G)
    ec, es, ez = ex.encode_k(_to_lists(x), n, b, G)
    assert kc.view(np.uint32).tolist() == ec
    assert _to_lists(ks) == es and _to_lists(kz) == ez
    kd = ref.decode_k(kc, ks, kz, n, b, G)
    assert _to_lists(kd) == ex.decode_k(ec, es, ez, n, b, G)
    # values (D < G: one padded group per token)
    vc, vs, vz = ref.encode_v(x, n, b, G)
    fc, fs, fz = ex.encode_v(_to_lists(x), n, b, G)
    assert vc.view(np.uint32).tolist() == fc
    assert _to_lists(vs) == fs and _to_lists(vz) == fz
    vd = ref.decode_v(vc, vs, vz, n, b, G, D)
    assert _to_lists(vd) == ex.decode_v(fc, fs, fz, n, b, G, D)


def test_exact_rounding_primitives():
    # round_binary against hand facts of the formats
    assert ex.f16(Fraction(1, 5)) == Fraction(1638, 8192)
    assert ex.f16_bits(ex.f16(Fraction(1, 5))) == 0x3266
    assert ex.f32(Fraction(1, 5)) == Fraction(13421773, 2 ** 26)
    assert ex.f16(Fraction(3, 2 ** 26)) == Fraction(1, 2 ** 24)      # 0.75 ulp -> 1 ulp
    assert ex.f16(Fraction(1, 2 ** 25)) == 0                          # half ulp, tie -> even 0
    assert ex.f16(Fraction(3, 2 ** 25)) == Fraction(2, 2 ** 24)       # 1.5 ulp -> 2 (even)
    assert ex.f16_bits(Fraction(65504)) == 0x7BFF
    with pytest.raises(ex.Overflow):
        ex.f16(Fraction(65520))
    assert ex.f16(Fraction(65519)) == 65504
    for b in (0x0001, 0x03FF, 0x0400, 0x3C00, 0xC000, 0x7BFF, 0x8001):
        assert ex.f16_bits(ex.f16_value(b)) == b
    assert ex.round_half_even(Fraction(5, 2)) == 2 and ex.round_half_even(Fraction(7, 2)) == 4


# ---------------------------------------------------------------------------
# nearest level by brute force
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("b", [2, 4, 8])
def test_codes_are_nearest_levels(b):
    rng = np.random.default_rng(100 + b)
    G = 32
    for trial in range(6):
        mode = ["normal", "coarse", "normal", "bits", "coarse", "normal"][trial]
        x = _random_fp16(rng, (1, 1, G), mode)
        codes, scale, zero = ref.encode_v(x, 1, b, G)
        q = ref.unpack_words(codes.view(np.uint32), b).ravel()
        sb, zb = int(_bits16(scale).ravel()[0]), int(_bits16(zero).ravel()[0])
        s = ex.f16_value(sb)
        for i, xb in enumerate(_bits16(x).ravel().tolist()):
            best = ex.nearest_level(xb, sb, zb, b)
            if s == 0:
                assert q[i] == 0
                continue
            exact_quot = (ex.f16_value(xb) - ex.f16_value(zb)) / s
            if exact_quot > 2 ** b - 1:
                assert q[i] == 2 ** b - 1
                continue
            if len(best) == 2:                       # exact tie: even code
                assert q[i] == [c for c in best if c % 2 == 0][0]
            elif q[i] != best[0]:
                # only a near-tie may go the other way, through the two fp32 roundings
                k = math.floor(exact_quot)
                assert abs(exact_quot - (k + Fraction(1, 2))) <= Fraction(1, 2 ** 22) * exact_quot


def test_rounding_is_half_even_not_half_up_or_truncation():
    # a quotient of exactly 1.5 -> 2, 2.5 -> 2, 0.5 -> 0; truncation would give 1, 2, 0
    x = np.array([0.0, 1.5, 2.5, 0.5, 3.0, 1.4, 1.6, 2.6] + [0.0] * 24, dtype=F16).reshape(1, 1, 32)
    c, s, z = ref.encode_v(x, 1, 2, 32)
    assert float(s.ravel()[0]) == 1.0
    q = ref.unpack_words(c.view(np.uint32), 2).ravel()[:8].tolist()
    assert q == [0, 2, 2, 0, 3, 1, 2, 3]


# ---------------------------------------------------------------------------
# invariants of min/max affine quantization
# ---------------------------------------------------------------------------

def _ulp16(a):
    a = np.abs(np.asarray(a, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


@pytest.mark.parametrize("b", [2, 4, 8])
@pytest.mark.parametrize("kind", ["k", "v"])
def test_error_bound(b, kind):
    rng = np.random.default_rng(7 * b)
    x = (rng.standard_normal((3, 70, 64)) * rng.choice([0.25, 1, 30], size=(3, 1, 64))).astype(F16)
    n, G = 70, 32
    if kind == "k":
        c, s, z = ref.encode_k(x, n, b, G)
        xh = ref.decode_k(c, s, z, n, b, G)
        sc = s[:, np.arange(n) // G, :]
    else:
        c, s, z = ref.encode_v(x, n, b, G)
        xh = ref.decode_v(c, s, z, n, b, G, 64)
        sc = s[:, :, np.arange(64) // G]
    sc = sc.astype(np.float64)
    assert np.all(sc >= 2.0 ** -14), "test needs normal fp16 scales"
    xd, xhd = x.astype(np.float64), xh.astype(np.float64)
    bound = sc / 2 + _ulp16(np.maximum(np.abs(xd), np.abs(xhd))) + sc * 2.0 ** -14
    assert np.all(np.abs(xd - xhd) <= bound)


def test_min_maps_to_zero_code_and_max_to_top_code():
    rng = np.random.default_rng(3)
    for b in (2, 4, 8):
        x = rng.standard_normal((2, 40, 16)).astype(F16)
        c, s, z = ref.encode_v(x, 40, b, 32)
        q = ref.unpack_words(c.view(np.uint32), b)[:, :, :16]
        xs = x.astype(np.float32)
        assert np.all(q[xs == xs.min(axis=-1, keepdims=True)] == 0)
        assert np.all(q[xs == xs.max(axis=-1, keepdims=True)] == 2 ** b - 1)
        assert np.array_equal(z, xs.min(axis=-1, keepdims=True).astype(F16))


@pytest.mark.parametrize("b", [2, 4, 8])
def test_round_trip_of_representable_values(b):
    rng = np.random.default_rng(11)
    G, L = 32, 2 ** b - 1
    for k_exp in (-6, -2, 0, 3):
        step = 2.0 ** k_exp
        base = step * int(rng.integers(-50, 50))
        q = rng.integers(0, L + 1, size=G)
        q[:2] = [0, L]
        x = (base + q * step).astype(F16)
        assert np.array_equal(x.astype(np.float64), base + q * step), "inputs must be exact"
        c, s, z = ref.encode_v(x.reshape(1, 1, G), 1, b, G)
        assert float(s.ravel()[0]) == step and float(z.ravel()[0]) == base
        xh = ref.decode_v(c, s, z, 1, b, G, G).ravel()
        assert np.array_equal(xh.view(np.uint16), x.view(np.uint16))


def test_scale_covariance_under_powers_of_two():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((2, 33, 32)).astype(F16)
    for b in (2, 4, 8):
        c0, s0, z0 = ref.encode_k(x, 33, b, 32)
        for k in (-3, 2, 5):
            xs = (x.astype(np.float64) * 2.0 ** k).astype(F16)
            assert np.array_equal(xs.astype(np.float64), x.astype(np.float64) * 2.0 ** k)
            c1, s1, z1 = ref.encode_k(xs, 33, b, 32)
            assert np.array_equal(c1, c0)
            assert np.array_equal(s1.astype(np.float64), s0.astype(np.float64) * 2.0 ** k)
            assert np.array_equal(z1.astype(np.float64), z0.astype(np.float64) * 2.0 ** k)


def test_permutation_within_group():
    rng = np.random.default_rng(17)
    x = rng.standard_normal((1, 1, 64)).astype(F16)
    perm = np.concatenate([rng.permutation(32), 32 + rng.permutation(32)])
    for b in (2, 4, 8):
        c0, s0, z0 = ref.encode_v(x, 1, b, 32)
        c1, s1, z1 = ref.encode_v(x[:, :, perm], 1, b, 32)
        assert np.array_equal(s0, s1) and np.array_equal(z0, z1)
        q0 = ref.unpack_words(c0.view(np.uint32), b).ravel()
        q1 = ref.unpack_words(c1.view(np.uint32), b).ravel()
        assert np.array_equal(q0[perm], q1)


def test_signed_zero_is_canonical():
    base = [0.5, 1.0, 0.25] + [0.75] * 29
    for zeros in ([-0.0, 0.0], [0.0, -0.0], [-0.0, -0.0]):
        x = np.array(zeros + base[:30], dtype=F16).reshape(1, 1, 32)
        c, s, z = ref.encode_v(x, 1, 4, 32)
        assert int(_bits16(z).ravel()[0]) == 0x0000
    x = np.full((1, 1, 32), -0.0, dtype=F16)
    c, s, z = ref.encode_v(x, 1, 2, 32)
    assert int(_bits16(s).ravel()[0]) == 0 and int(_bits16(z).ravel()[0]) == 0


def test_subnormal_scale_clamps_codes():
    # group {0, 4 ulp}: 4/3 ulp rounds to a 1-ulp fp16 scale; the max's quotient 4 is clamped to 3
    x = np.zeros((1, 1, 32), dtype=F16)
    x[0, 0, 1] = F16(4 * 2.0 ** -24)
    c, s, z = ref.encode_v(x, 1, 2, 32)
    assert int(_bits16(s).ravel()[0]) == 0x0001
    assert ref.unpack_words(c.view(np.uint32), 2).ravel()[1] == 3
    # a range far below one fp16 ulp per level rounds the scale to zero -> all codes 0
    x[0, 0, 1] = F16(2.0 ** -24)
    c, s, z = ref.encode_v(x, 1, 8, 32)
    assert int(_bits16(s).ravel()[0]) == 0 and not c.any()


# ---------------------------------------------------------------------------
# packing identities
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("b", [2, 4, 8])
def test_packing_positions_exhaustive(b):
    per = 32 // b
    for i in range(per):
        for v in range(2 ** b):
            codes = np.zeros(per, dtype=np.uint32)
            codes[i] = v
            w = ref.pack_words(codes, b)
            assert w.tolist() == [v << (b * i)]
            assert ex.pack(codes.tolist(), b) == [v << (b * i)]


@pytest.mark.parametrize("b", [2, 4, 8])
def test_pack_is_a_bijection(b):
    rng = np.random.default_rng(b)
    words = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    codes = ref.unpack_words(words, b)
    assert codes.max() < 2 ** b
    assert np.array_equal(ref.pack_words(codes, b), words)
    codes2 = rng.integers(0, 2 ** b, size=(5_000, 32 // b)).astype(np.uint32)
    assert np.array_equal(ref.unpack_words(ref.pack_words(codes2, b), b), codes2)
    sample = words[:200].tolist()
    assert ex.pack(ex.unpack(sample, b), b) == sample


def test_key_words_pack_along_tokens_and_value_words_along_channels():
    # a single non-zero element moves exactly one bit-field in the expected word
    G, b = 32, 4
    x = np.zeros((1, 32, 32), dtype=F16)
    x[0, 0, :] = F16(-1.0)           # makes every key group/column range non-zero
    x[0, :, 0] = F16(-1.0)           # and every value group
    x[0, 13, 5] = F16(2.0)
    kc, _, _ = ref.encode_k(x, 32, b, G)
    kq = kc.view(np.uint32)
    # key: channel 5, token 13 -> word 13 // 8 = 1 of the group, field 13 % 8 = 5
    assert (int(kq[0, 1, 5]) >> (4 * 5)) & 15 == 15
    vc, _, _ = ref.encode_v(x, 32, b, G)
    vq = vc.view(np.uint32)
    # value: token 13, channel 5 -> word 5 // 8 = 0 of the row, field 5
    assert (int(vq[0, 13, 0]) >> (4 * 5)) & 15 == 15


# ---------------------------------------------------------------------------
# full cache split and streaming
# ---------------------------------------------------------------------------

def test_streaming_equals_one_shot_encode():
    rng = np.random.default_rng(23)
    S, D, G, R, T0, steps = 3, 16, 32, 40, 100, 150
    k_all = rng.standard_normal((S, T0 + steps, D)).astype(F16)
    v_all = rng.standard_normal((S, T0 + steps, D)).astype(F16)
    st = ref.StreamRef(2, 4, G, R)
    st.prefill(k_all[:, :T0], v_all[:, :T0], T0)
    assert st.n_quant == 32 and st.res_k.shape[1] == T0 - 32   # floor((100-40)/32)*32 = 32
    flush_steps = []
    for i in range(steps):
        if st.append(k_all[:, T0 + i], v_all[:, T0 + i]):
            flush_steps.append(i)
        n_res = st.res_k.shape[1]
        assert n_res <= R, "after every step the residual holds at most R tokens"
        assert st.n_quant + n_res == T0 + i + 1
    # residual after the G-aligned prefill: 68 tokens.  Step 0 makes it 69 > R -> flush to 37;
    # step 4 makes it 41 -> flush to 9; from then on every 32 steps (9 + 32 = 41).
    assert flush_steps == [0, 4, 36, 68, 100, 132]
    nq = st.n_quant
    kc, ks, kz = st.key_arrays()
    k1, s1, z1 = ref.encode_k(k_all, nq, 2, G)
    assert np.array_equal(kc, k1) and np.array_equal(ks, s1) and np.array_equal(kz, z1)
    vc, vs, vz = st.value_arrays()
    v1, t1, u1 = ref.encode_v(v_all, nq, 4, G)
    assert np.array_equal(vc, v1) and np.array_equal(vs, t1) and np.array_equal(vz, u1)
    assert np.array_equal(st.res_k, k_all[:, nq:T0 + steps])


def test_stream_flush_schedule_at_batch64_shape():
    # prefill 2048 with R 128, G 32: 1920 tokens quantized, 128 residual;
    # over 512 steps the flush fires at steps 0, 32, ..., 480 (16 flushes)
    G, R = 32, 128
    count, n_quant, flushes = 2048 - 1920, 1920, []
    for step in range(512):
        count += 1
        if ref.flush_due(count, R, G):
            count -= G
            n_quant += G
            flushes.append(step)
    assert flushes == list(range(0, 512, 32)) and n_quant == 2432 and count == 128


def test_flush_rule_with_short_residual():
    # R = 0: the residual gives away a whole group once it holds G tokens
    assert not ref.flush_due(1, 0, 32) and ref.flush_due(32, 0, 32)
    assert ref.flush_due(129, 128, 32) and not ref.flush_due(128, 128, 32)


# ---------------------------------------------------------------------------
# adversarial roundings (inputs found by scanning the fp16 grid; expected
# results come from the exact-rational tier at test time)
# ---------------------------------------------------------------------------

# (x, scale) with zero = 0 where x/scale is exactly k + 1/2 but x times the
# float32-rounded reciprocal of scale lands just above or below it
TIE_QUOTIENTS = [(0x3E18, 0x3380), (0x40EC, 0x3380), (0x4155, 0x3690), (0x41B0, 0x3700),
                 (0x4578, 0x3700), (0x3CA6, 0x3770), (0x420B, 0x3770), (0x3EB3, 0x37A8),
                 (0x3CEC, 0x37E0), (0x406E, 0x37E0)]

# (max, min, bits) whose float32 range divided by 2**b - 1 rounds, in float32,
# onto an fp16 rounding midpoint: a single rounding to fp16 would differ
RANGE_MIDPOINTS = [(0x3C00, 0x87FF, 2), (0x4800, 0x93FF, 2), (0x5400, 0x9FFF, 2),
                   (0x3C03, 0x81FF, 4), (0x3C02, 0x8601, 4), (0x4403, 0x87FC, 4),
                   (0x3C7B, 0x801F, 8), (0x3C7A, 0x8061, 8), (0x447B, 0x807C, 8)]


@pytest.mark.parametrize("b", [4, 8])
def test_exact_tie_quotients_round_to_even(b):
    for xb, sb in TIE_QUOTIENTS:
        quot = ex.f16_value(xb) / ex.f16_value(sb)
        assert quot.denominator == 2, "input must be an exact tie"
        want = ex.quantize(xb, sb, 0, b)
        assert want % 2 == 0
        got = ref.quantize(np.array([xb], np.uint16).view(F16), np.array([sb], np.uint16).view(F16),
                           np.zeros(1, F16), b)
        assert int(got[0]) == want


def test_scale_is_rounded_twice():
    for mxb, mnb, b in RANGE_MIDPOINTS:
        mx, mn = ex.f16_value(mxb), ex.f16_value(mnb)
        single = ex.f16((mx - mn) / (2 ** b - 1))
        double = ex.f16(ex.f32(ex.f32(mx - mn) / (2 ** b - 1)))
        assert single != double, "input must separate the two readings"
        want = ex.group_params([mnb, mxb], b)
        assert want[0] == ex.f16_bits(double)
        sc, zr = ref.group_params(np.array([mnb, mxb], np.uint16).view(F16), b)
        assert (int(sc.view(np.uint16)), int(zr.view(np.uint16))) == want
