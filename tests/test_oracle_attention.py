"""Pins of the decode-attention oracle (oracle/attention_ref.py) to facts
outside itself, and the planted mistakes they must catch.

* the exact dequantization equals ``code * scale + zero`` in rational
  arithmetic (codes unpacked by the independent exact tier), and rounds to
  the codec's own fp16 decode;
* the attention equals torch's float64 ``scaled_dot_product_attention`` (a
  library routine the oracle does not call) on the same tokens;
* closed forms: a query that singles out one token returns that token's
  value; a zero query returns the mean of all cached values;
* invariants: grouped query heads are independent queries of one KV head;
  the residual ring's start slot does not change the result.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import attention_ref as att
from oracle import kivi_exact as ex
from oracle import kivi_ref as ref

F16 = np.float16


def _cache(seed, S=2, n_quant=70, n_res=9, D=64, kb=2, vb=4, G=32, scale=1.0):
    """Encode random fp16 K/V for ``S`` slices; return payloads and residual."""
    rng = np.random.default_rng(seed)
    T = n_quant + n_res
    k = (rng.standard_normal((S, T, D)) * scale).astype(F16)
    v = (rng.standard_normal((S, T, D)) * scale).astype(F16)
    kp = ref.encode_k(k, n_quant, kb, G)
    vp = ref.encode_v(v, n_quant, vb, G)
    return k, v, kp, vp, k[:, n_quant:], v[:, n_quant:]


def _sdpa(q, k, v, sm_scale):
    """torch float64 SDPA: q [S, r, D], k/v [S, T, D] shared by the r heads."""
    S, r, D = q.shape
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64)).reshape(S, r, 1, D)
    kt = torch.from_numpy(np.asarray(k, dtype=np.float64))[:, None].expand(S, r, -1, D)
    vt = torch.from_numpy(np.asarray(v, dtype=np.float64))[:, None].expand(S, r, -1, D)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=float(sm_scale))
    return o.reshape(S, r, D).numpy()


# ---------------------------------------------------------------------------
# dequantization
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kb,vb,G", [(2, 4, 32), (4, 2, 64), (8, 8, 128)])
def test_exact_dequant_is_rational_code_times_scale_plus_zero(kb, vb, G):
    S, n, D = 1, G + 5, 64
    _, _, kp, vp, _, _ = _cache(3, S=S, n_quant=n, n_res=0, D=D, kb=kb, vb=vb, G=G, scale=3.0)
    kd = att.dequantize_exact_k(*kp, n, kb, G)
    vd = att.dequantize_exact_v(*vp, n, vb, G, D)
    kw = kp[0].view(np.uint32)[0]                  # [ng*W, D]
    ks, kz = kp[1].view(np.uint16)[0], kp[2].view(np.uint16)[0]
    for d in range(0, D, 7):
        codes = ex.unpack([int(x) for x in kw[:, d]], kb)       # along tokens
        for t in range(n):
            want = Fraction(codes[t]) * ex.f16_value(int(ks[t // G, d])) + ex.f16_value(int(kz[t // G, d]))
            assert kd[0, t, d] == float(want), (d, t)
    vw = vp[0].view(np.uint32)[0]                  # [n, ngv*W]
    vs, vz = vp[1].view(np.uint16)[0], vp[2].view(np.uint16)[0]
    for t in range(0, n, 5):
        codes = ex.unpack([int(x) for x in vw[t]], vb)          # along channels
        for d in range(D):
            want = Fraction(codes[d]) * ex.f16_value(int(vs[t, d // G])) + ex.f16_value(int(vz[t, d // G]))
            assert vd[0, t, d] == float(want), (t, d)


def test_exact_dequant_rounds_to_the_codec_decode():
    _, _, kp, vp, _, _ = _cache(5, S=3, n_quant=100, n_res=0, D=128, kb=2, vb=2, G=32)
    kd = att.dequantize_exact_k(*kp, 100, 2, 32)
    vd = att.dequantize_exact_v(*vp, 100, 2, 32, 128)
    kdec = ref.decode_k(*kp, 100, 2, 32)
    vdec = ref.decode_v(*vp, 100, 2, 32, 128)
    assert np.array_equal(kd.astype(np.float32).astype(F16).view(np.uint16), kdec.view(np.uint16))
    assert np.array_equal(vd.astype(np.float32).astype(F16).view(np.uint16), vdec.view(np.uint16))


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("r", [1, 4])
def test_residual_only_matches_torch_sdpa(r):
    rng = np.random.default_rng(11)
    S, T, D = 3, 37, 64
    q = rng.standard_normal((S, r, D)).astype(F16)
    k = rng.standard_normal((S, T, D)).astype(F16)
    v = rng.standard_normal((S, T, D)).astype(F16)
    got = att.decode_attention(q, None, None, 0, k, v, 2, 2, 32, 0.125)
    assert np.allclose(got, _sdpa(q, k, v, 0.125), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("kb,vb,G,n_quant,n_res", [(2, 2, 32, 96, 16), (2, 4, 32, 70, 9),
                                                   (4, 8, 64, 130, 0), (8, 2, 128, 129, 1)])
def test_quantized_cache_matches_torch_sdpa_over_dequantized_tokens(kb, vb, G, n_quant, n_res):
    D = 64
    _, _, kp, vp, rk, rv = _cache(7, n_quant=n_quant, n_res=n_res, D=D, kb=kb, vb=vb, G=G)
    q = np.random.default_rng(8).standard_normal((2, 2, D)).astype(F16)
    got = att.decode_attention(q, kp, vp, n_quant, rk, rv, kb, vb, G, D ** -0.5)
    kd = att.dequantize_exact_k(*kp, n_quant, kb, G)
    vd = att.dequantize_exact_v(*vp, n_quant, vb, G, D)
    kk = np.concatenate([kd, rk.astype(np.float64)], axis=1)
    vv = np.concatenate([vd, rv.astype(np.float64)], axis=1)
    assert kk.shape[1] == n_quant + n_res
    assert np.allclose(got, _sdpa(q, kk, vv, D ** -0.5), rtol=1e-13, atol=1e-13)


def _one_hot_case(t_star, n_quant=96, n_res=20, D=64, G=32):
    """Cache where token t_star has key channel 0 = 30 and every other key
    element lies in [-1, 1]; q = 4 e_0 gives it a logit lead above 100."""
    rng = np.random.default_rng(21)
    S, T = 2, n_quant + n_res
    k = rng.uniform(-1, 1, (S, T, D)).astype(F16)
    v = rng.standard_normal((S, T, D)).astype(F16)
    k[:, t_star, 0] = 30.0
    kp = ref.encode_k(k, n_quant, 2, G)
    vp = ref.encode_v(v, n_quant, 2, G)
    q = np.zeros((S, 1, D), dtype=F16)
    q[:, :, 0] = 4.0
    out = att.decode_attention(q, kp, vp, n_quant, k[:, n_quant:], v[:, n_quant:], 2, 2, G, 1.0)
    if t_star < n_quant:          # the token's value, dequantized (pinned above)
        want = att.dequantize_exact_v(*vp, n_quant, 2, G, D)[:, t_star]
    else:                         # a residual token: its fp16 value
        want = v[:, t_star].astype(np.float64)
    return out, want


@pytest.mark.parametrize("t_star", [0, 31, 32, 95, 96, 115])
def test_one_hot_query_returns_that_tokens_value(t_star):
    out, want = _one_hot_case(t_star)
    assert np.allclose(out[:, 0], want, rtol=0, atol=1e-30)


def test_zero_query_returns_the_mean_of_all_cached_values():
    D = 64
    _, _, kp, vp, rk, rv = _cache(9, n_quant=70, n_res=9, D=D)
    q = np.zeros((2, 3, D), dtype=F16)
    out = att.decode_attention(q, kp, vp, 70, rk, rv, 2, 4, 32, 0.3)
    vd = att.dequantize_exact_v(*vp, 70, 4, 32, D)
    mean = (vd.sum(axis=1) + rv.astype(np.float64).sum(axis=1)) / (70 + 9)
    assert np.allclose(out, mean[:, None, :], rtol=1e-14, atol=1e-14)


def test_grouped_query_heads_are_independent_queries():
    D = 64
    _, _, kp, vp, rk, rv = _cache(13, n_quant=64, n_res=5, D=D)
    q = np.random.default_rng(14).standard_normal((2, 4, D)).astype(F16)
    both = att.decode_attention(q, kp, vp, 64, rk, rv, 2, 4, 32, 0.2)
    for h in range(4):
        one = att.decode_attention(q[:, h:h + 1], kp, vp, 64, rk, rv, 2, 4, 32, 0.2)
        assert np.array_equal(both[:, h:h + 1], one)


def test_ring_start_slot_does_not_change_the_result():
    rng = np.random.default_rng(17)
    S, slots, count, D = 2, 12, 7, 64
    toks_k = rng.standard_normal((S, count, D)).astype(F16)
    toks_v = rng.standard_normal((S, count, D)).astype(F16)
    q = rng.standard_normal((S, 2, D)).astype(F16)
    want = att.decode_attention(q, None, None, 0, toks_k, toks_v, 2, 2, 32, 0.5)
    for head in (0, 5, 11):
        ring_k = (rng.standard_normal((S, slots, D)) * 50).astype(F16)   # stale slots
        ring_v = (rng.standard_normal((S, slots, D)) * 50).astype(F16)
        idx = (head + np.arange(count)) % slots
        ring_k[:, idx] = toks_k
        ring_v[:, idx] = toks_v
        rk = att.ring_tokens(ring_k, head, count)
        rv = att.ring_tokens(ring_v, head, count)
        got = att.decode_attention(q, None, None, 0, rk, rv, 2, 2, 32, 0.5)
        assert np.allclose(got, want, rtol=1e-14, atol=1e-14)


def test_empty_cache_is_rejected():
    q = np.zeros((1, 1, 64), dtype=F16)
    empty = np.zeros((1, 0, 64), dtype=F16)
    with pytest.raises(ValueError):
        att.decode_attention(q, None, None, 0, empty, empty, 2, 2, 32, 1.0)


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------

def _checks():
    return [
        lambda: [test_exact_dequant_is_rational_code_times_scale_plus_zero(*c)
                 for c in [(2, 4, 32), (4, 2, 64)]],
        lambda: test_exact_dequant_rounds_to_the_codec_decode(),
        lambda: [test_residual_only_matches_torch_sdpa(r) for r in (1, 4)],
        lambda: [test_one_hot_query_returns_that_tokens_value(t) for t in (0, 32, 96, 115)],
        lambda: test_zero_query_returns_the_mean_of_all_cached_values(),
        lambda: test_ring_start_slot_does_not_change_the_result(),
    ]


def _caught():
    for chk in _checks():
        try:
            chk()
        except Exception:         # a failed assertion or a crash both expose it
            return True
    return False


def _no_zero_k(codes, scale, zero, n, bits, G):
    w = np.asarray(codes).view(np.uint32)
    q = np.moveaxis(ref.unpack_words(np.moveaxis(w, 1, 2), bits), 2, 1)[:, :n].astype(np.float64)
    return q * np.asarray(scale)[:, np.arange(n) // G].astype(np.float64)


def _fp16_rounded_v(codes, scale, zero, n, bits, G, D):
    return ref.decode_v(codes, scale, zero, n, bits, G, D).astype(np.float64)


def _ring_from_slot_zero(ring, head, count):
    return np.asarray(ring)[:, :count, :]


def _drop_residual(k_payload, v_payload, n_quant, res_k, res_v, *rest, _orig=att.cache_tokens):
    if n_quant == 0:
        return _orig(k_payload, v_payload, n_quant, res_k, res_v, *rest)
    return _orig(k_payload, v_payload, n_quant, None, None, *rest)


def _unscaled_logits(q, k, v, sm_scale, _orig=att.softmax_attention):
    return _orig(q, k, v, 1.0)


def _value_row_group_by_token(codes, scale, zero, n, bits, G, D):
    w = np.asarray(codes).view(np.uint32)[:, :n, :]
    q = ref.unpack_words(w, bits)[:, :, :D].astype(np.float64)
    grp = np.minimum(np.arange(n) // G, np.asarray(scale).shape[2] - 1)   # wrong axis
    s = np.asarray(scale)[:, :n, :][:, :, grp[:1]].astype(np.float64)
    z = np.asarray(zero)[:, :n, :][:, :, grp[:1]].astype(np.float64)
    return q * s + z


@pytest.mark.parametrize("target,mutant", [
    ("dequantize_exact_k", _no_zero_k),
    ("dequantize_exact_v", _fp16_rounded_v),
    ("dequantize_exact_v", _value_row_group_by_token),
    ("ring_tokens", _ring_from_slot_zero),
    ("cache_tokens", _drop_residual),
    ("softmax_attention", _unscaled_logits),
])
def test_planted_mistake_is_caught(monkeypatch, target, mutant):
    assert not _caught(), "the unmodified oracle must pass every pin"
    monkeypatch.setattr(att, target, mutant)
    assert _caught(), f"mutation of {target} went unnoticed"
