"""Pins of the per-layer bit-mix oracle (oracle/layer_mix_ref.py).

* hand cases of the boundary rule (vLLM turboquant/config.py,
  get_boundary_skip_layers): first n and last n layers, n capped at half
  the layer count, overlapping sets merged, nothing for n <= 0 or no layers;
* brute force over small models: a layer is protected exactly when fewer
  than min(n, L // 2) layers lie before it or after it;
* the mixed encode of a model equals, layer by layer, the single-config
  codec at that layer's bits, and each layer's payload has the size of its
  own bit width (so a dropped mix would be seen);
* planted mistakes (no cap, cap at L instead of L // 2, last set off by
  one, protection for n = 0) are caught.
"""

import numpy as np
import pytest

from oracle import kivi_ref as ref
from oracle import layer_mix_ref as mix

HAND = [
    (32, 2, [0, 1, 30, 31]),      # a dense 32-layer model, the page's n = 2
    (28, 2, [0, 1, 26, 27]),
    (5, 3, [0, 1, 3, 4]),         # n capped at 5 // 2 = 2: the middle layer stays base
    (4, 2, [0, 1, 2, 3]),         # 2n = L: every layer protected
    (3, 2, [0, 2]),               # cap 1
    (2, 5, [0, 1]),
    (1, 2, []),                   # cap 0
    (8, 0, []),
    (8, -1, []),
    (0, 2, []),
    (6, 1, [0, 5]),
]


@pytest.mark.parametrize("L,n,want", HAND)
def test_hand_cases(L, n, want):
    assert mix.boundary_layers(L, n) == want


def test_brute_force_small_models():
    for L in range(0, 13):
        for n in range(-1, 9):
            m = min(max(n, 0), L // 2)
            want = [l for l in range(L) if l < m or L - 1 - l < m]
            assert mix.boundary_layers(L, n) == want, (L, n)


def test_layer_bits():
    bits = mix.layer_bits(6, 1, (2, 2), (8, 4))
    assert bits == [(8, 4), (2, 2), (2, 2), (2, 2), (2, 2), (8, 4)]


def test_mixed_encode_is_per_layer_codec():
    rng = np.random.default_rng(5)
    L, S, T, D, G = 4, 2, 70, 64, 32
    x = rng.standard_normal((L, S, T, D)).astype(np.float16)
    bits = mix.layer_bits(L, 1, (2, 2), (8, 4))
    for keys in (True, False):
        pays = mix.encode_layers(x, 65, bits, G, keys)
        outs = mix.decode_layers(pays, 65, bits, G, D, keys)
        for l in range(L):
            b = bits[l][0 if keys else 1]
            enc = ref.encode_k if keys else ref.encode_v
            want = enc(x[l], 65, b, G)
            assert all(np.array_equal(a, w) for a, w in zip(pays[l], want))
            words = ref.k_code_words(65, D, b, G) if keys else ref.v_code_words(65, D, b, G)
            assert pays[l][0].size == S * words        # the layer's own bit width
            err = np.abs(outs[l].astype(np.float64) - x[l, :, :65].astype(np.float64)).max()
            # a b-bit code is within half a step of the group's range
            assert err <= (np.abs(x[l]).max() * 2) / (2 ** b - 1) / 2 * 1.01 + 2 ** -10


# planted mistakes -----------------------------------------------------------

def _no_cap(L, n):
    if n <= 0 or L <= 0:
        return []
    return sorted(set(range(min(n, L))) | set(range(max(L - n, 0), L)))


def _cap_at_l(L, n):
    if n <= 0 or L <= 0:
        return []
    n = min(n, L)
    return sorted(set(range(n)) | set(range(L - n, L)))


def _last_off_by_one(L, n):
    if n <= 0 or L <= 0:
        return []
    n = min(n, L // 2)
    return sorted(set(range(n)) | set(range(L - n - 1, L - 1)))


def _zero_protects_one(L, n):
    if L <= 0 or n < 0:
        return []
    n = max(min(n, L // 2), 1 if L > 1 else 0)
    return sorted(set(range(n)) | set(range(L - n, L)))


def _caught():
    try:
        for L, n, want in HAND:
            test_hand_cases(L, n, want)
        test_brute_force_small_models()
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("mutant", [_no_cap, _cap_at_l, _last_off_by_one, _zero_protects_one])
def test_planted_mistake_is_caught(monkeypatch, mutant):
    assert not _caught()
    monkeypatch.setattr(mix, "boundary_layers", mutant)
    assert _caught()
