"""The seeded input generators produce the structure their docstrings promise."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from kvsynth import WORKLOADS, layer_kv, stream_tokens, uniform_with_ties
from oracle import kivi_ref as ref

F16 = np.float16


@pytest.mark.parametrize("b", [2, 4, 8])
@pytest.mark.parametrize("axis", ["token", "channel"])
def test_tie_groups_give_about_one_percent_exact_ties(b, axis):
    S, T, D, G, n = 4, 1000, 96, 32, 1000 - 128
    x = uniform_with_ties(S, T, D, axis=axis, n_valid=n, bits=b, group_size=G, seed=b)
    assert x.dtype == F16 and np.all(np.abs(x.astype(np.float32)) <= 8)
    if axis == "token":
        _, sc, zr = ref.encode_k(x, n, b, G)
        s = sc[:, np.arange(n) // G, :].astype(np.float64)
        z = zr[:, np.arange(n) // G, :].astype(np.float64)
        xs = x[:, :n, :].astype(np.float64)
    else:
        _, sc, zr = ref.encode_v(x, n, b, G)
        s = sc[:, :, np.arange(D) // G].astype(np.float64)
        z = zr[:, :, np.arange(D) // G].astype(np.float64)
        xs = x[:, :n, :].astype(np.float64)
    ok = s > 0
    quot = np.where(ok, (xs - z) / np.where(ok, s, 1), 0)   # exact in float64 here
    ties = ok & (np.abs(quot - np.floor(quot) - 0.5) == 0)
    frac = ties.mean()
    assert 0.005 < frac < 0.03, frac
    # spot-check exactness of a few ties with rationals
    for idx in list(zip(*np.nonzero(ties)))[:20]:
        q = (Fraction(float(xs[idx])) - Fraction(float(z[idx]))) / Fraction(float(s[idx]))
        assert q.denominator == 2


def test_generators_are_deterministic_and_shaped():
    w = WORKLOADS["single_layer_4bit"]
    k1, v1 = layer_kv(w, 0)
    k2, v2 = layer_kv(w, 0)
    assert k1.shape == (8, 512, 128) and k1.dtype == torch.float16
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    assert not torch.equal(k1, v1)
    # 4 outlier key channels per head, scaled x20
    amp = k1.float().abs().mean(dim=1)                # [8 heads, 128]
    assert all(int((amp[h] > 5).sum()) == 4 for h in range(8))
    ks, vs = stream_tokens(WORKLOADS["stream_b64"], 2)
    assert ks.shape == (2, 16384, 128)


def test_mistral_shape_is_heavy_tailed_with_key_bias():
    w = WORKLOADS["mistral_7b_k2v4"]
    k, v = layer_kv(w, 3, tokens=256)
    assert k.shape == (w.batch * w.heads, 256, 128)
    vf = v.float()
    kurt = ((vf - vf.mean()) ** 4).mean() / vf.var() ** 2
    assert kurt > 4.5                                # Gaussian: 3
    per_chan_mean = k.float().mean(dim=1)            # [slices, D]
    assert per_chan_mean.abs().mean() > 1.0          # bias ~ N(0, 3)
