"""The host-side comparison behind the every-slice GPU parity tests
(tests/gpu_util.oracle_check_chunk) reports every kind of planted
difference and nothing on agreement.  Runs on the CPU: the "device" outputs
here are the oracle's own, with one planted change at a time."""

import numpy as np
import pytest

from oracle import kivi_ref as ref

U = pytest.importorskip("tests.gpu_util")


def _device_like(kind, x, n, b, G, D):
    if kind == "k":
        c, s, z = ref.encode_k(x, n, b, G)
        d = ref.decode_k(c, s, z, n, b, G)
    else:
        c, s, z = ref.encode_v(x, n, b, G)
        d = ref.decode_v(c, s, z, n, b, G, D)
    return [c.view(np.uint32).copy(), s.view(np.uint16).copy(), z.view(np.uint16).copy(),
            d.view(np.uint16).copy()]


@pytest.mark.parametrize("kind,b", [("k", 2), ("v", 4), ("k", 8)])
def test_agreement_and_each_planted_difference(kind, b):
    rng = np.random.default_rng(5)
    S, T, D, G, n = 3, 80, 64, 32, 70
    x = rng.standard_normal((S, T, D)).astype(np.float16)
    good = _device_like(kind, x, n, b, G, D)
    assert U.oracle_check_chunk(kind, x, *good, n, b, G, D) == []
    side = "key" if kind == "k" else "value"
    for i, what in enumerate(("codes", "scale", "zero", "decode")):
        bad = [a.copy() for a in good]
        bad[i].reshape(-1)[bad[i].size // 2] ^= 1          # one bit of one element
        msgs = U.oracle_check_chunk(kind, x, *bad, n, b, G, D, s0=100)
        assert len(msgs) == 1 and msgs[0].startswith(f"{side} {what}: 1 mismatches"), msgs
        first = tuple(np.argwhere(bad[i] != good[i])[0])
        assert f"first at ({first[0] + 100}," in msgs[0]  # slice index shifted by s0


def test_shape_mismatch_is_reported():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 40, 32)).astype(np.float16)
    good = _device_like("v", x, 40, 2, 32, 32)
    good[3] = good[3][:, :39]
    msgs = U.oracle_check_chunk("v", x, *good, 40, 2, 32, 32)
    assert msgs and "shape" in msgs[0]
