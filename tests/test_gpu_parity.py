"""Bit-exact parity of the HIP codec (through the C ABI) with the CPU oracle.

Codes and fp16 scale/zero words must match exactly; decoded fp16 values are
required to match exactly too (a tighter bar than the 1-ulp allowance).
Sizes span several tiles and blocks and always include ragged tails.
"""

import itertools
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from kvsynth import WORKLOADS, layer_kv, uniform_with_ties  # noqa: E402
from tests import gpu_util as U  # noqa: E402
from tests.test_oracle_pins import RANGE_MIDPOINTS, TIE_QUOTIENTS  # noqa: E402

import kv_cache_quantization_codec_amd as K  # noqa: E402

F16 = np.float16


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    K.binding.lib()          # raises if the HIP library is missing


def test_single_layer_4bit_workload():
    w = WORKLOADS["single_layer_4bit"]
    cfg = K.Config(w.k_bits, w.v_bits, w.group_size, w.residual_length, w.head_dim)
    k, v = layer_kv(w, 0)
    n = w.tokens - w.residual_length
    _log(f"single layer: S={k.shape[0]} T={w.tokens} n={n}")
    U.check_round_trip("k", cfg, k.numpy().view(F16), n)
    U.check_round_trip("v", cfg, v.numpy().view(F16), n)


EDGE = list(itertools.product([64, 96, 128], [1000, 3077], [32, 64, 128], [128, 0], [2, 4, 8]))


@pytest.mark.parametrize("D,T,G,R,b", EDGE, ids=[f"D{d}-T{t}-G{g}-R{r}-b{b}" for d, t, g, r, b in EDGE])
def test_edge_shapes_with_exact_ties(D, T, G, R, b):
    seed = hash((D, T, G, R, b)) % 2 ** 31
    n = max(T - R, 0)
    S = 4
    _log(f"edge D={D} T={T} G={G} R={R} b={b} seed={seed}")
    xk = uniform_with_ties(S, T, D, axis="token", n_valid=n, bits=b, group_size=G, seed=seed)
    xv = uniform_with_ties(S, T, D, axis="channel", n_valid=n, bits=b, group_size=G, seed=seed + 1)
    cfg = K.Config(b, b, G, R, D)
    U.check_round_trip("k", cfg, xk, n)
    U.check_round_trip("v", cfg, xv, n)


@pytest.mark.parametrize("b", [2, 8])
def test_xcd_ordered_grids_with_tails(b):
    """Key encode, value encode and value decode hand each XCD runs of
    consecutive work items, except in a tail of workgroups past the last whole
    super-chunk (8 runs), which keeps launch order.  At 23 slices x 3000
    tokens, D = 128, G = 32 the grids have both parts: key encode 23 x 24 =
    552 workgroups (runs of 16: 4 super-chunks of 128, tail 40), value encode
    23 x 47 = 1081 (runs of 128: 1 super-chunk of 1024, tail 57), value
    decode 1081 (runs of 16: 8 super-chunks, tail 57).  Every output is
    compared bit for bit, and nothing outside the valid region is written."""
    S, T, D = 23, 3000, 128
    x = np.random.default_rng(23 + b).standard_normal((S, T, D)).astype(F16)
    cfg = K.Config(b, b, 32, 0, D)
    _log(f"xcd-ordered grids S={S} T={T} b={b}")
    U.check_round_trip("k", cfg, x, T)
    U.check_round_trip("v", cfg, x, T)


@pytest.mark.parametrize("kind", ["k", "v"])
@pytest.mark.parametrize("D,G", [(128, 32), (96, 64), (64, 128), (8, 32), (256, 128), (40, 32), (256, 32), (32, 32)])
def test_strided_input_and_capacity(kind, D, G):
    rng = np.random.default_rng(D + G)
    S, T, n = 5, 300, 211
    x = rng.standard_normal((S, T, D)).astype(F16)
    for b in (2, 4, 8):
        cfg = K.Config(b, b, G, T - n, D)
        _log(f"strided {kind} D={D} G={G} b={b}")
        U.check_round_trip(kind, cfg, x, n, cap=n + 3 * G + 5, extra_tokens=8)


@pytest.mark.parametrize("kind", ["k", "v"])
def test_tiny_counts(kind):
    rng = np.random.default_rng(3)
    for n in (1, 2, 31, 32, 33, 63, 65, 129, 255, 257):
        x = rng.standard_normal((3, n, 64)).astype(F16)
        for b, G in ((2, 32), (4, 64), (8, 128), (4, 32), (8, 32)):
            U.check_round_trip(kind, K.Config(b, b, G, 0, 64), x, n)


def test_zero_tokens_and_zero_slices_write_nothing():
    cfg = K.Config(2, 2, 32, 128, 128)
    x = torch.zeros((2, 64, 128), dtype=torch.float16, device="cuda")
    for kind in ("k", "v"):
        codes, scale, zero = U.gpu_encode(kind, cfg, x, 0, cap=64)
        assert U.is_poison(U.words(codes)) and U.is_poison(U.bits16(scale))
        out = U.gpu_decode(kind, cfg, codes, scale, zero, 0, 64, cap=64)
        assert U.is_poison(U.bits16(out))
    torch.cuda.synchronize()


def _adversarial_rows(D: int) -> np.ndarray:
    """Rows (one value group each, G = D) with hard cases: exact quotient ties
    where a rounded reciprocal misleads, ranges whose fp32 step lands on an fp16
    midpoint, subnormals, signed zeros, constant rows, and the fp16 extremes."""
    rows = []
    for xb, sb in TIE_QUOTIENTS:
        # zero = 0, max = 15*scale (exact) so the 4-bit scale is exactly `scale`
        s = np.array([sb], np.uint16).view(F16)[0]
        r = np.zeros(D, F16)
        r[1] = F16(15 * float(s))
        r[2] = np.array([xb], np.uint16).view(F16)[0]
        if float(r[1]) == 15 * float(s) and float(r[2]) <= float(r[1]):
            rows.append(r)
    for mxb, mnb, _ in RANGE_MIDPOINTS:
        r = np.zeros(D, F16)
        r[::2] = np.array([mnb], np.uint16).view(F16)[0]
        r[1::2] = np.array([mxb], np.uint16).view(F16)[0]
        r[3] = F16(0.5 * float(r[1]))
        rows.append(r)
    rng = np.random.default_rng(9)
    rows.append((rng.integers(-6, 7, D) * 2.0 ** -24).astype(F16))        # subnormal scale
    r = np.zeros(D, F16)
    r[: D // 2] = F16(-0.0)
    rows.append(r)                                                         # +-0 only
    rows.append(np.full(D, F16(1.5)))                                      # constant
    r = np.full(D, F16(-0.0))
    r[5] = F16(2.0 ** -24)
    rows.append(r)
    r = rng.uniform(-1, 1, D).astype(F16)
    r[0], r[1] = F16(-65504.0), F16(65504.0)
    rows.append(r)                                                         # widest range
    bits = rng.integers(0, 0x10000, D, dtype=np.uint32).astype(np.uint16)
    bits = np.where((bits & 0x7C00) == 0x7C00, bits & 0x83FF, bits).astype(np.uint16)
    rows.append(bits.view(F16))                                            # any finite fp16
    return np.stack(rows)


@pytest.mark.parametrize("b", [2, 4, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
def test_adversarial_groups(b, G):
    D = 128
    rows = _adversarial_rows(D)
    T = rows.shape[0]
    # values: each row is a token; keys: the same data transposed so that each
    # row runs along tokens of one channel
    xv = rows[None, :, :].copy()
    tok = max(G, 128)
    xk = np.zeros((1, tok, D), F16)
    m = min(T, D)
    xk[0, :, :m] = np.resize(rows[:m, :].T, (tok, m)).astype(F16)
    cfg = K.Config(b, b, G, 0, D)
    _log(f"adversarial b={b} G={G} rows={T}")
    U.check_round_trip("v", cfg, xv, T)
    U.check_round_trip("k", cfg, xk, tok)
    U.check_round_trip("k", cfg, xk, tok - 7)
