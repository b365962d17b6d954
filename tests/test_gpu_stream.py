"""Streaming decode phase on the GPU (prefill, then one kivi_append_flush per
step) against the oracle's StreamRef: every flushed group is compared when
it is produced, and the final quantized arrays and fp16 residual at the end."""

import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from oracle import kivi_ref as ref  # noqa: E402
from tests import gpu_util as U  # noqa: E402

import kv_cache_quantization_codec_amd as K  # noqa: E402

F16 = np.float16


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.float16).cuda()


def compare_stream(st: K.Stream, sr: ref.StreamRef, slices=None, group_range=None):
    """Compare quantized groups [g0, g1) and the residual of slices ``slices``."""
    cfg = st.cfg
    G = cfg.group_size
    sel = slice(None) if slices is None else slices
    assert st.n_quant == sr.n_quant
    g0, g1 = (0, sr.n_quant // G) if group_range is None else group_range
    if g1 > g0:
        Wk = G * cfg.k_bits // 32
        kc, ks, kz = st.keys
        oc, os_, oz = sr.key_arrays()
        U.assert_equal("stream key codes", U.words(kc[sel][:, g0 * Wk:g1 * Wk]),
                       oc.view(np.uint32)[:, g0 * Wk:g1 * Wk])
        U.assert_equal("stream key scale", U.bits16(ks[sel][:, g0:g1]), os_.view(np.uint16)[:, g0:g1])
        U.assert_equal("stream key zero", U.bits16(kz[sel][:, g0:g1]), oz.view(np.uint16)[:, g0:g1])
        vc, vs, vz = st.values
        pc, ps, pz = sr.value_arrays()
        r0, r1 = g0 * G, g1 * G
        U.assert_equal("stream value codes", U.words(vc[sel][:, r0:r1]), pc.view(np.uint32)[:, r0:r1])
        U.assert_equal("stream value scale", U.bits16(vs[sel][:, r0:r1]), ps.view(np.uint16)[:, r0:r1])
        U.assert_equal("stream value zero", U.bits16(vz[sel][:, r0:r1]), pz.view(np.uint16)[:, r0:r1])
    rk, rv = U.ring_residual(st)
    U.assert_equal("residual k", U.bits16(rk[sel]), sr.res_k.view(np.uint16))
    U.assert_equal("residual v", U.bits16(rv[sel]), sr.res_v.view(np.uint16))
    # value rows are quantized on arrival: the residual's rows (below the
    # capacity) already hold the codes of the residual tokens
    n_res = sr.res_v.shape[1]
    r0, r1 = sr.n_quant, min(sr.n_quant + n_res, st.state.cap_tokens)
    if r1 > r0:
        qc, qs, qz = ref.encode_v(sr.res_v[:, :r1 - r0], r1 - r0, cfg.v_bits, G)
        vc, vs, vz = st.values
        U.assert_equal("residual value codes", U.words(vc[sel][:, r0:r1]), qc.view(np.uint32))
        U.assert_equal("residual value scale", U.bits16(vs[sel][:, r0:r1]), qs.view(np.uint16))
        U.assert_equal("residual value zero", U.bits16(vz[sel][:, r0:r1]), qz.view(np.uint16))


CASES = [
    # k_bits, v_bits, G, R, D, prefill tokens, steps
    (2, 2, 32, 128, 128, 300, 200),
    (4, 8, 64, 5, 96, 130, 260),
    (8, 2, 128, 0, 64, 260, 300),
    (2, 4, 32, 31, 128, 40, 130),     # R = G - 1: the new token is the last of the flushed group
    (4, 4, 32, 7, 8, 3, 100),
    (8, 8, 64, 200, 256, 500, 150),
]


@pytest.mark.parametrize("kb,vb,G,R,D,T0,steps", CASES)
def test_stream_matches_oracle_every_flush(kb, vb, G, R, D, T0, steps):
    run_stream(kb, vb, G, R, D, T0, steps, S=6)


# Flushes whose key group lies straight in the ring (R >= G, no wrap) take
# a lane per 8 channels and 8 tokens: (G/8) x (D/8) lanes per slice and
# 256 / that many slices per block, unless a slice would need more than a
# block (G = 128 with D > 128); the others take one lane per channel pair.
# These cases reach the row layout's edges: idle lanes in a block (D = 96),
# 64 slices per block (D = 8), half code words exchanged between lanes
# (2-bit keys at G = 32, 64 and 128), 4- and 8-bit keys, a whole block per
# slice (G = 128, D = 128; G = 64, D = 256), the fallback (G = 128,
# D = 256), a ring length that alternates the two layouts (R = 40, G = 32:
# groups at slots 0, 32, then 64..23 wrapping), and partial last blocks
# (37 slices at D = 96, 5 at G = 64).
SPLIT_CASES = [
    # k_bits, v_bits, G, R, D, prefill tokens, steps, slices
    (4, 2, 32, 64, 96, 100, 120, 6),
    (8, 4, 128, 128, 64, 300, 300, 6),
    (2, 8, 32, 40, 8, 50, 150, 6),
    (2, 2, 32, 32, 96, 70, 100, 37),
    (2, 4, 64, 64, 128, 100, 140, 5),
    (2, 2, 128, 128, 128, 200, 280, 3),
    (4, 8, 128, 160, 64, 170, 300, 4),
    (8, 2, 128, 128, 256, 140, 270, 3),
    (2, 4, 32, 64, 256, 90, 100, 3),
]


@pytest.mark.parametrize("kb,vb,G,R,D,T0,steps,S", SPLIT_CASES)
def test_stream_split_flush_layouts(kb, vb, G, R, D, T0, steps, S):
    run_stream(kb, vb, G, R, D, T0, steps, S=S)


def _adversarial_columns(S, T, D, seed):
    """Keys whose channels run along the hard rows of the codec tests
    (ties that a rounded reciprocal misleads, ranges on fp16 midpoints,
    subnormal and zero scales, signed zeros, constants, the widest range),
    one row per channel, cycled along tokens."""
    from tests.test_gpu_parity import _adversarial_rows
    rows = _adversarial_rows(D)
    rng = np.random.default_rng(seed)
    pick = rng.integers(0, rows.shape[0], size=(S, D))
    t = np.arange(T) % rows.shape[1]
    return np.stack([rows[pick[s]][:, t].T for s in range(S)]).astype(F16)


# Keys with exact rounding ties and with the hard rows above, so that every
# flush path takes its redo pass and its exact (non-fast) groups.
ADVERSARIAL_CASES = [
    # k_bits, v_bits, G, R, D, prefill tokens, steps, slices
    (2, 2, 32, 128, 128, 160, 200, 5),
    (4, 4, 64, 64, 96, 100, 200, 4),
    (8, 2, 128, 128, 64, 140, 300, 3),
    (2, 8, 32, 40, 64, 60, 140, 3),       # alternates with the one-lane-per-pair layout
    (4, 2, 128, 128, 256, 130, 260, 2),   # the one-lane-per-pair layout only
]


@pytest.mark.parametrize("kind", ["ties", "rows"])
@pytest.mark.parametrize("kb,vb,G,R,D,T0,steps,S", ADVERSARIAL_CASES)
def test_stream_adversarial_keys(kind, kb, vb, G, R, D, T0, steps, S):
    from kvsynth import uniform_with_ties

    def data(rng):
        T = T0 + steps
        if kind == "ties":
            k = uniform_with_ties(S, T, D, axis="token", n_valid=T, bits=kb, group_size=G,
                                  seed=kb + G + D, grid_group_fraction=0.3, tie_fraction_in_group=0.25)
        else:
            k = _adversarial_columns(S, T, D, seed=kb + G + D)
        v = uniform_with_ties(S, T, D, axis="channel", n_valid=T, bits=vb, group_size=G, seed=vb + G + D + 1)
        return k, v

    run_stream(kb, vb, G, R, D, T0, steps, S=S, data=data)


def run_stream(kb, vb, G, R, D, T0, steps, S, data=None):
    print(f"stream kb={kb} vb={vb} G={G} R={R} D={D} T0={T0} steps={steps} S={S}", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(kb * 100 + vb * 10 + G + R + D)
    if data is None:
        k_all = rng.standard_normal((S, T0 + steps, D)).astype(F16)
        v_all = (rng.standard_normal((S, T0 + steps, D)) * 3).astype(F16)
    else:
        k_all, v_all = data(rng)
    cap = -(-(T0 + steps) // G) * G
    cfg = K.Config(kb, vb, G, R, D)
    st = K.Stream(cfg, S, cap)
    for t in (*st.keys, *st.values):
        U.poisoned(t)
    K.kivi_stream_prefill(st, _t(k_all[:, :T0]), _t(v_all[:, :T0]), T0)
    sr = ref.StreamRef(kb, vb, G, R)
    sr.prefill(k_all[:, :T0], v_all[:, :T0], T0)
    assert (st.n_quant, st.ring_head, st.ring_count) == (sr.n_quant, 0, sr.res_k.shape[1])
    compare_stream(st, sr)
    k_new = _t(np.moveaxis(k_all[:, T0:], 1, 0))     # [steps, S, D]
    v_new = _t(np.moveaxis(v_all[:, T0:], 1, 0))
    for i in range(steps):
        flushed = K.kivi_append_flush(st, k_new[i], v_new[i])
        want = sr.append(k_all[:, T0 + i], v_all[:, T0 + i])
        assert flushed == want, f"step {i}"
        assert st.ring_count == sr.res_k.shape[1]
        if flushed:
            g = sr.n_quant // G
            compare_stream(st, sr, group_range=(g - 1, g))
    compare_stream(st, sr)
    # nothing beyond the quantized prefix was written
    Wk = G * kb // 32
    g = st.n_quant // G
    assert U.is_poison(U.words(st.keys[0][:, g * Wk:])) and U.is_poison(U.bits16(st.keys[1][:, g:]))
    assert U.is_poison(U.words(st.values[0][:, st.n_quant + st.ring_count:]))
    # the stream's quantized prefix equals a one-shot encode of the same tokens
    oc, _, _ = ref.encode_k(k_all, st.n_quant, kb, G)
    U.assert_equal("one-shot keys", U.words(st.keys[0][:, :g * Wk]), oc.view(np.uint32))


def test_capacity_error_leaves_stream_unchanged():
    cfg = K.Config(2, 2, 32, 4, 64)
    S = 3
    st = K.Stream(cfg, S, 32)
    x = torch.randn((S, 36, 64), device="cuda").half()
    K.kivi_stream_prefill(st, x, x, 36)                  # 32 quantized, 4 residual: store full
    assert (st.n_quant, st.ring_count) == (32, 4)
    tok = torch.randn((S, 64), device="cuda").half()
    before = U.words(st.keys[0]).copy()
    flushes = 0
    with pytest.raises(K.KiviError) as e:
        for _ in range(40):
            flushes += K.kivi_append_flush(st, tok, tok)
    assert "CAPACITY" in str(e.value) and flushes == 0
    # appends 1..27 take the residual to 31; the 28th would make it 32 = G and flush
    assert st.n_quant == 32 and st.ring_count == 31
    torch.cuda.synchronize()
    assert np.array_equal(U.words(st.keys[0]), before)
