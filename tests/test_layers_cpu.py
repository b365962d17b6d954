"""Host-side checks of the per-layer bit-mix entry points: the boundary-layer
helper against the oracle, and argument validation of the layer-wise codec
calls.  Every codec call here returns before any HIP call (pointers are never
dereferenced), so no GPU is needed."""

import ctypes

import pytest

from oracle import layer_mix_ref as mix

K = pytest.importorskip("kv_cache_quantization_codec_amd")
B = K.binding

E = {name: code for code, name in B.STATUS_NAMES.items()}
FAKE = 0x10000          # 16-byte aligned, never dereferenced


@pytest.mark.parametrize("L", list(range(0, 41)) + [80, 126])
def test_boundary_layers_match_the_oracle(L):
    for n in range(-2, 30):
        assert K.kivi_boundary_layers(L, n) == mix.boundary_layers(L, n), (L, n)


def test_boundary_layers_errors_and_count():
    lib = B.lib()
    flags = (ctypes.c_int32 * 32)()
    assert lib.kivi_boundary_layers(32, 2, flags) == 4
    assert lib.kivi_boundary_layers(-1, 2, flags) == E["KIVI_E_SHAPE"]
    assert lib.kivi_boundary_layers(4, 2, None) == E["KIVI_E_NULL"]
    assert lib.kivi_boundary_layers(0, 2, None) == 0


def _cfgs(*bits, G=32, D=128):
    return (B.kivi_config * len(bits))(*[B.kivi_config(kb, vb, G, 128, D) for kb, vb in bits])


def _arr(vals):
    return (ctypes.c_void_p * len(vals))(*vals)


def _enc(cfgs, L, *, x=FAKE, lstride=None, S=4, n=100, sstride=128 * 128, cap=128, codes=None,
         scale=None, zero=None, keys=True):
    lstride = S * sstride if lstride is None else lstride
    codes = _arr([FAKE] * L) if codes is None else codes
    scale = _arr([FAKE] * L) if scale is None else scale
    zero = _arr([FAKE] * L) if zero is None else zero
    fn = B.lib().kivi_encode_k_layers if keys else B.lib().kivi_encode_v_layers
    return fn(cfgs, L, x, lstride, S, n, sstride, cap, codes, scale, zero, None)


def _dec(cfgs, L, *, out=FAKE, lstride=None, S=4, n=100, sstride=128 * 128, cap=128, keys=True):
    lstride = S * sstride if lstride is None else lstride
    fn = B.lib().kivi_decode_k_layers if keys else B.lib().kivi_decode_v_layers
    return fn(cfgs, L, _arr([FAKE] * L), _arr([FAKE] * L), _arr([FAKE] * L), S, n, cap, out, lstride,
              sstride, None)


MIX = [(8, 8), (2, 2), (2, 2), (8, 8)]


@pytest.mark.parametrize("keys", [True, False])
def test_layer_argument_errors(keys):
    c = _cfgs(*MIX)
    assert _enc(c, -1, keys=keys) == E["KIVI_E_SHAPE"]
    assert _enc(None, 4, keys=keys) == E["KIVI_E_NULL"]
    assert _enc(_cfgs((8, 8), (2, 3), (2, 2), (8, 8)), 4, keys=keys) == E["KIVI_E_BITS"]
    bad_g = (B.kivi_config * 2)(B.kivi_config(2, 2, 32, 128, 128), B.kivi_config(2, 2, 48, 128, 128))
    assert _enc(bad_g, 2, keys=keys) == E["KIVI_E_GROUP"]
    mixed_d = (B.kivi_config * 2)(B.kivi_config(2, 2, 32, 128, 128), B.kivi_config(2, 2, 32, 128, 64))
    assert _enc(mixed_d, 2, keys=keys) == E["KIVI_E_HEAD_DIM"]
    assert _enc(c, 4, cap=64, keys=keys) == E["KIVI_E_SHAPE"]                 # cap < n
    assert _enc(c, 4, sstride=100 * 128 - 8, keys=keys) == E["KIVI_E_SHAPE"]  # slice stride < n*D
    assert _enc(c, 4, lstride=4 * 128 * 128 - 8, keys=keys) == E["KIVI_E_SHAPE"]  # layers overlap
    assert _enc(c, 4, lstride=4 * 128 * 128 + 4, keys=keys) == E["KIVI_E_ALIGN"]
    assert _enc(c, 4, lstride=1 << 62, keys=keys) == E["KIVI_E_SHAPE"]        # span overflows
    assert _enc(c, 4, x=0, keys=keys) == E["KIVI_E_NULL"]
    assert _enc(c, 4, x=FAKE + 8, keys=keys) == E["KIVI_E_ALIGN"]
    assert _enc(c, 4, codes=_arr([FAKE, FAKE, 0, FAKE]), keys=keys) == E["KIVI_E_NULL"]
    assert _enc(c, 4, scale=_arr([FAKE, FAKE, FAKE, FAKE + 2]), keys=keys) == E["KIVI_E_ALIGN"]
    assert _enc(c, 4, zero=_arr([FAKE + 8, FAKE, FAKE, FAKE]), keys=keys) == E["KIVI_E_ALIGN"]
    fn = B.lib().kivi_encode_k_layers if keys else B.lib().kivi_encode_v_layers
    assert fn(c, 4, FAKE, 4 * 128 * 128, 4, 100, 128 * 128, 128, None, _arr([FAKE] * 4),
              _arr([FAKE] * 4), None) == E["KIVI_E_NULL"]
    assert _dec(c, 4, out=0, keys=keys) == E["KIVI_E_NULL"]
    assert _dec(c, 4, lstride=4 * 128 * 128 - 128, keys=keys) == E["KIVI_E_SHAPE"]
    assert _dec(_cfgs((8, 8), (2, 5)), 2, keys=keys) == E["KIVI_E_BITS"]


@pytest.mark.parametrize("keys", [True, False])
def test_no_work_calls_touch_no_pointer(keys):
    c = _cfgs(*MIX)
    assert _enc(c, 0, x=0, keys=keys) == E["KIVI_OK"]
    assert _enc(c, 4, S=0, x=0, codes=_arr([0] * 4), keys=keys) == E["KIVI_OK"]
    assert _enc(c, 4, n=0, x=0, keys=keys) == E["KIVI_OK"]
    assert _enc(c, 4, S=-1, keys=keys) == E["KIVI_E_SHAPE"]
    assert _dec(c, 4, n=0, out=0, keys=keys) == E["KIVI_OK"]


def test_alignment_is_required_of_run_starts_only():
    """Layers 1 and 2 (same config) continue a run when their arrays start
    where the previous layer's end; then only layer 1's arrays must be
    aligned.  A misaligned layer 2 outside a run is an error.  (Checked
    with zero-length fp16 layers so that no launch happens: the error paths
    return first, and the success path is not called here.)"""
    c = _cfgs((8, 8), (2, 2), (2, 2), (8, 8), D=96, G=128)
    S, cap = 5, 333
    code_b = 4 * S * B.lib().kivi_v_code_words(ctypes.byref(c[1]), cap)
    stat_b = 2 * S * B.lib().kivi_v_stat_elems(ctypes.byref(c[1]), cap)
    assert stat_b % 16 != 0
    base = 0x100000
    codes = _arr([FAKE, base, base + code_b, FAKE])
    scale = _arr([FAKE, 2 * base, 2 * base + stat_b, FAKE])
    zero = _arr([FAKE, 3 * base, 3 * base + stat_b + 16, FAKE])      # not back to back
    assert _enc(c, 4, S=S, n=300, sstride=300 * 96, cap=cap, codes=codes, scale=scale, zero=zero,
                keys=False) == E["KIVI_E_ALIGN"]
