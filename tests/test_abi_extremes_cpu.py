"""Extreme counts, strides and sizes at the C ABI: every call returns an
error code (or -1 from a sizing entry point) before any HIP call, and the
arithmetic that decides it never overflows.  tests/test_host_sanitizers.py
runs this module against a build under AddressSanitizer and
UndefinedBehaviorSanitizer, where a signed overflow in a check would abort.
No GPU needed; no pointer here is ever dereferenced."""

import ctypes

import pytest

K = pytest.importorskip("kv_cache_quantization_codec_amd")
B = K.binding

E = {name: code for code, name in B.STATUS_NAMES.items()}
FAKE = 0x10000
I64_MAX = 2 ** 63 - 1
# slice counts whose arrays overflow 64-bit byte sizes at 4096 x 128 fp16
# elements per slice (smaller counts are valid calls that would launch)
BIG = [2 ** 44, 2 ** 62, I64_MAX - 7]


def _cfg(kb=2, vb=2, G=32, R=128, D=128):
    return ctypes.byref(B.kivi_config(kb, vb, G, R, D))


@pytest.mark.parametrize("n", [2 ** 30 + 1, 2 ** 40, 2 ** 62, I64_MAX])
def test_sizing_helpers_reject_token_counts_past_the_limit(n):
    lib = B.lib()
    for fn in (lib.kivi_k_code_words, lib.kivi_k_stat_elems, lib.kivi_v_code_words, lib.kivi_v_stat_elems):
        assert fn(_cfg(8, 8, 32, 128, 256), n) == -1
    assert lib.kivi_k_code_words(_cfg(), 2 ** 30) == 2 ** 30 // 32 * 2 * 128


@pytest.mark.parametrize("S", BIG)
def test_codec_calls_with_huge_slice_counts(S):
    lib = B.lib()
    for name in ("kivi_encode_k", "kivi_encode_v"):
        assert getattr(lib, name)(_cfg(), FAKE, S, 4096, 4096 * 128, 4096, FAKE, FAKE, FAKE, None) == E["KIVI_E_SHAPE"]
    for name in ("kivi_decode_k", "kivi_decode_v"):
        assert getattr(lib, name)(_cfg(), FAKE, FAKE, FAKE, S, 4096, 4096, FAKE, 4096 * 128, None) == E["KIVI_E_SHAPE"]


@pytest.mark.parametrize("stride", [I64_MAX - 7, 2 ** 62, 2 ** 60])
def test_codec_calls_with_huge_strides(stride):
    lib = B.lib()
    assert lib.kivi_encode_k(_cfg(), FAKE, 8, 4096, stride, 4096, FAKE, FAKE, FAKE, None) == E["KIVI_E_SHAPE"]
    assert lib.kivi_decode_v(_cfg(), FAKE, FAKE, FAKE, 8, 4096, 4096, FAKE, stride, None) == E["KIVI_E_SHAPE"]


@pytest.mark.parametrize("n,cap", [(2 ** 30 + 1, 2 ** 30 + 1), (32, I64_MAX), (I64_MAX, I64_MAX), (-1, 32), (32, -1)])
def test_codec_calls_with_extreme_token_counts(n, cap):
    lib = B.lib()
    stride = 2 ** 40
    assert lib.kivi_encode_v(_cfg(), FAKE, 1, n, stride, cap, FAKE, FAKE, FAKE, None) == E["KIVI_E_SHAPE"]
    assert lib.kivi_decode_k(_cfg(), FAKE, FAKE, FAKE, 1, n, cap, FAKE, stride, None) == E["KIVI_E_SHAPE"]


def test_fp8_calls_with_extremes():
    lib = B.lib()
    for args in ((FAKE, I64_MAX, 16, 128, 2048, FAKE, 2048), (FAKE, 1, I64_MAX, 128, 2048, FAKE, 2048),
                 (FAKE, 2 ** 40, 16, 128, 2 ** 40, FAKE, 2048), (FAKE, 1, 16, 128, I64_MAX - 15, FAKE, 2048)):
        assert lib.kivi_fp8_encode(*args, None) == E["KIVI_E_SHAPE"]
        assert lib.kivi_fp8_decode(*args, None) == E["KIVI_E_SHAPE"]


def _stream(**over):
    f = dict(k_codes=FAKE, v_codes=FAKE, k_scale=FAKE, k_zero=FAKE, v_scale=FAKE, v_zero=FAKE,
             k_ring=FAKE, v_ring=FAKE, n_slices=4, cap_tokens=256, n_quant=64, ring_head=3, ring_count=100)
    f.update(over)
    return B.kivi_stream(*(f[n] for n, _ in B.kivi_stream._fields_))


@pytest.mark.parametrize("over", [dict(n_slices=I64_MAX), dict(n_slices=2 ** 60), dict(cap_tokens=I64_MAX - 31),
                                  dict(n_quant=I64_MAX - 31), dict(ring_head=I64_MAX), dict(ring_count=I64_MAX),
                                  dict(ring_head=-I64_MAX), dict(cap_tokens=2 ** 40)])
def test_stream_calls_with_extreme_state(over):
    lib = B.lib()
    st = _stream(**over)
    before = (st.n_quant, st.ring_head, st.ring_count)
    rc = lib.kivi_append_flush(_cfg(), ctypes.byref(st), FAKE, FAKE, None)
    assert rc in (E["KIVI_E_SHAPE"], E["KIVI_E_STATE"], E["KIVI_E_CAPACITY"])
    assert (st.n_quant, st.ring_head, st.ring_count) == before
    rc = lib.kivi_stream_prefill(_cfg(), ctypes.byref(st), FAKE, FAKE, 1 << 20, 1 << 27, None)
    assert rc in (E["KIVI_E_SHAPE"], E["KIVI_E_STATE"], E["KIVI_E_CAPACITY"])
    assert lib.kivi_stream_offload(_cfg(), ctypes.byref(st), FAKE, I64_MAX, None) in (
        E["KIVI_E_SHAPE"], E["KIVI_E_STATE"])


@pytest.mark.parametrize("S", [I64_MAX, 2 ** 56])
def test_image_and_workspace_sizes_with_huge_slice_counts(S):
    lib = B.lib()
    assert lib.kivi_stream_image_bytes(_cfg(), S, 3968 - 3968 % 32) == -1
    assert lib.kivi_attention_workspace_bytes(_cfg(), S, 8, 3968, 128) == -1


@pytest.mark.parametrize("nq", [I64_MAX, 2 ** 30 + 1])
def test_image_and_workspace_sizes_with_huge_token_counts(nq):
    lib = B.lib()
    assert lib.kivi_stream_image_bytes(_cfg(), 8192, nq - nq % 32 + 32 if nq < 2 ** 40 else nq) == -1
    assert lib.kivi_attention_workspace_bytes(_cfg(), 8192, 8, nq, 128) == -1


def _cache(**over):
    f = dict(k_codes=FAKE, k_scale=FAKE, k_zero=FAKE, v_codes=FAKE, v_scale=FAKE, v_zero=FAKE,
             cap_tokens=256, n_quant=200, res_k=FAKE, res_v=FAKE, res_slice_stride=160 * 128,
             res_slots=160, res_head=5, res_count=40, n_quant_per_slice=0, res_count_per_slice=0)
    f.update(over)
    return B.kivi_attn_cache(*(f[n] for n, _ in B.kivi_attn_cache._fields_))


@pytest.mark.parametrize("S,over", [(I64_MAX, {}), (2 ** 40, {}), (4, dict(res_slice_stride=I64_MAX - 7)),
                                    (4, dict(cap_tokens=I64_MAX)), (4, dict(res_slots=I64_MAX, res_count=1)),
                                    (2 ** 33, dict(res_slice_stride=2 ** 33))])
def test_attention_calls_with_extremes(S, over):
    lib = B.lib()
    cache = _cache(**over)
    assert lib.kivi_decode_attention(_cfg(), ctypes.byref(cache), S, 2, FAKE, 0.1, FAKE, FAKE, I64_MAX,
                                     None) == E["KIVI_E_SHAPE"]
    assert lib.kivi_decode_attention_noalloc(_cfg(), ctypes.byref(cache), S, 2, FAKE, 0.1, FAKE,
                                             None) in (E["KIVI_E_SHAPE"], E["KIVI_E_SCRATCH"])


@pytest.mark.parametrize("S,lstride,sstride", [(4, I64_MAX - 7, 4096 * 128), (I64_MAX - 7, 2 ** 40, 4096 * 128),
                                              (4, 2 ** 62, 4096 * 128), (2 ** 40, 2 ** 62, 2 ** 20)])
def test_layer_calls_with_extremes(S, lstride, sstride):
    lib = B.lib()
    cfgs = (B.kivi_config * 2)(*[B.kivi_config(2, 2, 32, 128, 128)] * 2)
    ptrs = (ctypes.c_void_p * 2)(FAKE, FAKE)
    assert lib.kivi_encode_k_layers(cfgs, 2, FAKE, lstride, S, 4096, sstride, 4096, ptrs, ptrs, ptrs,
                                    None) == E["KIVI_E_SHAPE"]
    assert lib.kivi_decode_v_layers(cfgs, 2, ptrs, ptrs, ptrs, S, 4096, 4096, FAKE, lstride, sstride,
                                    None) == E["KIVI_E_SHAPE"]
