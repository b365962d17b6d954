"""Host-side checks of the compact cache image: its size against the
oracle's per-array closed forms, and argument validation of offload and
restore (every call here returns before any HIP call)."""

import ctypes

import pytest

from oracle import kivi_ref as ref

K = pytest.importorskip("kv_cache_quantization_codec_amd")
B = K.binding
E = {name: code for code, name in B.STATUS_NAMES.items()}
FAKE = 0x10000


def _cfg(kb=2, vb=4, G=32, R=128, D=128):
    return B.kivi_config(kb, vb, G, R, D)


@pytest.mark.parametrize("kb,vb,G,R,D", [(2, 2, 32, 128, 128), (4, 8, 64, 96, 96), (8, 2, 128, 0, 64)])
@pytest.mark.parametrize("S,nq", [(1, 0), (3, 128), (16384, 2432)])
def test_image_size_is_the_sum_of_the_packed_arrays(kb, vb, G, R, D, S, nq):
    c = _cfg(kb, vb, G, R, D)
    nq = nq - nq % G
    want = S * (4 * ref.k_code_words(nq, D, kb, G) + 2 * 2 * ref.k_stat_elems(nq, D, G)
                + 4 * ref.v_code_words(nq, D, vb, G) + 2 * 2 * ref.v_stat_elems(nq, D, G)
                + 2 * 2 * (R + G) * D)
    assert B.lib().kivi_stream_image_bytes(ctypes.byref(c), S, nq) == want


def test_image_size_rejects_bad_sizes():
    c = _cfg()
    assert B.lib().kivi_stream_image_bytes(ctypes.byref(c), 1, 33) == -1      # not a multiple of G
    assert B.lib().kivi_stream_image_bytes(ctypes.byref(c), -1, 32) == -1
    assert B.lib().kivi_stream_image_bytes(None, 1, 32) == -1


def _stream(S=4, cap=256, nq=64, head=3, count=40):
    return B.kivi_stream(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, S, cap, nq, head, count)


def test_offload_errors():
    c = _cfg()
    need = B.lib().kivi_stream_image_bytes(ctypes.byref(c), 4, 64)
    st = _stream()
    off = lambda st, host=FAKE, n=need: B.lib().kivi_stream_offload(ctypes.byref(c), ctypes.byref(st), host, n, None)
    assert off(st, n=need - 1) == E["KIVI_E_SHAPE"]
    assert off(st, host=0) == E["KIVI_E_NULL"]
    assert off(_stream(nq=65)) == E["KIVI_E_STATE"]
    assert off(_stream(head=160)) == E["KIVI_E_STATE"]
    assert off(_stream(S=0), host=0, n=0) == E["KIVI_OK"]


@pytest.mark.parametrize("args,status", [
    ((65, 0, 0), "KIVI_E_STATE"),       # n_quant not a multiple of G
    ((288, 0, 0), "KIVI_E_CAPACITY"),   # beyond cap_tokens
    ((-32, 0, 0), "KIVI_E_STATE"),
    ((64, 160, 0), "KIVI_E_STATE"),     # ring_head outside R + G slots
    ((64, 0, 160), "KIVI_E_STATE"),     # ring_count > R + G - 1
    ((64, -1, 0), "KIVI_E_STATE"),
])
def test_restore_errors_leave_counters(args, status):
    c = _cfg()
    st = _stream()
    need = B.lib().kivi_stream_image_bytes(ctypes.byref(c), 4, max(args[0], 0) - max(args[0], 0) % 32)
    rc = B.lib().kivi_stream_restore(ctypes.byref(c), ctypes.byref(st), FAKE, max(need, 1 << 40), *args, None)
    assert rc == E[status]
    assert (st.n_quant, st.ring_head, st.ring_count) == (64, 3, 40)


def test_restore_host_size_and_null():
    c = _cfg()
    st = _stream()
    need = B.lib().kivi_stream_image_bytes(ctypes.byref(c), 4, 128)
    rs = lambda host, n: B.lib().kivi_stream_restore(ctypes.byref(c), ctypes.byref(st), host, n, 128, 5, 7, None)
    assert rs(FAKE, need - 1) == E["KIVI_E_SHAPE"]
    assert rs(0, need) == E["KIVI_E_NULL"]
    assert (st.n_quant, st.ring_head, st.ring_count) == (64, 3, 40)


def test_restore_without_slices_sets_counters_only():
    c = _cfg()
    st = _stream(S=0)
    assert B.lib().kivi_stream_restore(ctypes.byref(c), ctypes.byref(st), 0, 0, 96, 10, 20, None) == E["KIVI_OK"]
    assert (st.n_quant, st.ring_head, st.ring_count) == (96, 10, 20)
