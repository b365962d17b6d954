"""The C-ABI library loads, exports what include/kivi.h declares, sizes
buffers like the oracle's closed forms, and rejects bad arguments before any
HIP call.  Runs without a GPU: no call here reaches a kernel launch."""

import ctypes
import os
import re

import pytest

from oracle import kivi_ref as ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kivi.h")

K = pytest.importorskip("kv_cache_quantization_codec_amd")
B = K.binding

E = {name: code for code, name in B.STATUS_NAMES.items()}
FAKE = 0x10000          # a 16-byte-aligned non-null address that is never dereferenced
MISALIGNED = 0x10008


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(kivi_\w+)\s*\(", src, flags=re.M))


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    declared = _declared_functions()
    assert {"kivi_encode_k", "kivi_encode_v", "kivi_decode_k", "kivi_decode_v",
            "kivi_append_flush"} <= declared
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == {n for n, _, _ in B.SIGNATURES}


def test_status_codes_match_header():
    src = open(HEADER).read()
    for name, val in re.findall(r"(KIVI_(?:OK|E_\w+))\s*=\s*(-?\d+)", src):
        assert B.STATUS_NAMES[int(val)] == name
        assert B.lib().kivi_status_string(int(val)).decode().startswith(name)


def _cfg(kb=2, vb=2, G=32, R=128, D=128):
    return B.kivi_config(kb, vb, G, R, D)


@pytest.mark.parametrize("kb,vb,G,D", [(2, 2, 32, 128), (4, 8, 64, 96), (8, 4, 128, 64),
                                       (2, 8, 128, 96), (4, 2, 32, 8), (8, 8, 32, 256)])
@pytest.mark.parametrize("n", [0, 1, 31, 32, 33, 1000, 3077])
def test_sizes_match_closed_forms(kb, vb, G, D, n):
    c = _cfg(kb, vb, G, 128, D)
    lib = B.lib()
    assert lib.kivi_k_code_words(ctypes.byref(c), n) == ref.k_code_words(n, D, kb, G)
    assert lib.kivi_k_stat_elems(ctypes.byref(c), n) == ref.k_stat_elems(n, D, G)
    assert lib.kivi_v_code_words(ctypes.byref(c), n) == ref.v_code_words(n, D, vb, G)
    assert lib.kivi_v_stat_elems(ctypes.byref(c), n) == ref.v_stat_elems(n, D, G)
    assert lib.kivi_ring_elems(ctypes.byref(c)) == (128 + G) * D


@pytest.mark.parametrize("field,value,status", [
    ("k_bits", 3, "KIVI_E_BITS"), ("v_bits", 1, "KIVI_E_BITS"), ("k_bits", 16, "KIVI_E_BITS"),
    ("group_size", 16, "KIVI_E_GROUP"), ("group_size", 256, "KIVI_E_GROUP"),
    ("head_dim", 0, "KIVI_E_HEAD_DIM"), ("head_dim", 100, "KIVI_E_HEAD_DIM"),
    ("head_dim", 264, "KIVI_E_HEAD_DIM"), ("residual_length", -1, "KIVI_E_RESIDUAL"),
])
def test_bad_config(field, value, status):
    c = _cfg()
    setattr(c, field, value)
    lib = B.lib()
    assert lib.kivi_validate_config(ctypes.byref(c)) == E[status]
    assert lib.kivi_k_code_words(ctypes.byref(c), 10) == -1
    assert lib.kivi_encode_k(ctypes.byref(c), FAKE, 1, 32, 4096, 32, FAKE, FAKE, FAKE, None) == E[status]
    assert lib.kivi_decode_v(ctypes.byref(c), FAKE, FAKE, FAKE, 1, 32, 32, FAKE, 4096, None) == E[status]


def test_null_config():
    lib = B.lib()
    assert lib.kivi_validate_config(None) == E["KIVI_E_NULL"]
    assert lib.kivi_encode_v(None, FAKE, 1, 32, 4096, 32, FAKE, FAKE, FAKE, None) == E["KIVI_E_NULL"]


ENC = ["kivi_encode_k", "kivi_encode_v"]
DEC = ["kivi_decode_k", "kivi_decode_v"]


def _enc(name, c, inp=FAKE, S=2, n=64, stride=128 * 128, cap=64, codes=FAKE, sc=FAKE, zr=FAKE):
    return getattr(B.lib(), name)(ctypes.byref(c), inp, S, n, stride, cap, codes, sc, zr, None)


def _dec(name, c, codes=FAKE, sc=FAKE, zr=FAKE, S=2, n=64, cap=64, out=FAKE, stride=128 * 128):
    return getattr(B.lib(), name)(ctypes.byref(c), codes, sc, zr, S, n, cap, out, stride, None)


@pytest.mark.parametrize("name", ENC)
def test_encode_argument_errors(name):
    c = _cfg()
    assert _enc(name, c, inp=0) == E["KIVI_E_NULL"]
    assert _enc(name, c, codes=0) == E["KIVI_E_NULL"]
    assert _enc(name, c, sc=0) == E["KIVI_E_NULL"]
    assert _enc(name, c, zr=0) == E["KIVI_E_NULL"]
    assert _enc(name, c, inp=MISALIGNED) == E["KIVI_E_ALIGN"]
    assert _enc(name, c, codes=MISALIGNED) == E["KIVI_E_ALIGN"]
    assert _enc(name, c, zr=FAKE + 2) == E["KIVI_E_ALIGN"]
    assert _enc(name, c, stride=128 * 64 + 4) == E["KIVI_E_ALIGN"]
    assert _enc(name, c, stride=128 * 63) == E["KIVI_E_SHAPE"]        # stride < n * D
    assert _enc(name, c, cap=63) == E["KIVI_E_SHAPE"]                 # cap < n
    assert _enc(name, c, S=-1) == E["KIVI_E_SHAPE"]
    assert _enc(name, c, n=-5) == E["KIVI_E_SHAPE"]
    assert _enc(name, c, n=(1 << 30) + 1, cap=(1 << 30) + 1, stride=((1 << 30) + 1) * 128) == E["KIVI_E_SHAPE"]
    assert _enc(name, c, S=1 << 50, stride=1 << 20) == E["KIVI_E_SHAPE"]  # byte size overflows


@pytest.mark.parametrize("name", DEC)
def test_decode_argument_errors(name):
    c = _cfg()
    assert _dec(name, c, codes=0) == E["KIVI_E_NULL"]
    assert _dec(name, c, out=0) == E["KIVI_E_NULL"]
    assert _dec(name, c, out=MISALIGNED) == E["KIVI_E_ALIGN"]
    assert _dec(name, c, sc=FAKE + 4) == E["KIVI_E_ALIGN"]
    assert _dec(name, c, stride=128 * 64 - 8) == E["KIVI_E_SHAPE"]
    assert _dec(name, c, cap=10) == E["KIVI_E_SHAPE"]


@pytest.mark.parametrize("name", ENC + DEC)
def test_empty_calls_are_noops_that_touch_nothing(name):
    c = _cfg()
    fn = _enc if name in ENC else _dec
    # null pointers are fine when there is nothing to do
    kw = dict(codes=0, sc=0, zr=0) | ({"inp": 0} if name in ENC else {"out": 0})
    assert fn(name, c, S=0, **kw) == 0
    assert fn(name, c, n=0, **kw) == 0


def _stream(c, S=4, cap=256, **over):
    st = B.kivi_stream(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, S, cap, 0, 0, 0)
    for k, v in over.items():
        setattr(st, k, v)
    return st


def _step(c, st, k=FAKE, v=FAKE):
    return B.lib().kivi_append_flush(ctypes.byref(c), ctypes.byref(st), k, v, None)


@pytest.mark.parametrize("over,status", [
    (dict(n_quant=16), "KIVI_E_STATE"),            # not a multiple of G
    (dict(n_quant=288), "KIVI_E_STATE"),           # beyond cap
    (dict(ring_head=160), "KIVI_E_STATE"),         # head outside [0, R + G)
    (dict(ring_head=-1), "KIVI_E_STATE"),
    (dict(ring_count=160), "KIVI_E_STATE"),        # more than R + G - 1 residual tokens
    (dict(ring_count=-1), "KIVI_E_STATE"),
    (dict(cap_tokens=100), "KIVI_E_STATE"),        # cap not a multiple of G
    (dict(n_slices=-1), "KIVI_E_SHAPE"),
    (dict(k_ring=0), "KIVI_E_NULL"),
    (dict(v_codes=0), "KIVI_E_NULL"),
    (dict(k_scale=MISALIGNED), "KIVI_E_ALIGN"),
])
def test_stream_state_errors_leave_counters(over, status):
    c = _cfg()
    st = _stream(c, **over)
    before = (st.n_quant, st.ring_head, st.ring_count)
    assert _step(c, st) == E[status]
    assert (st.n_quant, st.ring_head, st.ring_count) == before


def test_stream_ring_slot_limit():
    # the flush kernels address a block's rings with 32-bit byte offsets, so
    # R + G is capped at 2^21 slots for every stream call
    lib = B.lib()
    ok = _cfg(G=32, R=(1 << 21) - 32)                     # exactly 2^21 slots
    st = _stream(ok, S=0, cap=64, ring_count=10)          # no slices: counters only
    assert _step(ok, st, k=0, v=0) == 0 and st.ring_count == 11
    big = _cfg(G=32, R=(1 << 21) - 31)
    for S in (0, 4):
        st = _stream(big, S=S, ring_count=10)
        assert _step(big, st) == E["KIVI_E_SHAPE"] and st.ring_count == 10
    st = _stream(big, S=4, cap=256)
    assert lib.kivi_stream_prefill(ctypes.byref(big), ctypes.byref(st), FAKE, FAKE, 64, 64 * 128,
                                   None) == E["KIVI_E_SHAPE"]


def test_stream_capacity_error_is_atomic():
    c = _cfg()
    # residual at R tokens: the next append would flush a group into a full store
    st = _stream(c, cap=256, n_quant=256, ring_head=7, ring_count=128)
    assert _step(c, st) == E["KIVI_E_CAPACITY"]
    assert (st.n_quant, st.ring_head, st.ring_count) == (256, 7, 128)
    assert _step(c, st, k=0) == E["KIVI_E_CAPACITY"]       # capacity is checked first


def test_stream_step_pointer_errors():
    c = _cfg()
    st = _stream(c, ring_count=10)
    assert _step(c, st, k=0) == E["KIVI_E_NULL"]
    assert _step(c, st, v=MISALIGNED) == E["KIVI_E_ALIGN"]
    assert st.ring_count == 10


def test_stream_with_no_slices_only_moves_counters():
    c = _cfg(G=32, R=4)
    st = _stream(c, S=0, cap=64, ring_count=0)
    flushes = 0
    for _ in range(70):
        n0 = st.n_quant
        assert _step(c, st, k=0, v=0) == 0
        flushes += st.n_quant != n0
        assert 0 <= st.ring_count <= 4 + 32 - 1
    # R = 4 < G: a flush needs G residual tokens, so it fires every 32 steps
    assert flushes == 2 and st.n_quant == 64 and st.ring_count == 70 - 64
    assert _step(c, _stream(c, S=0, cap=64, n_quant=64, ring_count=31), k=0, v=0) == E["KIVI_E_CAPACITY"]


def test_prefill_counters_without_slices():
    c = _cfg(G=32, R=128)
    lib = B.lib()
    for n, nq, rest in [(2048, 1920, 128), (2053, 1920, 133), (100, 0, 100), (160, 32, 128), (0, 0, 0)]:
        st = _stream(c, S=0, cap=4096)
        assert lib.kivi_stream_prefill(ctypes.byref(c), ctypes.byref(st), 0, 0, n, n * 128, None) == 0
        assert (st.n_quant, st.ring_head, st.ring_count) == (nq, 0, rest)
        assert nq == (ref.quantized_tokens(n, 128) // 32) * 32
    st = _stream(c, S=0, cap=1024)
    assert lib.kivi_stream_prefill(ctypes.byref(c), ctypes.byref(st), 0, 0, 2048, 2048 * 128, None) \
        == E["KIVI_E_CAPACITY"]


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "libkivi.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(ImportError):
        B.lib()
