"""Host-side checks of the decode-attention entry points: workspace sizing and
argument validation.  Every call here returns before any HIP call (the
pointers are never dereferenced), so no GPU is needed."""

import ctypes

import pytest

K = pytest.importorskip("kv_cache_quantization_codec_amd")
B = K.binding

E = {name: code for code, name in B.STATUS_NAMES.items()}
FAKE = 0x10000          # 16-byte aligned, never dereferenced


def _cfg(kb=2, vb=2, G=32, R=128, D=128):
    return B.kivi_config(kb, vb, G, R, D)


def _ws(c, S, r, nq, nres):
    return B.lib().kivi_attention_workspace_bytes(ctypes.byref(c), S, r, nq, nres)


def _cache(**over):
    f = dict(k_codes=FAKE, k_scale=FAKE, k_zero=FAKE, v_codes=FAKE, v_scale=FAKE, v_zero=FAKE,
             cap_tokens=256, n_quant=200, res_k=FAKE, res_v=FAKE, res_slice_stride=160 * 128,
             res_slots=160, res_head=5, res_count=40, n_quant_per_slice=0, res_count_per_slice=0)
    f.update(over)
    return B.kivi_attn_cache(*(f[n] for n, _ in B.kivi_attn_cache._fields_))


def _call(c, cache, S=4, r=2, q=FAKE, sm=0.125, out=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return B.lib().kivi_decode_attention(ctypes.byref(c), ctypes.byref(cache) if cache else None,
                                         S, r, q, sm, out, ws, ws_bytes, None)


@pytest.mark.parametrize("S,r,nq,nres", [(8192, 1, 3968, 128), (256, 1, 3968, 128), (4096, 4, 16256, 128),
                                         (8, 1, 0, 128), (8192, 1, 3968, 0), (3, 8, 65, 1), (1, 1, 1, 0)])
def test_workspace_is_whole_partials_or_nothing(S, r, nq, nres):
    c = _cfg()
    ws = _ws(c, S, r, nq, nres)
    per_split = S * r * (c.head_dim + 2) * 4        # (max, sum, D outputs) fp32 per head
    assert ws >= 0 and ws % per_split == 0
    splits = ws // per_split
    assert splits != 1                              # one split writes the output directly
    blocks = -(-nq // 32)
    assert splits <= blocks + (1 if nres else 0)


def test_small_batches_are_split_and_residual_only_is_not():
    c = _cfg()
    assert _ws(c, 8, 1, 16256, 128) > 0             # few slices, long cache: split
    assert _ws(c, 8, 1, 0, 128) == 0                # residual only: one pass
    assert _ws(c, 1, 1, 32, 0) == 0                 # one block


@pytest.mark.parametrize("D,status", [(96, "KIVI_OK"), (64, "KIVI_OK"), (32, "KIVI_OK"),
                                      (80, "KIVI_E_HEAD_DIM"), (256, "KIVI_E_HEAD_DIM"),
                                      (160, "KIVI_E_HEAD_DIM")])
def test_head_dim_limits(D, status):
    c = _cfg(D=D)
    cache = _cache(res_slice_stride=160 * D)
    assert _call(c, cache, S=0) == E[status]
    assert (_ws(c, 4, 1, 64, 8) >= 0) == (status == "KIVI_OK")


ARGUMENT_ERRORS = [
    ({}, {"r": 0}, "KIVI_E_SHAPE"),
    ({}, {"r": 9}, "KIVI_E_SHAPE"),
    ({}, {"S": -1}, "KIVI_E_SHAPE"),
    ({"n_quant": 300}, {}, "KIVI_E_SHAPE"),           # beyond cap_tokens
    ({"n_quant": -1}, {}, "KIVI_E_SHAPE"),
    ({"res_count": 161}, {}, "KIVI_E_SHAPE"),         # beyond res_slots
    ({"res_head": 160}, {}, "KIVI_E_SHAPE"),
    ({"res_head": -1}, {}, "KIVI_E_SHAPE"),
    ({"n_quant": 0, "res_count": 0}, {}, "KIVI_E_SHAPE"),   # empty cache
    ({}, {"sm": float("inf")}, "KIVI_E_SHAPE"),
    ({}, {"sm": float("nan")}, "KIVI_E_SHAPE"),
    ({}, {"ws_bytes": 0}, "KIVI_E_SHAPE"),            # split plan needs a workspace
    ({"res_slice_stride": 160 * 128 - 8}, {}, "KIVI_E_SHAPE"),
    ({"res_slice_stride": 160 * 128 + 4}, {}, "KIVI_E_ALIGN"),
    ({}, {"q": 0}, "KIVI_E_NULL"),
    ({}, {"out": 0}, "KIVI_E_NULL"),
    ({}, {"ws": 0}, "KIVI_E_NULL"),
    ({"k_codes": 0}, {}, "KIVI_E_NULL"),
    ({"v_zero": 0}, {}, "KIVI_E_NULL"),
    ({"res_v": 0}, {}, "KIVI_E_NULL"),
    ({}, {"q": FAKE + 8}, "KIVI_E_ALIGN"),
    ({}, {"ws": FAKE + 4}, "KIVI_E_ALIGN"),
    ({"k_scale": FAKE + 2}, {}, "KIVI_E_ALIGN"),
    ({"res_k": FAKE + 8}, {}, "KIVI_E_ALIGN"),
    ({"n_quant_per_slice": FAKE + 2}, {}, "KIVI_E_ALIGN"),
    ({"res_count_per_slice": FAKE + 1}, {}, "KIVI_E_ALIGN"),
]


@pytest.mark.parametrize("over,kw,status", ARGUMENT_ERRORS)
def test_argument_errors(over, kw, status):
    c = _cfg()
    assert _ws(c, 4, 2, 200, 40) > 0, "the reference call must need a workspace"
    assert _call(c, _cache(**over), **kw) == E[status]


def test_unused_parts_may_be_null():
    c = _cfg()
    # residual only: quantized arrays unused; quantized only: residual unused
    q_only = _cache(res_k=0, res_v=0, res_count=0, res_slots=0, res_head=0, res_slice_stride=0)
    r_only = _cache(k_codes=0, k_scale=0, k_zero=0, v_codes=0, v_scale=0, v_zero=0, n_quant=0)
    for cache in (q_only, r_only):
        assert _call(c, cache, S=0) == E["KIVI_OK"]


def test_null_cache_and_config():
    c = _cfg()
    assert _call(c, None) == E["KIVI_E_NULL"]
    assert B.lib().kivi_decode_attention(None, ctypes.byref(_cache()), 4, 2, FAKE, 0.1, FAKE, FAKE,
                                         1 << 40, None) == E["KIVI_E_NULL"]
    assert B.lib().kivi_attention_workspace_bytes(None, 4, 2, 64, 8) == -1


def test_no_slices_is_a_noop_after_config_checks():
    c = _cfg()
    assert _call(c, _cache(), S=0, q=0, out=0, ws=0, ws_bytes=0) == E["KIVI_OK"]
    assert _call(_cfg(kb=3), _cache(), S=0) == E["KIVI_E_BITS"]


# ---- the no-allocation variant (library-owned static scratch) ----

def _call_noalloc(c, cache, S=4, r=2, q=FAKE, sm=0.125, out=FAKE):
    return B.lib().kivi_decode_attention_noalloc(ctypes.byref(c) if c else None,
                                                 ctypes.byref(cache) if cache else None,
                                                 S, r, q, sm, out, None)


@pytest.mark.parametrize("over,kw,status", [e for e in ARGUMENT_ERRORS if not set(e[1]) & {"ws", "ws_bytes"}])
def test_noalloc_argument_errors_match(over, kw, status):
    c = _cfg()
    assert _call_noalloc(c, _cache(**over), **kw) == E[status]


def test_noalloc_rejects_calls_beyond_the_scratch():
    c = _cfg()
    # 8192 slices x 8 query heads x 16256 quantized tokens: 4 splits of
    # (max, sum, 128 outputs) fp32 per head = 136,314,880 bytes > 128 MiB
    cache = _cache(cap_tokens=16384, n_quant=16256, res_k=0, res_v=0, res_count=0, res_slots=0,
                   res_head=0, res_slice_stride=0)
    need = _ws(c, 8192, 8, 16256, 0)
    assert need == 8192 * 4 * 8 * 130 * 4 > B.ATTENTION_SCRATCH_BYTES
    assert _call_noalloc(c, cache, S=8192, r=8) == E["KIVI_E_SCRATCH"]
    assert B.lib().kivi_status_string(E["KIVI_E_SCRATCH"]).decode().startswith("KIVI_E_SCRATCH")
    # config and cache checks come first, as in kivi_decode_attention
    assert _call_noalloc(None, cache, S=8192, r=8) == E["KIVI_E_NULL"]
    assert _call_noalloc(c, None) == E["KIVI_E_NULL"]
    assert _call_noalloc(c, _cache(), S=0, q=0, out=0) == E["KIVI_OK"]


def test_scratch_size_matches_header():
    import os
    import re
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "include", "kivi.h")).read()
    m = re.search(r"#define KIVI_ATTENTION_SCRATCH_BYTES \((\d+)LL << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == B.ATTENTION_SCRATCH_BYTES
