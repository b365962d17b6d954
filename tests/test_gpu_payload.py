"""GPU round trip of the compact cache image: offload a streaming cache to
pinned host memory, restore it into a fresh stream, and check that the
restored stream is the same cache -- bit for bit, against the oracle's
encoding of the same tokens, and by continuing both streams."""

import numpy as np
import pytest
import torch

import kv_cache_quantization_codec_amd as K
from oracle import kivi_ref as ref

pytestmark = pytest.mark.gpu

F16 = np.float16


def _dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.float16).cuda()


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16) \
        if t.dtype == torch.float16 else t.detach().cpu().contiguous().numpy().view(np.uint32)


def _poison(st):
    for t in (*st.keys, *st.values, st.k_ring, st.v_ring):
        (t.view(torch.int16) if t.dtype == torch.float16 else t).fill_(0x5A5A)


def _state_equal(a: K.Stream, b: K.Stream):
    assert (a.n_quant, a.ring_head, a.ring_count) == (b.n_quant, b.ring_head, b.ring_count)
    cfg, nq = a.cfg, a.n_quant
    G = cfg.group_size
    ngk = -(-nq // G)
    for x, y in zip(a.keys, b.keys):
        assert np.array_equal(_bits(x)[:, :ngk * (x.shape[1] // max(1, -(-a.state.cap_tokens // G)))],
                              _bits(y)[:, :ngk * (y.shape[1] // max(1, -(-b.state.cap_tokens // G)))])
    rows = min(nq + a.ring_count, a.state.cap_tokens, b.state.cap_tokens)
    for x, y in zip(a.values, b.values):
        assert np.array_equal(_bits(x)[:, :rows], _bits(y)[:, :rows])
    slots = a.k_ring.shape[1]
    idx = [(a.ring_head + i) % slots for i in range(a.ring_count)]
    assert np.array_equal(_bits(a.k_ring)[:, idx], _bits(b.k_ring)[:, idx])
    assert np.array_equal(_bits(a.v_ring)[:, idx], _bits(b.v_ring)[:, idx])


@pytest.mark.parametrize("kb,vb,G,R,D", [(2, 2, 32, 128, 128), (4, 2, 64, 96, 96), (8, 4, 32, 0, 64)])
def test_offload_restore_round_trip_and_continuation(kb, vb, G, R, D):
    cfg = K.Config(kb, vb, G, R, D)
    S, T0, steps, more = 5, 300, 70, 90
    rng = np.random.default_rng(kb * 100 + vb * 10 + G)
    allk = rng.standard_normal((S, T0 + steps + more, D)).astype(F16)
    allv = rng.standard_normal((S, T0 + steps + more, D)).astype(F16)
    kd, vd = _dev16(allk), _dev16(allv)
    a = K.Stream(cfg, S, 640, "cuda")
    _poison(a)
    K.kivi_stream_prefill(a, kd[:, :T0], vd[:, :T0], T0)
    for i in range(steps):
        K.kivi_append_flush(a, kd[:, T0 + i].contiguous(), vd[:, T0 + i].contiguous())
    nq, head, count = a.n_quant, a.ring_head, a.ring_count
    nbytes = K.kivi_stream_image_bytes(cfg, S, nq)
    host = torch.empty(nbytes, dtype=torch.uint8).pin_memory()
    K.kivi_stream_offload(a, host)
    torch.cuda.synchronize()

    # the image's prefix arrays are the oracle's encoding of the first nq tokens
    img = host.numpy()
    kc, ks, kz = ref.encode_k(allk, nq, kb, G)
    vc, vs, vz = ref.encode_v(allv, nq, vb, G)
    off = 0
    for arr in (kc, ks, kz, vc, vs, vz):
        n = arr.nbytes
        assert np.array_equal(img[off:off + n], np.ascontiguousarray(arr).view(np.uint8).ravel())
        off += n
    assert off + 2 * S * (R + G) * D * 2 == nbytes

    b = K.Stream(cfg, S, 512, "cuda")       # another capacity: other pitches
    _poison(b)
    K.kivi_stream_restore(b, host, nq, head, count)
    torch.cuda.synchronize()
    _state_equal(a, b)
    for i in range(steps, steps + more):       # both streams go on identically
        for st in (a, b):
            K.kivi_append_flush(st, kd[:, T0 + i].contiguous(), vd[:, T0 + i].contiguous())
    torch.cuda.synchronize()
    assert b.n_quant > nq
    _state_equal(a, b)


def test_attention_is_unchanged_by_offload_and_restore():
    cfg = K.Config(2, 4, 32, 128, 128)
    S, T0 = 6, 700
    rng = np.random.default_rng(4)
    k = _dev16(rng.standard_normal((S, T0, 128)).astype(F16))
    v = _dev16(rng.standard_normal((S, T0, 128)).astype(F16))
    a = K.Stream(cfg, S, 1024, "cuda")
    K.kivi_stream_prefill(a, k, v, T0)
    q = _dev16(rng.standard_normal((S, 4, 128)).astype(F16))
    out_a = torch.empty_like(q)
    K.kivi_decode_attention(cfg, K.AttnCache.from_stream(a), q, 128 ** -0.5, out_a)
    host = torch.empty(K.kivi_stream_image_bytes(cfg, S, a.n_quant), dtype=torch.uint8).pin_memory()
    K.kivi_stream_offload(a, host)
    b = K.Stream(cfg, S, 768, "cuda")
    K.kivi_stream_restore(b, host, a.n_quant, a.ring_head, a.ring_count)
    out_b = torch.empty_like(q)
    K.kivi_decode_attention(cfg, K.AttnCache.from_stream(b), q, 128 ** -0.5, out_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
