"""kivi_decode_attention_noalloc (the entry point for callers that cannot
allocate device memory) against kivi_decode_attention with a caller
workspace, through the C ABI: same kernels and split plan, so the outputs
must agree bit for bit.  Two calls in a row on the shared static scratch, the
second on a smaller cache, both split over several workgroups per slice (so
the scratch holds partial sums); plus a ragged batch, a call that needs no
scratch, and a call too large for the scratch."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import kv_cache_quantization_codec_amd as K

pytestmark = pytest.mark.gpu


def _cache(cfg, S, n_quant, n_res, seed, ragged=False):
    """A cache encoded by the codec from seeded fp16 K/V (the prefix of
    n_quant tokens packed, the next n_res tokens as the fp16 residual)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    D = cfg.head_dim
    T = n_quant + n_res
    k = torch.randn((S, max(T, 1), D), generator=g, device="cuda").to(torch.float16)
    v = torch.randn((S, max(T, 1), D), generator=g, device="cuda").to(torch.float16)
    cap = max(n_quant, 1)
    keys = K.alloc_keys(cfg, S, cap, "cuda")
    vals = K.alloc_values(cfg, S, cap, "cuda")
    if n_quant:
        K.kivi_encode_k(cfg, k, n_quant, *keys, cap_tokens=cap)
        K.kivi_encode_v(cfg, v, n_quant, *vals, cap_tokens=cap)
    kw = {}
    if ragged:
        rng = np.random.default_rng(seed)
        kw = dict(n_quant_per_slice=torch.tensor(rng.integers(0, n_quant + 1, S), dtype=torch.int32,
                                                 device="cuda"),
                  res_count_per_slice=torch.tensor(rng.integers(0, n_res + 1, S), dtype=torch.int32,
                                                   device="cuda"))
    res = (k[:, n_quant:], v[:, n_quant:]) if n_res else (None, None)
    return K.AttnCache(cfg, keys, vals, n_quant, *res, 0, n_res, **kw)


def _compare(cfg, S, r, n_quant, n_res, seed, ragged=False):
    cache = _cache(cfg, S, n_quant, n_res, seed, ragged)
    g = torch.Generator(device="cuda").manual_seed(seed + 1)
    q = torch.randn((S, r, cfg.head_dim), generator=g, device="cuda").to(torch.float16)
    sm = cfg.head_dim ** -0.5
    want = torch.empty_like(q)
    K.kivi_decode_attention(cfg, cache, q, sm, want)
    got = torch.full_like(q, float("nan"))
    K.kivi_decode_attention_noalloc(cfg, cache, q, sm, got)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), \
        f"S={S} r={r} n_quant={n_quant} n_res={n_res}: outputs differ"
    assert not torch.isnan(got).any()
    return K.kivi_attention_workspace_bytes(cfg, S, r, n_quant, n_res)


def test_noalloc_twice_second_smaller():
    print("noalloc: two calls, 2/2-bit then 4/2-bit", flush=True)
    cfg = K.Config(2, 2, 32, 128, 128)
    need1 = _compare(cfg, 256, 2, 3968, 128, seed=11)
    cfg2 = K.Config(4, 2, 64, 128, 64)
    need2 = _compare(cfg2, 24, 4, 1000, 77, seed=12)
    # both calls split, so both went through the static scratch; the second
    # is smaller, so the scratch still holds the first call's partials past
    # the second's (which the second never reads)
    assert need1 > need2 > 0
    assert need1 <= K.ATTENTION_SCRATCH_BYTES


def test_noalloc_ragged_and_unsplit():
    print("noalloc: ragged batch, then a call with no split", flush=True)
    cfg = K.Config(2, 4, 32, 128, 128)
    assert _compare(cfg, 64, 4, 2048, 128, seed=21, ragged=True) > 0
    assert _compare(cfg, 8, 1, 0, 100, seed=22) == 0          # residual only: no scratch used


def test_noalloc_rejects_more_than_the_scratch():
    print("noalloc: a call beyond the scratch", flush=True)
    cfg = K.Config(2, 2, 32, 128, 128)
    S, r, nq = 8192, 8, 16256
    need = K.kivi_attention_workspace_bytes(cfg, S, r, nq, 0)
    assert need > K.ATTENTION_SCRATCH_BYTES
    # the size check comes before any launch: nothing is read or written
    keys = K.alloc_keys(cfg, S, nq, "cuda")
    vals = K.alloc_values(cfg, S, nq, "cuda")
    cache = K.AttnCache(cfg, keys, vals, nq)
    q = torch.zeros((S, r, 128), dtype=torch.float16, device="cuda")
    out = torch.zeros_like(q)
    with pytest.raises(K.KiviError) as e:
        K.kivi_decode_attention_noalloc(cfg, cache, q, 0.1, out)
    assert e.value.status == -11
    torch.cuda.synchronize()
    assert not out.any()
