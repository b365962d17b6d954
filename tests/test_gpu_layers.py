"""GPU parity of the layer-wise codec calls (per-layer bit mixes) with the
oracle (oracle/layer_mix_ref.py), through the C ABI.

Each model's layers are coded by kivi_{encode,decode}_{k,v}_layers; every
layer's codes, sidecars and decoded values must equal the oracle's coding of
that layer with its own configuration bit for bit, and nothing outside the
written region may change (outputs start poisoned).  Layouts cover runs
that one launch codes (payloads back to back, from alloc_layers) and
layouts that force a launch per layer (separate allocations, padded fp16
layers)."""

import sys

import numpy as np
import pytest
import torch

import kv_cache_quantization_codec_amd as K
from oracle import kivi_ref as ref
from oracle import layer_mix_ref as mix
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

F16 = np.float16


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _model(seed, L, S, T, D):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((L, S, T, D))
    ch = rng.random((L, S, 1, D)) < 0.05
    k = np.where(ch, k * 10 + 3, k)
    v = rng.standard_normal((L, S, T, D)) * rng.uniform(0.5, 2.0, (L, S, T, 1))
    return k.astype(F16), v.astype(F16)


def _dev(x, layer_pad=0):
    """fp16 [L, S, T, D] on the device, optionally with layer_pad spare
    elements between layers."""
    L, S, T, D = x.shape
    flat = torch.zeros((L, S * T * D + layer_pad), dtype=torch.int16)
    flat[:, :S * T * D] = torch.from_numpy(x.reshape(L, -1).view(np.int16))
    t = flat.cuda().view(torch.float16)
    return t.as_strided((L, S, T, D), (S * T * D + layer_pad, T * D, D, 1))


def _payloads(cfgs, S, cap, keys, contiguous):
    if contiguous:
        lay = K.alloc_layers(cfgs, S, cap, "cuda", keys=keys)
    else:
        alloc = K.alloc_keys if keys else K.alloc_values
        lay = [alloc(c, S, cap, "cuda") for c in cfgs]
    for p in lay:
        for t in p:
            U.poisoned(t)
    return lay


def run_model(cfgs, S, T, n, *, cap=None, contiguous=True, layer_pad=0, seed=0):
    L, D = len(cfgs), cfgs[0].head_dim
    cap = n if cap is None else cap
    k, v = _model(seed, L, S, T, D)
    _log(f"layers: L={L} S={S} T={T} n={n} cap={cap} contiguous={contiguous} pad={layer_pad} "
         f"cfgs={[(c.k_bits, c.v_bits, c.group_size) for c in cfgs]}")
    for keys, x in ((True, k), (False, v)):
        xd = _dev(x, layer_pad)
        lay = _payloads(cfgs, S, cap, keys, contiguous)
        enc = K.kivi_encode_k_layers if keys else K.kivi_encode_v_layers
        dec = K.kivi_decode_k_layers if keys else K.kivi_decode_v_layers
        enc(cfgs, xd, n, lay, cap_tokens=cap)
        out = U.poisoned(torch.empty((L, S, T + 2, D), dtype=torch.float16, device="cuda"))
        dec(cfgs, lay, n, out, cap_tokens=cap)
        torch.cuda.synchronize()
        for l, c in enumerate(cfgs):
            G, b = c.group_size, (c.k_bits if keys else c.v_bits)
            bits = [(cc.k_bits, cc.v_bits) for cc in cfgs]
            oc, os_, oz = mix.encode_layers(x[l:l + 1], n, bits[l:l + 1], G, keys)[0]
            gc, gs, gz = (U.words(lay[l][0]), U.bits16(lay[l][1]), U.bits16(lay[l][2]))
            side = "key" if keys else "value"
            if keys:
                ng, W = ref.n_groups(n, G), G * b // 32
                U.assert_equal(f"layer {l} {side} codes", gc[:, :ng * W], oc.view(np.uint32))
                U.assert_equal(f"layer {l} {side} scale", gs[:, :ng], os_.view(np.uint16))
                U.assert_equal(f"layer {l} {side} zero", gz[:, :ng], oz.view(np.uint16))
                assert U.is_poison(gc[:, ng * W:]) and U.is_poison(gs[:, ng:])
            else:
                U.assert_equal(f"layer {l} {side} codes", gc[:, :n], oc.view(np.uint32))
                U.assert_equal(f"layer {l} {side} scale", gs[:, :n], os_.view(np.uint16))
                U.assert_equal(f"layer {l} {side} zero", gz[:, :n], oz.view(np.uint16))
                assert U.is_poison(gc[:, n:]) and U.is_poison(gs[:, n:])
            od = mix.decode_layers([(oc, os_, oz)], n, bits[l:l + 1], G, D, keys)[0]
            go = U.bits16(out[l])
            U.assert_equal(f"layer {l} {side} decoded", go[:, :n], od.view(np.uint16))
            assert U.is_poison(go[:, n:]), f"layer {l}: decode wrote beyond n_tokens"


def _boundary_cfgs(L, n, base, prot, G=32, D=128):
    return [K.Config(kb, vb, G, 128, D) for kb, vb in mix.layer_bits(L, n, base, prot)]


@pytest.mark.parametrize("contiguous", [True, False])
def test_boundary_mix(contiguous):
    cfgs = _boundary_cfgs(8, 2, (2, 2), (8, 8))
    run_model(cfgs, S=3, T=300, n=250, cap=256, contiguous=contiguous, seed=1)


def test_boundary_mix_padded_layers():
    # fp16 layers not back to back: one launch per layer
    cfgs = _boundary_cfgs(6, 1, (2, 4), (4, 8))
    run_model(cfgs, S=4, T=200, n=173, cap=192, layer_pad=24, seed=2)


def test_mixed_group_sizes_and_head_dim():
    cfgs = [K.Config(4, 2, 128, 0, 96), K.Config(2, 2, 32, 0, 96), K.Config(2, 2, 32, 0, 96),
            K.Config(2, 2, 64, 0, 96), K.Config(8, 4, 64, 0, 96)]
    run_model(cfgs, S=5, T=400, n=333, seed=3)


def test_one_layer_and_uniform_model():
    run_model([K.Config(4, 4, 64, 0, 128)], S=7, T=130, n=129, seed=4)
    run_model([K.Config(2, 2, 32, 0, 64)] * 5, S=2, T=96, n=96, seed=5)


def test_uniform_model_equals_one_call_over_all_slices():
    """A model whose layers share one configuration is one run: the result
    equals a single-layer call over all L*S slices, bit for bit."""
    L, S, T, D = 4, 6, 260, 128
    cfg = K.Config(2, 4, 32, 0, D)
    k, v = _model(6, L, S, T, D)
    for keys, x in ((True, k), (False, v)):
        xd = _dev(x)
        lay = _payloads([cfg] * L, S, T, keys, True)
        (K.kivi_encode_k_layers if keys else K.kivi_encode_v_layers)([cfg] * L, xd, T, lay)
        alloc = K.alloc_keys if keys else K.alloc_values
        one = alloc(cfg, L * S, T, "cuda")
        (K.kivi_encode_k if keys else K.kivi_encode_v)(cfg, xd.reshape(L * S, T, D), T, *one)
        torch.cuda.synchronize()
        for i in range(3):
            assert torch.equal(torch.cat([lay[l][i] for l in range(L)]), one[i])


def test_full_model_boundary_shape():
    """A 32-layer model with its first and last two layers at 8 bits, at a
    reduced slice count (the oracle codes every layer)."""
    cfgs = _boundary_cfgs(32, 2, (2, 2), (8, 8))
    run_model(cfgs, S=2, T=160, n=160 - 128 + 5, seed=7)
