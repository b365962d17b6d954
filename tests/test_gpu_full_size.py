"""The full-size workloads, in the launch configuration the benchmark times
(one kivi_encode_* / kivi_decode_* call over every slice of every layer).
The two model-shaped caches are compared with the oracle on every slice,
bit for bit; the others on sampled slices; size-independent properties are
checked on every element."""

import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from kvsynth import WORKLOADS, layer_kv, stream_tokens  # noqa: E402
from oracle import kivi_ref as ref  # noqa: E402
from tests import gpu_util as U  # noqa: E402
from tests.test_gpu_stream import compare_stream  # noqa: E402

import kv_cache_quantization_codec_amd as K  # noqa: E402

F16 = np.float16


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def full_cache(w, tokens=None):
    """K and V of all layers as one [L*B*H, T, D] fp16 tensor each, on the GPU."""
    T = w.tokens if tokens is None else tokens
    S = w.slices
    k = torch.empty((S, T, w.head_dim), dtype=torch.float16, device="cuda")
    v = torch.empty_like(k)
    spl = w.slices_per_layer
    for layer in range(w.layers):
        kl, vl = layer_kv(w, layer, device="cuda", tokens=T)
        k[layer * spl:(layer + 1) * spl] = kl
        v[layer * spl:(layer + 1) * spl] = vl
        del kl, vl
    return k, v


def sample_slices(S, seed):
    rng = np.random.default_rng(seed)
    return sorted({0, 1, S // 2, S - 1, *rng.integers(0, S, 4).tolist()})


def _bound_check(kind, cfg, x, xhat, scale, n):
    """|x - xhat| <= scale/2 + ulp16 for every element of normal-scale groups."""
    G = cfg.group_size
    for s0 in range(0, x.shape[0], 256):
        xs = x[s0:s0 + 256, :n].float()
        xh = xhat[s0:s0 + 256, :n].float()
        if kind == "k":
            sc = scale[s0:s0 + 256].float().repeat_interleave(G, dim=1)[:, :n]
        else:
            sc = scale[s0:s0 + 256, :n].float().repeat_interleave(G, dim=2)[:, :, :cfg.head_dim]
        mag = torch.maximum(xs.abs(), xh.abs()).clamp_min(2.0 ** -14)
        ulp = torch.exp2(torch.floor(torch.log2(mag)) - 10)
        ok = (xs - xh).abs() <= sc * (0.5 + 2.0 ** -14) + ulp
        ok |= sc < 2.0 ** -14
        assert bool(ok.all()), f"error bound violated in slices {s0}..{s0 + 256}"


MODEL_CACHES = ["llama2_7b_2bit", "mistral_7b_k2v4"]
LAYER_RANGES = [(0, 8), (8, 16), (16, 24), (24, 32)]


@pytest.fixture(scope="module")
def coded():
    """Lazily built per workload and kept for the module: the whole cache
    generated on the device and coded in the benchmark's launch configuration
    (one kivi_encode_k / kivi_encode_v / kivi_decode_k / kivi_decode_v call
    over every slice of every layer) into poisoned buffers.  Both model
    caches together hold about 115 GB of device memory."""
    made = {}

    def get(name):
        if name not in made:
            w = WORKLOADS[name]
            cfg = K.Config(w.k_bits, w.v_bits, w.group_size, w.residual_length, w.head_dim)
            n = w.tokens - w.residual_length
            _log(f"{name}: generating S={w.slices} T={w.tokens}, coding n={n}")
            k, v = full_cache(w)
            kq = U.gpu_encode("k", cfg, k, n)
            vq = U.gpu_encode("v", cfg, v, n)
            kd = U.gpu_decode("k", cfg, *kq, n, w.tokens)
            vd = U.gpu_decode("v", cfg, *vq, n, w.tokens)
            torch.cuda.synchronize()
            made[name] = dict(w=w, cfg=cfg, n=n, k=k, v=v, kq=kq, vq=vq, kd=kd, vd=vd)
        return made[name]

    yield get
    made.clear()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", MODEL_CACHES)
@pytest.mark.parametrize("layers", LAYER_RANGES, ids=lambda r: f"layers{r[0]}-{r[1] - 1}")
def test_every_slice_bit_exact(coded, name, layers):
    """Every slice of the layers in range, keys and values: codes, scale and
    zero words equal the oracle's encoding, and the decoded tokens its
    decoding, bit for bit.  Each layer is copied to the host in turn and
    checked in chunks of slices on a thread pool (the oracle is numpy, whose
    array loops run without the GIL) while the next layer is copied."""
    c = coded(name)
    w, cfg, n = c["w"], c["cfg"], c["n"]
    spl = w.slices_per_layer
    chunk = max(1, spl // 16)
    l0, l1 = layers
    t0 = time.perf_counter()
    problems, pending = [], []
    with ThreadPoolExecutor(U.host_threads()) as pool:
        for layer in range(l0, l1):
            s0, s1 = layer * spl, (layer + 1) * spl
            futs = (U.oracle_check_slices("k", cfg, c["k"], c["kq"], c["kd"], n, s0, s1, pool, chunk)
                    + U.oracle_check_slices("v", cfg, c["v"], c["vq"], c["vd"], n, s0, s1, pool, chunk))
            pending.append((layer, futs))
            while len(pending) > 2:             # at most three layers' host copies alive
                lay, fs = pending.pop(0)
                problems += [f"layer {lay}: {m}" for f in fs for m in f.result()]
        for lay, fs in pending:
            problems += [f"layer {lay}: {m}" for f in fs for m in f.result()]
    assert not problems, "\n".join(problems[:20])
    _log(f"{name}: layers {l0}-{l1 - 1}, slices {l0 * spl}..{l1 * spl - 1}: keys and values bit-exact "
         f"({time.perf_counter() - t0:.1f} s, {U.host_threads()} threads)")


@pytest.mark.parametrize("name", MODEL_CACHES)
def test_error_bound_and_bounds_every_element(coded, name):
    """Properties that hold at any size, on every element of the cache:
    |x - xhat| <= scale/2 + ulp16(x) for normal-scale groups, and the
    decoders write nothing past the n quantized tokens of a slice."""
    c = coded(name)
    cfg, n, w = c["cfg"], c["n"], c["w"]
    _bound_check("k", cfg, c["k"], c["kd"], c["kq"][1], n)
    _bound_check("v", cfg, c["v"], c["vd"], c["vq"][1], n)
    for dec in (c["kd"], c["vd"]):
        assert bool((dec[:, n:].view(torch.int16) == U.POISON16).all()), "decode wrote past n_tokens"
    _log(f"{name}: error bound holds on all {2 * w.slices * n * w.head_dim} elements")


def test_stream_batch64_full_size_sampled():
    w = WORKLOADS["stream_b64"]
    cfg = K.Config(w.k_bits, w.v_bits, w.group_size, w.residual_length, w.head_dim)
    S, G = w.slices, w.group_size
    _log(f"stream: generating S={S} prefill {w.tokens}, {w.steps} steps")
    k, v = full_cache(w)
    kn, vn = stream_tokens(w, w.steps, device="cuda")
    cap = w.tokens + w.steps
    st = K.Stream(cfg, S, cap)
    for t in (*st.keys, *st.values):
        U.poisoned(t)
    K.kivi_stream_prefill(st, k, v, w.tokens)
    assert (st.n_quant, st.ring_count) == (1920, 128)
    flushes = []
    for i in range(w.steps):
        if K.kivi_append_flush(st, kn[i], vn[i]):
            flushes.append(i)
    torch.cuda.synchronize()
    assert flushes == list(range(0, 512, 32)) and st.n_quant == 2432 and st.ring_count == 128
    picks = sample_slices(S, 4)
    _log(f"stream: oracle on slices {picks}")
    sr = ref.StreamRef(w.k_bits, w.v_bits, G, w.residual_length)
    sr.prefill(U.bits16(k[picks]).view(F16), U.bits16(v[picks]).view(F16), w.tokens)
    knh = U.bits16(kn[:, picks]).view(F16)
    vnh = U.bits16(vn[:, picks]).view(F16)
    for i in range(w.steps):
        sr.append(knh[i], vnh[i])
    compare_stream(st, sr, slices=picks)


# ---- next rows at their full sizes ------------------------------------------

@pytest.mark.parametrize("name", MODEL_CACHES)
def test_attention_full_size_sampled(coded, name):
    """Decode attention over the whole cache in one call (the split plan the
    benchmark times).  Sampled slices: the oracle's attention over the
    oracle's own encoding of those slices, within the derived tolerance.
    Every slice: outputs are finite and lie within the range of the slice's
    values widened by half a quantization step (a weighted mean of
    dequantized values cannot leave it)."""
    from kvsynth import decode_queries
    from oracle import attention_ref as att
    from tests.gpu_util import attention_bound as _bound

    c = coded(name)
    w, cfg, k, v, kq, vq = c["w"], c["cfg"], c["k"], c["v"], c["kq"], c["vq"]
    n, R, S, D, G = w.tokens - w.residual_length, w.residual_length, w.slices, w.head_dim, w.group_size
    q = decode_queries(w, "cuda")
    out = torch.full_like(q, float("nan"))
    sm_scale = D ** -0.5
    cache = K.AttnCache(cfg, kq, vq, n, k[:, n:], v[:, n:], 0, R)
    ws = K.kivi_attention_workspace_bytes(cfg, S, w.q_per_kv, n, R)
    n_splits = max(1, ws // (S * w.q_per_kv * (D + 2) * 4))
    _log(f"{name} attention: one call, {n_splits} splits per slice")
    K.kivi_decode_attention(cfg, cache, q, sm_scale, out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    # every slice: within [min v - step/2, max v + step/2] per channel
    b = w.v_bits
    for s0 in range(0, S, 512):
        vs = v[s0:s0 + 512].float()
        lo, hi = vs.min(dim=1).values, vs.max(dim=1).values                    # [s, D]
        step = (vs.amax(dim=(1, 2)) - vs.amin(dim=(1, 2))) / (2 ** b - 1)      # [s]
        pad = (0.5 * step * 1.01)[:, None, None] + 2.0 ** -10 * torch.maximum(lo.abs(), hi.abs())[:, None, :]
        o = out[s0:s0 + 512].float()
        assert bool((o >= lo[:, None, :] - pad).all() and (o <= hi[:, None, :] + pad).all()), \
            f"slices {s0}..{s0 + 512}: output outside the value range"
    picks = sample_slices(S, w.number + 100)
    _log(f"{name} attention: oracle on slices {picks}")
    kh, vh = U.bits16(k[picks]).view(F16), U.bits16(v[picks]).view(F16)
    kp = ref.encode_k(kh, n, w.k_bits, G)
    vp = ref.encode_v(vh, n, w.v_bits, G)
    qh = U.bits16(q[picks]).view(F16)
    want = att.decode_attention(qh, kp, vp, n, kh[:, n:], vh[:, n:], w.k_bits, w.v_bits, G, sm_scale)
    tol = _bound(qh, kp, vp, n, kh[:, n:], vh[:, n:], w.k_bits, w.v_bits, G, sm_scale, want, n_splits)
    got = out[picks].float().cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    assert np.all(err <= tol), f"max err/tol {np.max(err / tol):.3g}"
    _log(f"{name} attention: max err/tol {np.max(err / tol):.3g}")


def test_k8v4_full_size_sampled():
    """FP8 keys and one-group 4-bit values of the whole Llama-shaped cache in
    the benchmark's launches; sampled slices bit-exact against the oracle."""
    from oracle import fp8_ref as f8

    w = WORKLOADS["llama2_7b_k8v4"]
    cfg = K.Config(w.k_bits, w.v_bits, w.group_size, w.residual_length, w.head_dim)
    n, S, D = w.tokens - w.residual_length, w.slices, w.head_dim
    _log(f"k8v4: generating S={S} T={w.tokens}")
    k, v = full_cache(w)
    kq = torch.full((S, n, D), 0x5A, dtype=torch.uint8, device="cuda")
    K.kivi_fp8_encode(k, n, kq)
    kd = U.poisoned(torch.empty((S, n + 2, D), dtype=torch.float16, device="cuda"))
    K.kivi_fp8_decode(kq, n, kd)
    vq = U.gpu_encode("v", cfg, v, n)
    torch.cuda.synchronize()
    picks = sample_slices(S, 55)
    _log(f"k8v4: oracle on slices {picks}")
    kh = U.bits16(k[picks]).view(F16)
    want = f8.encode_keys(kh, n)
    assert np.array_equal(kq[picks].cpu().numpy(), want)
    assert np.array_equal(U.bits16(kd[picks][:, :n]), f8.decode(want).view(np.uint16))
    assert U.is_poison(U.bits16(kd[picks][:, n:]))
    vh = U.bits16(v[picks]).view(F16)
    pc, ps, pz = ref.encode_v(vh, n, w.v_bits, w.group_size)
    U.assert_equal("value codes", U.words(vq[0][picks]), pc.view(np.uint32))
    U.assert_equal("value scale", U.bits16(vq[1][picks]), ps.view(np.uint16))
    U.assert_equal("value zero", U.bits16(vq[2][picks]), pz.view(np.uint16))


def test_layer_mix_full_size_sampled():
    """The 32-layer mix (first and last two layers at 8/8 bits) coded by the
    layer-wise calls in the benchmark's layout; sampled slices of every
    layer bit-exact against the oracle at that layer's bits."""
    from oracle import layer_mix_ref as mix

    w = WORKLOADS["llama2_7b_mix"]
    n, spl, T, D, G = w.tokens - w.residual_length, w.slices_per_layer, w.tokens, w.head_dim, w.group_size
    bits = mix.layer_bits(w.layers, w.boundary, (w.k_bits, w.v_bits), w.boundary_bits)
    cfgs = [K.Config(kb, vb, G, w.residual_length, D) for kb, vb in bits]
    _log(f"mix: generating {w.layers} layers x {spl} slices, T={T}")
    k, v = full_cache(w)
    for keys, x in ((True, k), (False, v)):
        lay = K.alloc_layers(cfgs, spl, n, "cuda", keys=keys)
        (K.kivi_encode_k_layers if keys else K.kivi_encode_v_layers)(cfgs, x.view(w.layers, spl, T, D), n, lay)
        torch.cuda.synchronize()
        rng = np.random.default_rng(7 if keys else 8)
        for l in range(w.layers):
            picks = sorted({0, spl - 1, int(rng.integers(0, spl))})
            xh = U.bits16(x[l * spl:(l + 1) * spl][picks]).view(F16)
            b = bits[l][0 if keys else 1]
            oc, os_, oz = (ref.encode_k if keys else ref.encode_v)(xh, n, b, G)
            side = "key" if keys else "value"
            U.assert_equal(f"layer {l} {side} codes", U.words(lay[l][0][picks]), oc.view(np.uint32))
            U.assert_equal(f"layer {l} {side} scale", U.bits16(lay[l][1][picks]), os_.view(np.uint16))
            U.assert_equal(f"layer {l} {side} zero", U.bits16(lay[l][2][picks]), oz.view(np.uint16))
        del lay
