"""The full-size workloads, in the launch configuration the benchmark times
(one kivi_encode_* / kivi_decode_* call over every slice of every layer),
checked on sampled slices against the oracle, plus size-independent
properties on every element."""

import sys

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


@pytest.mark.parametrize("name", ["llama2_7b_2bit", "mistral_7b_k2v4"])
def test_full_cache_sampled(name):
    w = WORKLOADS[name]
    cfg = K.Config(w.k_bits, w.v_bits, w.group_size, w.residual_length, w.head_dim)
    n = w.tokens - w.residual_length
    S = w.slices
    _log(f"{name}: generating S={S} T={w.tokens}")
    k, v = full_cache(w)
    _log(f"{name}: encode/decode n={n}")
    kq = U.gpu_encode("k", cfg, k, n)
    vq = U.gpu_encode("v", cfg, v, n)
    kd = U.gpu_decode("k", cfg, *kq, n, w.tokens)
    torch.cuda.synchronize()
    _log(f"{name}: bound check keys")
    _bound_check("k", cfg, k, kd, kq[1], n)
    picks = sample_slices(S, w.number)
    kh = U.bits16(k[picks]).view(F16)
    oc, os_, oz = ref.encode_k(kh, n, w.k_bits, w.group_size)
    U.assert_equal("key codes", U.words(kq[0][picks]), oc.view(np.uint32))
    U.assert_equal("key scale", U.bits16(kq[1][picks]), os_.view(np.uint16))
    U.assert_equal("key zero", U.bits16(kq[2][picks]), oz.view(np.uint16))
    od = ref.decode_k(oc, os_, oz, n, w.k_bits, w.group_size)
    U.assert_equal("key decode", U.bits16(kd[picks][:, :n]), od.view(np.uint16))
    assert U.is_poison(U.bits16(kd[picks][:, n:]))
    del kd
    vd = U.gpu_decode("v", cfg, *vq, n, w.tokens)
    torch.cuda.synchronize()
    _log(f"{name}: bound check values")
    _bound_check("v", cfg, v, vd, vq[1], n)
    vh = U.bits16(v[picks]).view(F16)
    pc, ps, pz = ref.encode_v(vh, n, w.v_bits, w.group_size)
    U.assert_equal("value codes", U.words(vq[0][picks]), pc.view(np.uint32))
    U.assert_equal("value scale", U.bits16(vq[1][picks]), ps.view(np.uint16))
    U.assert_equal("value zero", U.bits16(vq[2][picks]), pz.view(np.uint16))
    pd = ref.decode_v(pc, ps, pz, n, w.v_bits, w.group_size, w.head_dim)
    U.assert_equal("value decode", U.bits16(vd[picks][:, :n]), pd.view(np.uint16))
    _log(f"{name}: sampled slices {picks} bit-exact")


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
