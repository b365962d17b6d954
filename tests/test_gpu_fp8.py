"""GPU parity of the FP8 key cast (and the k8v4 layout built from it) with
the oracle, bit for bit, through the C ABI."""

import numpy as np
import pytest
import torch

import kv_cache_quantization_codec_amd as K
from oracle import fp8_ref as f8
from oracle import kivi_ref as ref

pytestmark = pytest.mark.gpu

F16 = np.float16


def _dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.float16).cuda()


def test_every_finite_fp16_value():
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = allh[np.isfinite(allh.view(F16))].view(F16)              # 63,488 finite patterns
    x = x[: x.size // 8 * 8].reshape(1, -1, 8)
    codes = torch.full(x.shape, 0xA5, dtype=torch.uint8, device="cuda")
    K.kivi_fp8_encode(_dev16(x), x.shape[1], codes)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), f8.encode(x))


def test_every_code_decodes():
    c = np.arange(256, dtype=np.uint8).reshape(1, 32, 8)
    out = torch.empty((1, 32, 8), dtype=torch.float16, device="cuda")
    K.kivi_fp8_decode(torch.from_numpy(c).cuda(), 32, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    want = f8.decode(c).view(np.uint16)
    finite = (c & 0x7F) != 0x7F
    assert np.array_equal(got[finite], want[finite])
    assert np.all(np.isnan(out.cpu().numpy()[~finite]))


@pytest.mark.parametrize("S,T,n,D", [(3, 100, 77, 128), (2, 40, 40, 64), (5, 33, 1, 96), (1, 9, 9, 8)])
def test_strided_keys_round_trip(S, T, n, D):
    rng = np.random.default_rng(S * T + D)
    k = (rng.standard_normal((S, T + 7, D)) * rng.choice([0.01, 1.0, 60.0, 600.0], (S, 1, D))).astype(F16)
    kd = _dev16(k)[:, :T]                                        # slice stride (T + 7) * D
    codes = torch.full((S, T + 3, D), 0xA5, dtype=torch.uint8, device="cuda")
    K.kivi_fp8_encode(kd, n, codes)
    out = torch.full((S, T + 5, D), float("nan"), dtype=torch.float16, device="cuda")
    K.kivi_fp8_decode(codes, n, out)
    torch.cuda.synchronize()
    c = codes.cpu().numpy()
    assert np.array_equal(c[:, :n], f8.encode_keys(k, n))
    assert np.all(c[:, n:] == 0xA5), "wrote past n_tokens"
    o = out.cpu().numpy()
    assert np.array_equal(o[:, :n].view(np.uint16), f8.decode(f8.encode_keys(k, n)).view(np.uint16))
    assert np.all(np.isnan(o[:, n:]))


def test_k8v4_layout():
    """FP8 keys plus 4-bit values with one group per head (the k8v4 layout)."""
    S, T, D = 4, 300, 128
    rng = np.random.default_rng(7)
    k = rng.standard_normal((S, T, D)).astype(F16)
    v = rng.standard_normal((S, T, D)).astype(F16)
    cfg = K.Config(8, 4, 128, 0, D)
    codes = torch.empty((S, T, D), dtype=torch.uint8, device="cuda")
    K.kivi_fp8_encode(_dev16(k), T, codes)
    vc, vs, vz = K.alloc_values(cfg, S, T, "cuda")
    K.kivi_encode_v(cfg, _dev16(v), T, vc, vs, vz)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), f8.encode_keys(k, T))
    oc, os_, oz = ref.encode_v(v, T, 4, 128)
    assert np.array_equal(vc.cpu().numpy().view(np.uint32), oc.view(np.uint32))
    assert np.array_equal(vs.cpu().numpy().view(np.uint16), os_.view(np.uint16))
    assert np.array_equal(vz.cpu().numpy().view(np.uint16), oz.view(np.uint16))
    # bytes per token and head: D for the keys, D*4/8 + 4 for the values
    assert codes[0, 0].numel() == D
    assert vc[0, 0].numel() * 4 + 2 + 2 == D * 4 // 8 + 4
