"""The binding rejects tensors that do not fit the C layouts before it calls
the library: host tensors, wrong dtypes, non-contiguous payloads, payloads
smaller than the layout of the call's slices and capacity, inputs with
fewer tokens than the call reads.  A kernel handed such a buffer would read
or write out of bounds, so these checks stand between Python and the GPU.

Runs without a GPU.  The library is replaced by a guard that serves only
the host-side sizing entry points and fails the test if any compute entry
point is reached.  Host tensors are first rejected as such; then, with the
device check widened to accept them, the size and layout checks are
exercised on host tensors standing in for device ones."""

from __future__ import annotations

import pytest
import torch

K = pytest.importorskip("kv_cache_quantization_codec_amd")
B = K.binding

HOST_SIDE = ("kivi_k_code_words", "kivi_k_stat_elems", "kivi_v_code_words", "kivi_v_stat_elems",
             "kivi_ring_elems", "kivi_status_string", "kivi_attention_workspace_bytes")


class _Guard:
    def __init__(self, real):
        self.real = real

    def __getattr__(self, name):
        if name in HOST_SIDE:
            return getattr(self.real, name)
        raise AssertionError(f"{name} was called: the binding must reject the arguments first")


@pytest.fixture
def guarded(monkeypatch):
    real = B.lib()
    monkeypatch.setattr(B, "lib", lambda: _Guard(real))


@pytest.fixture
def host_as_device(guarded, monkeypatch):
    """The device check accepts host tensors (all on one device), so that the
    remaining checks can be exercised without a GPU."""
    def on_device(t, what, device=None):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{what}: expected a torch tensor")
        if device is not None and t.device != device:
            raise ValueError(f"{what}: other device")
        return t.device
    monkeypatch.setattr(B, "_on_device", on_device)


CFG = K.Config(2, 4, 32, 128, 128)
S, T, N, D = 3, 100, 70, 128


def _fp16(*shape):
    return torch.zeros(shape, dtype=torch.float16)


def _keys(cap=N, short=None):
    words = B.kivi_k_code_words(CFG, cap)
    stats = B.kivi_k_stat_elems(CFG, cap)
    c = torch.zeros(S * words - (1 if short == "codes" else 0), dtype=torch.int32)
    s = torch.zeros(S * stats - (1 if short == "scale" else 0), dtype=torch.float16)
    z = torch.zeros(S * stats - (1 if short == "zero" else 0), dtype=torch.float16)
    return c, s, z


def _values(cap=N, short=None):
    words = B.kivi_v_code_words(CFG, cap)
    stats = B.kivi_v_stat_elems(CFG, cap)
    c = torch.zeros(S * words - (1 if short == "codes" else 0), dtype=torch.int32)
    s = torch.zeros(S * stats - (1 if short == "scale" else 0), dtype=torch.float16)
    z = torch.zeros(S * stats - (1 if short == "zero" else 0), dtype=torch.float16)
    return c, s, z


# ---- host tensors never reach the library ----

def test_host_tensors_are_rejected(guarded):
    x = _fp16(S, T, D)
    with pytest.raises(ValueError, match="GPU tensor"):
        K.kivi_encode_k(CFG, x, N, *_keys())
    with pytest.raises(ValueError, match="GPU tensor"):
        K.kivi_encode_v(CFG, x, N, *_values())
    with pytest.raises(ValueError, match="GPU tensor"):
        K.kivi_decode_k(CFG, *_keys(), N, x)
    with pytest.raises(ValueError, match="GPU tensor"):
        K.kivi_decode_v(CFG, *_values(), N, x)
    with pytest.raises(ValueError, match="GPU tensor"):
        K.kivi_fp8_encode(x, N, torch.zeros((S, T, D), dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU tensor"):
        K.kivi_encode_k_layers([CFG] * 2, _fp16(2, S, T, D), N, [_keys(), _keys()])
    with pytest.raises(ValueError, match="GPU tensor"):
        K.AttnCache(CFG, _keys(), (torch.zeros((S, N, 8), dtype=torch.int32), _fp16(S, N, 4),
                                   _fp16(S, N, 4)), N)


# ---- sizes, dtypes and layouts (host tensors standing in for device ones) ----

@pytest.mark.parametrize("short", ["codes", "scale", "zero"])
def test_short_payloads_are_rejected(host_as_device, short):
    x = _fp16(S, T, D)
    for call in (lambda: K.kivi_encode_k(CFG, x, N, *_keys(short=short)),
                 lambda: K.kivi_decode_k(CFG, *_keys(short=short), N, x),
                 lambda: K.kivi_encode_v(CFG, x, N, *_values(short=short)),
                 lambda: K.kivi_decode_v(CFG, *_values(short=short), N, x)):
        with pytest.raises(ValueError, match=short):
            call()


def test_payload_for_a_smaller_capacity_is_rejected(host_as_device):
    x = _fp16(S, T, D)
    with pytest.raises(ValueError, match="codes"):
        K.kivi_encode_k(CFG, x, N, *_keys(cap=N - 32), cap_tokens=N)
    with pytest.raises(ValueError, match="codes"):
        K.kivi_encode_v(CFG, x, N, *_values(cap=N), cap_tokens=N + 1)


def test_payload_for_fewer_bits_is_rejected(host_as_device):
    x = _fp16(S, T, D)
    kc, ks, kz = _keys()                               # sized for 2-bit keys
    with pytest.raises(ValueError, match="codes"):
        K.kivi_encode_k(K.Config(4, 4, 32, 128, 128), x, N, kc, ks, kz)


def test_wrong_dtypes_and_layouts_are_rejected(host_as_device):
    x = _fp16(S, T, D)
    kc, ks, kz = _keys()
    with pytest.raises(ValueError, match="codes"):
        K.kivi_encode_k(CFG, x, N, kc.to(torch.int64), ks, kz)
    with pytest.raises(ValueError, match="scale"):
        K.kivi_encode_k(CFG, x, N, kc, ks.to(torch.float32), kz)
    wide = torch.zeros(2 * kc.numel(), dtype=torch.int32)[::2]    # strided, large enough
    with pytest.raises(ValueError, match="contiguous"):
        K.kivi_encode_k(CFG, x, N, wide, ks, kz)
    with pytest.raises(ValueError, match="float16"):
        K.kivi_encode_k(CFG, x.float(), N, kc, ks, kz)
    with pytest.raises(ValueError, match="tensor"):
        K.kivi_encode_k(CFG, x, N, kc, ks, None)


def test_inputs_and_outputs_must_hold_the_tokens(host_as_device):
    short = _fp16(S, N - 1, D)
    with pytest.raises(ValueError, match="tokens per slice"):
        K.kivi_encode_k(CFG, short, N, *_keys())
    with pytest.raises(ValueError, match="tokens per slice"):
        K.kivi_decode_v(CFG, *_values(), N, short)
    with pytest.raises(ValueError, match="tokens per slice"):
        K.kivi_fp8_encode(_fp16(S, T, D), T, torch.zeros((S, T - 1, D), dtype=torch.uint8))


def test_layer_payloads_are_checked_per_layer(host_as_device):
    x = _fp16(2, S, T, D)
    with pytest.raises(ValueError, match="layer 1"):
        K.kivi_encode_k_layers([CFG, CFG], x, N, [_keys(), _keys(short="zero")])
    with pytest.raises(ValueError, match="payloads"):
        K.kivi_encode_v_layers([CFG, CFG], x, N, [_values()])
    with pytest.raises(ValueError, match="tokens per slice"):
        K.kivi_decode_k_layers([CFG, CFG], [_keys(), _keys()], T + 1, x)


def test_attention_cache_and_queries_are_checked(host_as_device):
    vals = tuple(t.view(S, N, -1) for t in _values())
    keys = tuple(t.view(S, -1, D) for t in _keys())
    short = torch.zeros((S, keys[0].shape[1] - 1, D), dtype=torch.int32)
    with pytest.raises(ValueError, match="codes"):
        K.AttnCache(CFG, (short,) + keys[1:], vals, N)
    with pytest.raises(ValueError, match="slice count"):
        K.AttnCache(CFG, keys, tuple(t[:2] for t in vals), N)
    cache = K.AttnCache(CFG, keys, vals, N)
    q = _fp16(S, 2, D)
    with pytest.raises(ValueError, match="slices"):
        K.kivi_decode_attention(CFG, cache, _fp16(S + 1, 2, D), 0.1, _fp16(S + 1, 2, D))
    with pytest.raises(ValueError, match="shape"):
        K.kivi_decode_attention_noalloc(CFG, cache, q, 0.1, _fp16(S, 1, D))
    with pytest.raises(ValueError, match="res_k"):
        K.AttnCache(CFG, keys, vals, N, _fp16(S + 1, 8, D), _fp16(S + 1, 8, D))


def test_sizes_come_from_the_library():
    """alloc_* shape the payloads by the library's sizing entry points."""
    for cfg in (K.Config(2, 4, 32, 128, 128), K.Config(8, 2, 128, 0, 96), K.Config(4, 8, 64, 16, 64)):
        for cap in (0, 1, 31, 64, 1000):
            kc, ks, kz = K.alloc_keys(cfg, 2, cap, "cpu")
            vc, vs, vz = K.alloc_values(cfg, 2, cap, "cpu")
            assert kc.numel() == 2 * K.kivi_k_code_words(cfg, cap)
            assert ks.numel() == kz.numel() == 2 * K.kivi_k_stat_elems(cfg, cap)
            assert vc.numel() == 2 * K.kivi_v_code_words(cfg, cap)
            assert vs.numel() == vz.numel() == 2 * K.kivi_v_stat_elems(cfg, cap)
            assert kc.shape[2] == cfg.head_dim and vc.shape[1] == cap


def test_binding_holds_no_layout_formulas():
    """Group counts and words per group come from the library, not from
    arithmetic in the binding."""
    import inspect
    src = inspect.getsource(B)
    for pattern in ("// G", "// cfg.group_size", "* cfg.k_bits", "* cfg.v_bits", "G * b // 32"):
        assert pattern not in src, pattern
