"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
poisoned output buffers and compare with the CPU oracle element by element."""

from __future__ import annotations

import numpy as np
import torch

import kv_cache_quantization_codec_amd as K
from oracle import kivi_ref as ref

POISON32 = 0x5A5A5A5A                 # fits a signed int32
POISON16 = 0x5A5A                     # an ordinary fp16 value (203.25)


def poisoned(t: torch.Tensor) -> torch.Tensor:
    if t.dtype == torch.int32:
        t.fill_(POISON32)
    else:
        t.view(torch.int16).fill_(POISON16)
    return t


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def words(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.uint32)


def is_poison(a: np.ndarray) -> bool:
    if a.dtype == np.uint32:
        return bool(np.all(a == np.uint32(POISON32 & 0xFFFFFFFF)))
    return bool(np.all(a == np.uint16(POISON16)))


def ring_residual(st):
    """Residual K and V tokens of a ``K.Stream`` in age order, fp16 [S, count, D]
    copies: residual token i sits in ring slot (ring_head + i) mod slots."""
    slots = st.k_ring.shape[1]
    idx = [(st.ring_head + i) % slots for i in range(st.ring_count)]
    return st.k_ring[:, idx], st.v_ring[:, idx]


def assert_equal(name, got: np.ndarray, want: np.ndarray):
    if got.shape != want.shape:
        raise AssertionError(f"{name}: shape {got.shape} != {want.shape}")
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} mismatches, first at {i}: "
                             f"got {got[i]:#x} want {want[i]:#x}")


def gpu_encode(kind, cfg, x_gpu, n, cap=None):
    """Encode with poisoned outputs of capacity ``cap``; returns (codes, scale, zero) tensors."""
    S = x_gpu.shape[0]
    cap = n if cap is None else cap
    alloc = K.alloc_keys if kind == "k" else K.alloc_values
    codes, scale, zero = (poisoned(t) for t in alloc(cfg, S, cap, x_gpu.device))
    fn = K.kivi_encode_k if kind == "k" else K.kivi_encode_v
    fn(cfg, x_gpu, n, codes, scale, zero, cap_tokens=cap)
    return codes, scale, zero


def gpu_decode(kind, cfg, codes, scale, zero, n, T_out, cap=None):
    S = codes.shape[0]
    out = poisoned(torch.empty((S, T_out, cfg.head_dim), dtype=torch.float16, device=codes.device))
    fn = K.kivi_decode_k if kind == "k" else K.kivi_decode_v
    fn(cfg, codes, scale, zero, n, out, cap_tokens=cap)
    return out


def check_round_trip(kind, cfg, x_host: np.ndarray, n: int, *, cap=None, extra_tokens=0,
                     device="cuda"):
    """Encode + decode ``x_host`` [S, T, D] (fp16) on the GPU; compare codes,
    sidecars and decoded values bit for bit with the oracle, and check that
    nothing outside the valid region was written."""
    S, T, D = x_host.shape
    G = cfg.group_size
    b = cfg.k_bits if kind == "k" else cfg.v_bits
    # input with padded slices: T + extra_tokens rows allocated per slice
    buf = torch.empty((S, T + extra_tokens, D), dtype=torch.float16)
    buf[:, :T] = torch.from_numpy(x_host.view(np.int16)).view(torch.float16)
    x_gpu = buf.to(device)[:, :T]
    cap_ = n if cap is None else cap
    codes, scale, zero = gpu_encode(kind, cfg, x_gpu, n, cap_)
    enc = ref.encode_k if kind == "k" else ref.encode_v
    oc, os_, oz = enc(x_host, n, b, G)
    gc, gs, gz = words(codes), bits16(scale), bits16(zero)
    if kind == "k":
        ng = ref.n_groups(n, G)
        W = G * b // 32
        assert_equal("key codes", gc[:, :ng * W], oc.view(np.uint32))
        assert_equal("key scale", gs[:, :ng], os_.view(np.uint16))
        assert_equal("key zero", gz[:, :ng], oz.view(np.uint16))
        assert is_poison(gc[:, ng * W:]) and is_poison(gs[:, ng:]) and is_poison(gz[:, ng:])
    else:
        assert_equal("value codes", gc[:, :n], oc.view(np.uint32))
        assert_equal("value scale", gs[:, :n], os_.view(np.uint16))
        assert_equal("value zero", gz[:, :n], oz.view(np.uint16))
        assert is_poison(gc[:, n:]) and is_poison(gs[:, n:]) and is_poison(gz[:, n:])
    # the input is read-only
    assert np.array_equal(bits16(x_gpu), x_host.view(np.uint16))
    out = gpu_decode(kind, cfg, codes, scale, zero, n, T + 3, cap_)
    if kind == "k":
        od = ref.decode_k(oc, os_, oz, n, b, G)
    else:
        od = ref.decode_v(oc, os_, oz, n, b, G, D)
    go = bits16(out)
    assert_equal("decoded", go[:, :n], od.view(np.uint16))
    assert is_poison(go[:, n:]), "decode wrote beyond n_tokens"
    return oc, os_, oz
