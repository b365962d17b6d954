"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
poisoned output buffers and compare with the CPU oracle element by element."""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import kv_cache_quantization_codec_amd as K
from oracle import attention_ref as att
from oracle import kivi_ref as ref

POISON32 = 0x5A5A5A5A                 # fits a signed int32
POISON16 = 0x5A5A                     # an ordinary fp16 value (203.25)
U_F32 = 2.0 ** -24                    # unit roundoff of fp32


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


def first_mismatch(name, got: np.ndarray, want: np.ndarray, offset=0):
    """None when equal, else a message naming the count and the first
    mismatching index (slice index shifted by ``offset``)."""
    if got.shape != want.shape:
        return f"{name}: shape {got.shape} != {want.shape}"
    bad = np.argwhere(got != want)
    if not bad.size:
        return None
    i = tuple(int(j) for j in bad[0])
    at = (i[0] + offset,) + i[1:]
    return f"{name}: {len(bad)} mismatches, first at {at}: got {got[i]:#x} want {want[i]:#x}"


def oracle_check_chunk(kind, x, codes, scale, zero, dec, n, bits, G, D, s0=0):
    """Oracle encode of fp16 ``x`` [s, T, D] (first n tokens) and decode of
    that encoding, compared bit for bit with a device run's host copies
    (codes as uint32, sidecars and decoded tokens as uint16 patterns).
    Returns the list of mismatch messages (empty when all agree)."""
    if kind == "k":
        oc, os_, oz = ref.encode_k(x, n, bits, G)
        od = ref.decode_k(oc, os_, oz, n, bits, G)
    else:
        oc, os_, oz = ref.encode_v(x, n, bits, G)
        od = ref.decode_v(oc, os_, oz, n, bits, G, D)
    side = "key" if kind == "k" else "value"
    msgs = [first_mismatch(f"{side} codes", codes, oc.view(np.uint32), s0),
            first_mismatch(f"{side} scale", scale, os_.view(np.uint16), s0),
            first_mismatch(f"{side} zero", zero, oz.view(np.uint16), s0),
            first_mismatch(f"{side} decode", dec, od.view(np.uint16), s0)]
    return [m for m in msgs if m]


def host_threads() -> int:
    """Worker threads for host-side oracle runs: the cores this process may
    use, at most 16 (numpy releases the GIL inside its array loops)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_check_slices(kind, cfg, x, payload, dec, n, s_begin, s_end, pool: ThreadPoolExecutor,
                        chunk: int):
    """Submits oracle checks of slices [s_begin, s_end) of a device run (fp16
    input ``x`` [S, T, D], payload (codes, scale, zero) for capacity n, decoded
    ``dec`` [S, >= n, D]) in chunks of ``chunk`` slices; copies that range to
    the host first.  Returns the futures (each yields a list of messages)."""
    bits = cfg.k_bits if kind == "k" else cfg.v_bits
    sl = slice(s_begin, s_end)
    xh = bits16(x[sl]).view(np.float16)
    ch, sh, zh = words(payload[0][sl]), bits16(payload[1][sl]), bits16(payload[2][sl])
    dh = bits16(dec[sl][:, :n])
    futs = []
    for c0 in range(0, s_end - s_begin, chunk):
        c = slice(c0, c0 + chunk)
        futs.append(pool.submit(oracle_check_chunk, kind, xh[c], ch[c], sh[c], zh[c], dh[c], n, bits,
                                cfg.group_size, cfg.head_dim, s_begin + c0))
    return futs


def attention_bound(q, kp, vp, n, res_k, res_v, kb, vb, G, sm_scale, want, n_splits):
    """Elementwise tolerance [S, r, D] of kivi_decode_attention against the
    float64 oracle ``want``, derived from the kernel's arithmetic (the
    derivation is the module docstring of tests/test_gpu_attention.py):
    per-token logit errors from the hi/lo fp16 split of q*scale (2^-21) and
    fp32 accumulation over D; exp2, online-rescale and merge errors; the
    weighted-mean perturbation bound; fp32 accumulation over T tokens of the
    value sums; one rounding of the output to fp16."""
    q64 = q.astype(np.float64)
    S, r, D = q.shape
    parts_a, parts_mv, parts_mvz = [], [], []
    if n:
        kd = att.dequantize_exact_k(*kp, n, kb, G)
        kz = np.asarray(kp[2]).astype(np.float64)[:, np.arange(n) // G, :]
        A = np.einsum("srd,std->srt", np.abs(q64), np.abs(kd) + 2 * np.abs(kz))
        vd = att.dequantize_exact_v(*vp, n, vb, G, D)
        vz = np.asarray(vp[2]).astype(np.float64)[:, :n, :][:, :, np.arange(D) // G]
        parts_a.append(A)
        parts_mv.append(np.abs(vd))
        parts_mvz.append(np.abs(vd) + 2 * np.abs(vz))
    if res_k.shape[1]:
        rk, rv = res_k.astype(np.float64), res_v.astype(np.float64)
        parts_a.append(np.einsum("srd,std->srt", np.abs(q64), np.abs(rk)))
        parts_mv.append(np.abs(rv))
        parts_mvz.append(np.abs(rv))
    A = np.concatenate(parts_a, axis=2)                     # [S, r, T]
    kk, _ = att.cache_tokens(kp, vp, n, res_k, res_v, kb, vb, G, D)
    logits = np.einsum("srd,std->srt", q64, kk) * sm_scale
    T = A.shape[2]
    delta = sm_scale * ((D + 2) * U_F32 + 2.0 ** -21) * A + 3 * U_F32 * np.abs(logits)
    spread = (logits.max(axis=2, keepdims=True) - logits) / np.log(2)
    eps = (delta.max(axis=2) + 2.0 ** -22 + U_F32 * spread.max(axis=2)
           + (-(-T // 32)) * 2.0 ** -21 + (n_splits + 2) * 2.0 ** -22)        # [S, r]
    mv = np.concatenate(parts_mv, axis=1).max(axis=1)       # [S, D]
    mvz = np.concatenate(parts_mvz, axis=1).max(axis=1)
    return (2.0 ** -11 * np.abs(want) + 2.0 ** -25
            + 2.1 * eps[:, :, None] * mv[:, None, :]
            + ((T + 8) * U_F32 + 2.0 ** -21) * mvz[:, None, :])
