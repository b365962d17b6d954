"""Thin Python binding over libkivi's C ABI (``include/kivi.h``).

Argument marshalling only: every function takes torch tensors that live on
the GPU, checks that they are device tensors of the expected dtype, layout
and size (sizes from the library's own sizing entry points), and passes
``data_ptr()`` values plus torch's current HIP stream to the entry point of
the same name.  A tensor that fails a check raises ``ValueError`` before
the library is called, so no kernel ever sees a host pointer or a buffer
smaller than its layout.  All codec work runs in the library's HIP kernels;
there is no fallback of any kind -- importing this module fails loudly when
``libkivi.so`` has not been built.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkivi.so")

KIVI_OK = 0
STATUS_NAMES = {
    0: "KIVI_OK", -1: "KIVI_E_NULL", -2: "KIVI_E_BITS", -3: "KIVI_E_GROUP",
    -4: "KIVI_E_HEAD_DIM", -5: "KIVI_E_RESIDUAL", -6: "KIVI_E_SHAPE", -7: "KIVI_E_ALIGN",
    -8: "KIVI_E_CAPACITY", -9: "KIVI_E_STATE", -10: "KIVI_E_HIP", -11: "KIVI_E_SCRATCH",
}

# bytes of the library's static attention scratch per device (KIVI_ATTENTION_SCRATCH_BYTES)
ATTENTION_SCRATCH_BYTES = 128 << 20


class KiviError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().kivi_status_string(status).decode()} ({status})")


class kivi_config(ctypes.Structure):
    _fields_ = [("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("residual_length", ctypes.c_int32),
                ("head_dim", ctypes.c_int32)]


class kivi_stream(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("k_zero", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("v_zero", ctypes.c_void_p),
                ("k_ring", ctypes.c_void_p), ("v_ring", ctypes.c_void_p),
                ("n_slices", ctypes.c_int64), ("cap_tokens", ctypes.c_int64),
                ("n_quant", ctypes.c_int64), ("ring_head", ctypes.c_int64),
                ("ring_count", ctypes.c_int64)]


class kivi_attn_cache(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("k_zero", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("v_zero", ctypes.c_void_p),
                ("cap_tokens", ctypes.c_int64), ("n_quant", ctypes.c_int64),
                ("res_k", ctypes.c_void_p), ("res_v", ctypes.c_void_p),
                ("res_slice_stride", ctypes.c_int64), ("res_slots", ctypes.c_int64),
                ("res_head", ctypes.c_int64), ("res_count", ctypes.c_int64),
                ("n_quant_per_slice", ctypes.c_void_p), ("res_count_per_slice", ctypes.c_void_p)]


# (name, restype, argtypes) of every symbol include/kivi.h declares
_P, _I64, _I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_CFG = ctypes.POINTER(kivi_config)
_ST = ctypes.POINTER(kivi_stream)
_AC = ctypes.POINTER(kivi_attn_cache)
SIGNATURES = [
    ("kivi_status_string", ctypes.c_char_p, [_I32]),
    ("kivi_last_hip_error", _I32, []),
    ("kivi_validate_config", _I32, [_CFG]),
    ("kivi_k_code_words", _I64, [_CFG, _I64]),
    ("kivi_k_stat_elems", _I64, [_CFG, _I64]),
    ("kivi_v_code_words", _I64, [_CFG, _I64]),
    ("kivi_v_stat_elems", _I64, [_CFG, _I64]),
    ("kivi_ring_elems", _I64, [_CFG]),
    ("kivi_encode_k", _I32, [_CFG, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P]),
    ("kivi_encode_v", _I32, [_CFG, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P]),
    ("kivi_decode_k", _I32, [_CFG, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P]),
    ("kivi_decode_v", _I32, [_CFG, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P]),
    ("kivi_boundary_layers", _I32, [_I64, _I64, _P]),
    ("kivi_encode_k_layers", _I32, [_CFG, _I64, _P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P]),
    ("kivi_encode_v_layers", _I32, [_CFG, _I64, _P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P]),
    ("kivi_decode_k_layers", _I32, [_CFG, _I64, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _I64, _P]),
    ("kivi_decode_v_layers", _I32, [_CFG, _I64, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _I64, _P]),
    ("kivi_stream_prefill", _I32, [_CFG, _ST, _P, _P, _I64, _I64, _P]),
    ("kivi_append_flush", _I32, [_CFG, _ST, _P, _P, _P]),
    ("kivi_fp8_encode", _I32, [_P, _I64, _I64, _I64, _I64, _P, _I64, _P]),
    ("kivi_fp8_decode", _I32, [_P, _I64, _I64, _I64, _I64, _P, _I64, _P]),
    ("kivi_stream_image_bytes", _I64, [_CFG, _I64, _I64]),
    ("kivi_stream_offload", _I32, [_CFG, _ST, _P, _I64, _P]),
    ("kivi_stream_restore", _I32, [_CFG, _ST, _P, _I64, _I64, _I64, _I64, _P]),
    ("kivi_attention_workspace_bytes", _I64, [_CFG, _I64, _I32, _I64, _I64]),
    ("kivi_decode_attention", _I32, [_CFG, _AC, _I64, _I32, _P, ctypes.c_float, _P, _P, _I64, _P]),
    ("kivi_decode_attention_noalloc", _I32, [_CFG, _AC, _I64, _I32, _P, ctypes.c_float, _P, _P]),
]

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m kv_cache_quantization_codec_amd.build` (there is no fallback path)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


@dataclass(frozen=True)
class Config:
    k_bits: int = 2
    v_bits: int = 2
    group_size: int = 32
    residual_length: int = 128
    head_dim: int = 128

    def c(self) -> kivi_config:
        return kivi_config(self.k_bits, self.v_bits, self.group_size,
                           self.residual_length, self.head_dim)


def _cfg(cfg) -> ctypes.POINTER(kivi_config):
    c = cfg.c() if isinstance(cfg, Config) else cfg
    return ctypes.byref(c)


def _stream_ptr(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _check(status: int, what: str):
    if status != KIVI_OK:
        raise KiviError(status, what)


def _on_device(t, what: str, device=None) -> torch.device:
    """The GPU device of tensor ``t`` (which must equal ``device`` when given)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{what}: expected a torch tensor, got {type(t).__name__}")
    if t.device.type != "cuda":
        raise ValueError(f"{what}: must be a GPU tensor, got one on {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{what}: on {t.device}, but the call's other tensors are on {device}")
    return t.device


def _fp16_cache(t: torch.Tensor, D: int, what: str, n_tokens: int | None = None, device=None):
    """(n_slices, slice_stride) of a GPU [S, T, D] fp16 tensor with token
    stride D (and T >= n_tokens when given)."""
    _on_device(t, what, device)
    if t.dtype != torch.float16 or t.dim() != 3 or t.shape[2] != D:
        raise ValueError(f"{what}: expected float16 [S, T, {D}], got {t.dtype} {tuple(t.shape)}")
    if t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != D):
        raise ValueError(f"{what}: tokens must be contiguous rows of {D} elements")
    if n_tokens is not None and t.shape[1] < n_tokens:
        raise ValueError(f"{what}: holds {t.shape[1]} tokens per slice, the call reads or writes {n_tokens}")
    return t.shape[0], t.stride(0)


def _sizes(cfg, keys: bool, cap_tokens: int):
    """(code words, elements of one sidecar) per slice of the key (or value)
    layouts for ``cap_tokens`` tokens, from the library's sizing entry points."""
    if keys:
        words, stats = kivi_k_code_words(cfg, cap_tokens), kivi_k_stat_elems(cfg, cap_tokens)
    else:
        words, stats = kivi_v_code_words(cfg, cap_tokens), kivi_v_stat_elems(cfg, cap_tokens)
    if words < 0 or stats < 0:
        raise ValueError(f"invalid configuration {cfg} or capacity {cap_tokens}")
    return words, stats


def _payload(cfg, payload, keys: bool, n_slices: int, cap_tokens: int, device, what: str):
    """Checks a (codes, scale, zero) triple against the C layouts: contiguous
    GPU tensors on ``device``, int32 / float16, each at least as large as
    ``n_slices`` slices of the layout for ``cap_tokens`` tokens."""
    if not isinstance(payload, (tuple, list)) or len(payload) != 3:
        raise ValueError(f"{what}: expected (codes, scale, zero)")
    words, stats = _sizes(cfg, keys, cap_tokens)
    for t, nm, dt, need in ((payload[0], "codes", torch.int32, words),
                            (payload[1], "scale", torch.float16, stats),
                            (payload[2], "zero", torch.float16, stats)):
        _on_device(t, f"{what} {nm}", device)
        if t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{what} {nm}: expected a contiguous {dt} tensor, got {t.dtype}")
        if t.numel() < n_slices * need:
            raise ValueError(f"{what} {nm}: {t.numel()} elements, the layout of {n_slices} slices "
                             f"x {cap_tokens} tokens needs {n_slices * need}")


# ---------------------------------------------------------------------------
# sizes
# ---------------------------------------------------------------------------

def kivi_k_code_words(cfg, n_tokens: int) -> int:
    return lib().kivi_k_code_words(_cfg(cfg), n_tokens)


def kivi_k_stat_elems(cfg, n_tokens: int) -> int:
    return lib().kivi_k_stat_elems(_cfg(cfg), n_tokens)


def kivi_v_code_words(cfg, n_tokens: int) -> int:
    return lib().kivi_v_code_words(_cfg(cfg), n_tokens)


def kivi_v_stat_elems(cfg, n_tokens: int) -> int:
    return lib().kivi_v_stat_elems(_cfg(cfg), n_tokens)


def kivi_ring_elems(cfg) -> int:
    return lib().kivi_ring_elems(_cfg(cfg))


def alloc_keys(cfg: Config, n_slices: int, cap_tokens: int, device="cuda"):
    """Empty key payload (codes, scale, zero) for ``cap_tokens`` tokens per slice,
    shaped [S, rows, D] like the C layouts (channel innermost), sized by the
    library."""
    words, stats = _sizes(cfg, True, cap_tokens)
    D = cfg.head_dim
    codes = torch.empty((n_slices, words // D, D), dtype=torch.int32, device=device)
    scale = torch.empty((n_slices, stats // D, D), dtype=torch.float16, device=device)
    zero = torch.empty((n_slices, stats // D, D), dtype=torch.float16, device=device)
    return codes, scale, zero


def alloc_values(cfg: Config, n_slices: int, cap_tokens: int, device="cuda"):
    """Empty value payload shaped [S, cap_tokens, per-row count] like the C
    layouts (one token row after another), sized by the library."""
    row_words, row_stats = _sizes(cfg, False, 1)
    codes = torch.empty((n_slices, cap_tokens, row_words), dtype=torch.int32, device=device)
    scale = torch.empty((n_slices, cap_tokens, row_stats), dtype=torch.float16, device=device)
    zero = torch.empty((n_slices, cap_tokens, row_stats), dtype=torch.float16, device=device)
    return codes, scale, zero


# ---------------------------------------------------------------------------
# codec entry points
# ---------------------------------------------------------------------------

def kivi_encode_k(cfg, k: torch.Tensor, n_tokens: int, codes, scale, zero,
                  cap_tokens: int | None = None, stream=None):
    """Per-channel key quantization of tokens [0, n_tokens) of ``k`` [S, T, D]."""
    S, stride = _fp16_cache(k, cfg.head_dim, "k", n_tokens)
    cap = n_tokens if cap_tokens is None else cap_tokens
    _payload(cfg, (codes, scale, zero), True, S, cap, k.device, "keys")
    _check(lib().kivi_encode_k(_cfg(cfg), _ptr(k), S, n_tokens, stride, cap, _ptr(codes),
                               _ptr(scale), _ptr(zero), _stream_ptr(stream)), "kivi_encode_k")


def kivi_encode_v(cfg, v: torch.Tensor, n_tokens: int, codes, scale, zero,
                  cap_tokens: int | None = None, stream=None):
    """Per-token value quantization of rows [0, n_tokens) of ``v`` [S, T, D]."""
    S, stride = _fp16_cache(v, cfg.head_dim, "v", n_tokens)
    cap = n_tokens if cap_tokens is None else cap_tokens
    _payload(cfg, (codes, scale, zero), False, S, cap, v.device, "values")
    _check(lib().kivi_encode_v(_cfg(cfg), _ptr(v), S, n_tokens, stride, cap, _ptr(codes),
                               _ptr(scale), _ptr(zero), _stream_ptr(stream)), "kivi_encode_v")


def kivi_decode_k(cfg, codes, scale, zero, n_tokens: int, out: torch.Tensor,
                  cap_tokens: int | None = None, stream=None):
    """Dequantize key tokens [0, n_tokens) into ``out`` [S, >=n_tokens, D]."""
    S, stride = _fp16_cache(out, cfg.head_dim, "out", n_tokens)
    cap = n_tokens if cap_tokens is None else cap_tokens
    _payload(cfg, (codes, scale, zero), True, S, cap, out.device, "keys")
    _check(lib().kivi_decode_k(_cfg(cfg), _ptr(codes), _ptr(scale), _ptr(zero), S, n_tokens, cap,
                               _ptr(out), stride, _stream_ptr(stream)), "kivi_decode_k")


def kivi_decode_v(cfg, codes, scale, zero, n_tokens: int, out: torch.Tensor,
                  cap_tokens: int | None = None, stream=None):
    """Dequantize value rows [0, n_tokens) into ``out`` [S, >=n_tokens, D]."""
    S, stride = _fp16_cache(out, cfg.head_dim, "out", n_tokens)
    cap = n_tokens if cap_tokens is None else cap_tokens
    _payload(cfg, (codes, scale, zero), False, S, cap, out.device, "values")
    _check(lib().kivi_decode_v(_cfg(cfg), _ptr(codes), _ptr(scale), _ptr(zero), S, n_tokens, cap,
                               _ptr(out), stride, _stream_ptr(stream)), "kivi_decode_v")


# ---------------------------------------------------------------------------
# per-layer bit mixes
# ---------------------------------------------------------------------------

def kivi_boundary_layers(n_layers: int, n: int) -> list[int]:
    """Indices of the protected (boundary) layers of an ``n_layers`` model."""
    flags = (ctypes.c_int32 * max(n_layers, 1))()
    count = lib().kivi_boundary_layers(n_layers, n, flags)
    if count < 0:
        raise KiviError(count, "kivi_boundary_layers")
    return [l for l in range(n_layers) if flags[l]]


def _side(c: Config, keys: bool):
    return (c.k_bits if keys else c.v_bits, c.group_size, c.head_dim)


def alloc_layers(cfgs, n_slices: int, cap_tokens: int, device="cuda", keys: bool = True):
    """Per-layer key (or value) payloads for a model whose layer l uses
    ``cfgs[l]``.  Consecutive layers with the same configuration on that side
    share one allocation, back to back, so the ``*_layers`` calls code each
    such run with one launch.  Returns a list of (codes, scale, zero) views."""
    out, l = [], 0
    alloc = alloc_keys if keys else alloc_values
    while l < len(cfgs):
        m = l + 1
        while m < len(cfgs) and _side(cfgs[m], keys) == _side(cfgs[l], keys):
            m += 1
        codes, scale, zero = alloc(cfgs[l], n_slices * (m - l), cap_tokens, device)
        for i in range(m - l):
            sl = slice(i * n_slices, (i + 1) * n_slices)
            out.append((codes[sl], scale[sl], zero[sl]))
        l = m
    return out


def _cfg_array(cfgs):
    return (kivi_config * max(len(cfgs), 1))(*[c.c() if isinstance(c, Config) else c for c in cfgs])


def _fp16_layers(t: torch.Tensor, D: int, what: str, n_tokens: int):
    """(n_layers, n_slices, layer_stride, slice_stride) of a GPU fp16
    [L, S, T >= n_tokens, D] tensor with contiguous token rows."""
    _on_device(t, what)
    if t.dtype != torch.float16 or t.dim() != 4 or t.shape[3] != D:
        raise ValueError(f"{what}: expected float16 [L, S, T, {D}], got {t.dtype} {tuple(t.shape)}")
    if t.stride(3) != 1 or (t.shape[2] > 1 and t.stride(2) != D):
        raise ValueError(f"{what}: tokens must be contiguous rows of {D} elements")
    if t.shape[2] < n_tokens:
        raise ValueError(f"{what}: holds {t.shape[2]} tokens per slice, the call reads or writes {n_tokens}")
    return t.shape[0], t.shape[1], t.stride(0), t.stride(1)


def _layer_ptrs(layers, L: int):
    if len(layers) != L:
        raise ValueError(f"expected {L} per-layer payloads, got {len(layers)}")
    arrs = [(ctypes.c_void_p * max(L, 1))(*[_ptr(p[i]) for p in layers]) for i in range(3)]
    return arrs


def _coded_layers(name: str, keys: bool, cfgs, x: torch.Tensor, n_tokens: int, layers, cap_tokens,
                  stream):
    L, S, lstride, sstride = _fp16_layers(x, cfgs[0].head_dim if cfgs else 0, "k" if keys else "v",
                                          n_tokens)
    if len(cfgs) != L:
        raise ValueError(f"expected {L} configurations, got {len(cfgs)}")
    cap = n_tokens if cap_tokens is None else cap_tokens
    if len(layers) != L:
        raise ValueError(f"expected {L} per-layer payloads, got {len(layers)}")
    for l in range(L):
        _payload(cfgs[l], layers[l], keys, S, cap, x.device, f"layer {l}")
    codes, scale, zero = _layer_ptrs(layers, L)
    fn = getattr(lib(), name)
    if name.startswith("kivi_encode"):
        st = fn(_cfg_array(cfgs), L, _ptr(x), lstride, S, n_tokens, sstride, cap, codes, scale, zero,
                _stream_ptr(stream))
    else:
        st = fn(_cfg_array(cfgs), L, codes, scale, zero, S, n_tokens, cap, _ptr(x), lstride, sstride,
                _stream_ptr(stream))
    _check(st, name)


def kivi_encode_k_layers(cfgs, k: torch.Tensor, n_tokens: int, layers, cap_tokens: int | None = None,
                         stream=None):
    """Keys ``k`` fp16 [L, S, T, D]: layer l coded with ``cfgs[l]`` into
    ``layers[l]`` = (codes, scale, zero)."""
    _coded_layers("kivi_encode_k_layers", True, cfgs, k, n_tokens, layers, cap_tokens, stream)


def kivi_encode_v_layers(cfgs, v: torch.Tensor, n_tokens: int, layers, cap_tokens: int | None = None,
                         stream=None):
    _coded_layers("kivi_encode_v_layers", False, cfgs, v, n_tokens, layers, cap_tokens, stream)


def kivi_decode_k_layers(cfgs, layers, n_tokens: int, out: torch.Tensor, cap_tokens: int | None = None,
                         stream=None):
    """Dequantize every layer's key tokens [0, n_tokens) into ``out`` fp16 [L, S, >=n_tokens, D]."""
    _coded_layers("kivi_decode_k_layers", True, cfgs, out, n_tokens, layers, cap_tokens, stream)


def kivi_decode_v_layers(cfgs, layers, n_tokens: int, out: torch.Tensor, cap_tokens: int | None = None,
                         stream=None):
    _coded_layers("kivi_decode_v_layers", False, cfgs, out, n_tokens, layers, cap_tokens, stream)


# ---------------------------------------------------------------------------
# streaming
# ---------------------------------------------------------------------------

class Stream:
    """Device buffers and host counters of one streaming cache (``kivi_stream``).

    ``k_ring`` / ``v_ring`` are fp16 [S, slots, D]; residual token i (0 =
    the oldest) of every slice sits in slot (ring_head + i) mod slots."""

    def __init__(self, cfg: Config, n_slices: int, cap_tokens: int, device="cuda"):
        D = cfg.head_dim
        if cap_tokens % cfg.group_size:
            raise ValueError("cap_tokens must be a multiple of group_size")
        ring = kivi_ring_elems(cfg)
        if ring < 0:
            raise ValueError(f"invalid configuration {cfg}")
        self.cfg = cfg
        self.keys = alloc_keys(cfg, n_slices, cap_tokens, device)
        self.values = alloc_values(cfg, n_slices, cap_tokens, device)
        self.k_ring = torch.empty((n_slices, ring // D, D), dtype=torch.float16, device=device)
        self.v_ring = torch.empty((n_slices, ring // D, D), dtype=torch.float16, device=device)
        kc, ks, kz = self.keys
        vc, vs, vz = self.values
        self.state = kivi_stream(_ptr(kc), _ptr(vc), _ptr(ks), _ptr(kz), _ptr(vs), _ptr(vz),
                                 _ptr(self.k_ring), _ptr(self.v_ring), n_slices, cap_tokens,
                                 0, 0, 0)

    @property
    def n_quant(self) -> int:
        return self.state.n_quant

    @property
    def ring_head(self) -> int:
        return self.state.ring_head

    @property
    def ring_count(self) -> int:
        return self.state.ring_count


def kivi_stream_prefill(st: Stream, k: torch.Tensor, v: torch.Tensor, n_tokens: int, stream=None):
    dev = st.k_ring.device
    S, stride = _fp16_cache(k, st.cfg.head_dim, "k", n_tokens, dev)
    S2, stride2 = _fp16_cache(v, st.cfg.head_dim, "v", n_tokens, dev)
    if S != st.state.n_slices or S2 != S or stride2 != stride:
        raise ValueError("k and v must match the stream's slices and share one stride")
    _check(lib().kivi_stream_prefill(_cfg(st.cfg), ctypes.byref(st.state), _ptr(k), _ptr(v),
                                     n_tokens, stride, _stream_ptr(stream)), "kivi_stream_prefill")


def kivi_append_flush(st: Stream, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> bool:
    """One decode step; returns True when a group was flushed."""
    D = st.cfg.head_dim
    for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
        _on_device(t, nm, st.k_ring.device)
        if t.dtype != torch.float16 or tuple(t.shape) != (st.state.n_slices, D) or not t.is_contiguous():
            raise ValueError(f"{nm}: expected contiguous float16 [{st.state.n_slices}, {D}]")
    before = st.state.n_quant
    _check(lib().kivi_append_flush(_cfg(st.cfg), ctypes.byref(st.state), _ptr(k_new), _ptr(v_new),
                                   _stream_ptr(stream)), "kivi_append_flush")
    return st.state.n_quant != before


# ---------------------------------------------------------------------------
# FP8 keys (k8v4 layout)
# ---------------------------------------------------------------------------

def _rows(t: torch.Tensor, dtype, what: str, n_tokens: int, device=None):
    """(n_slices, n_rows_allocated, D, slice_stride) of a GPU [S, T >= n_tokens, D]
    tensor with contiguous rows."""
    _on_device(t, what, device)
    if t.dtype != dtype or t.dim() != 3 or t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != t.shape[2]):
        raise ValueError(f"{what}: expected {dtype} [S, T, D] with contiguous token rows")
    if t.shape[1] < n_tokens:
        raise ValueError(f"{what}: holds {t.shape[1]} tokens per slice, the call reads or writes {n_tokens}")
    return t.shape[0], t.shape[1], t.shape[2], t.stride(0)


def kivi_fp8_encode(k: torch.Tensor, n_tokens: int, out: torch.Tensor, stream=None):
    """FP8 (E4M3) codes of tokens [0, n_tokens) of ``k`` fp16 [S, T, D] into
    ``out`` uint8 [S, T', D]."""
    S, _, D, si = _rows(k, torch.float16, "k", n_tokens)
    S2, _, D2, so = _rows(out, torch.uint8, "out", n_tokens, k.device)
    if (S2, D2) != (S, D):
        raise ValueError("out must match k's slices and head_dim")
    _check(lib().kivi_fp8_encode(_ptr(k), S, n_tokens, D, si, _ptr(out), so, _stream_ptr(stream)),
           "kivi_fp8_encode")


def kivi_fp8_decode(codes: torch.Tensor, n_tokens: int, out: torch.Tensor, stream=None):
    S, _, D, si = _rows(codes, torch.uint8, "codes", n_tokens)
    S2, _, D2, so = _rows(out, torch.float16, "out", n_tokens, codes.device)
    if (S2, D2) != (S, D):
        raise ValueError("out must match the codes' slices and head_dim")
    _check(lib().kivi_fp8_decode(_ptr(codes), S, n_tokens, D, si, _ptr(out), so, _stream_ptr(stream)),
           "kivi_fp8_decode")


# ---------------------------------------------------------------------------
# compact host image of a streaming cache
# ---------------------------------------------------------------------------

def kivi_stream_image_bytes(cfg, n_slices: int, n_quant: int) -> int:
    return lib().kivi_stream_image_bytes(_cfg(cfg), n_slices, n_quant)


def _host_bytes(host: torch.Tensor) -> int:
    if host.device.type != "cpu" or not host.is_contiguous():
        raise ValueError("host image must be a contiguous CPU tensor (pinned for async copies)")
    return host.numel() * host.element_size()


def kivi_stream_offload(st: Stream, host: torch.Tensor, stream=None):
    """Enqueue the copies of ``st``'s image into ``host`` (uint8 CPU tensor of
    at least :func:`kivi_stream_image_bytes` bytes)."""
    _check(lib().kivi_stream_offload(_cfg(st.cfg), ctypes.byref(st.state), _ptr(host), _host_bytes(host),
                                     _stream_ptr(stream)), "kivi_stream_offload")


def kivi_stream_restore(st: Stream, host: torch.Tensor, n_quant: int, ring_head: int, ring_count: int,
                        stream=None):
    """Enqueue the copies of an image into ``st`` and set its counters."""
    _check(lib().kivi_stream_restore(_cfg(st.cfg), ctypes.byref(st.state), _ptr(host), _host_bytes(host),
                                     n_quant, ring_head, ring_count, _stream_ptr(stream)),
           "kivi_stream_restore")


# ---------------------------------------------------------------------------
# decode attention over the quantized cache
# ---------------------------------------------------------------------------

class AttnCache:
    """A ``kivi_attn_cache`` plus references to the tensors it points into.

    ``keys`` / ``values``: payloads laid out for ``cap_tokens`` tokens per
    slice (as from :func:`alloc_keys` / :func:`alloc_values`); ``n_quant`` of
    them are read.  ``res_k`` / ``res_v``: fp16 ``[S, slots, D]`` tensors (any
    slice stride) holding the residual as a ring whose oldest token is at
    slot ``res_head``; ``res_count`` defaults to all slots.

    Ragged batches: ``n_quant_per_slice`` / ``res_count_per_slice`` (int32
    device tensors ``[S]``) give each slice its own counts, clamped to
    ``[0, n_quant]`` / ``[0, res_count]``, which then act as upper bounds;
    a slice with no token at all gets a zero output."""

    def __init__(self, cfg: Config, keys, values, n_quant: int, res_k=None, res_v=None,
                 res_head: int = 0, res_count: int | None = None,
                 n_quant_per_slice: torch.Tensor | None = None,
                 res_count_per_slice: torch.Tensor | None = None):
        D = cfg.head_dim
        vc, vs, vz = values
        kc, ks, kz = keys
        dev = _on_device(kc, "key codes")
        if kc.dim() != 3 or vc.dim() != 3 or vc.shape[0] != kc.shape[0]:
            raise ValueError("key codes [S, rows, D] and value codes [S, cap_tokens, words per row] "
                             "expected, with one slice count")
        S, cap = kc.shape[0], vc.shape[1]
        _payload(cfg, keys, True, S, cap, dev, "keys")
        _payload(cfg, values, False, S, cap, dev, "values")
        stride, slots = 0, 0
        if res_k is not None and res_k.shape[1] == 0:     # an empty residual
            res_k = res_v = None
        if res_k is not None:
            for t, nm in ((res_k, "res_k"), (res_v, "res_v")):
                _on_device(t, nm, dev)
                if t.dtype != torch.float16 or t.dim() != 3 or t.shape[2] != D or t.stride(2) != 1 \
                        or (t.shape[1] > 1 and t.stride(1) != D) or t.shape[0] != S:
                    raise ValueError(f"{nm}: expected float16 [{S}, slots, {D}] with contiguous rows")
            if res_v.stride(0) != res_k.stride(0) or res_v.shape[1] != res_k.shape[1]:
                raise ValueError("res_k and res_v must share slots and slice stride")
            stride, slots = res_k.stride(0), res_k.shape[1]
        count = slots if res_count is None else res_count
        for t, nm in ((n_quant_per_slice, "n_quant_per_slice"), (res_count_per_slice, "res_count_per_slice")):
            if t is not None:
                _on_device(t, nm, dev)
                if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous() or t.shape[0] != S:
                    raise ValueError(f"{nm}: expected contiguous int32 [n_slices] on the device")
        self.cfg = cfg
        self.device = dev
        self.n_slices = S
        self._refs = (keys, values, res_k, res_v, n_quant_per_slice, res_count_per_slice)
        self.c = kivi_attn_cache(_ptr(kc), _ptr(ks), _ptr(kz), _ptr(vc), _ptr(vs), _ptr(vz),
                                 cap, n_quant, _ptr(res_k), _ptr(res_v), stride, slots,
                                 res_head, count, _ptr(n_quant_per_slice), _ptr(res_count_per_slice))

    @classmethod
    def from_stream(cls, st: Stream) -> "AttnCache":
        return cls(st.cfg, st.keys, st.values, st.n_quant, st.k_ring, st.v_ring,
                   st.ring_head, st.ring_count)


def kivi_attention_workspace_bytes(cfg, n_slices: int, q_per_kv: int, n_quant: int,
                                   res_count: int) -> int:
    return lib().kivi_attention_workspace_bytes(_cfg(cfg), n_slices, q_per_kv, n_quant, res_count)


def _attention_io(cfg, cache: AttnCache, q: torch.Tensor, out: torch.Tensor):
    D = cfg.head_dim
    for t, nm in ((q, "q"), (out, "out")):
        _on_device(t, nm, cache.device)
        if t.dtype != torch.float16 or t.dim() != 3 or t.shape[2] != D or not t.is_contiguous():
            raise ValueError(f"{nm}: expected contiguous float16 [S, q_per_kv, {D}]")
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if q.shape[0] != cache.n_slices:
        raise ValueError(f"q has {q.shape[0]} slices, the cache {cache.n_slices}")
    return q.shape[0], q.shape[1]


def kivi_decode_attention(cfg, cache: AttnCache, q: torch.Tensor, sm_scale: float,
                          out: torch.Tensor, workspace: torch.Tensor | None = None, stream=None):
    """Attention of ``q`` fp16 [S, q_per_kv, D] over ``cache`` into ``out``
    (same shape).  A workspace of the size the library asks for is allocated
    on ``q``'s device when none is given."""
    S, r = _attention_io(cfg, cache, q, out)
    need = kivi_attention_workspace_bytes(cfg, S, r, cache.c.n_quant, cache.c.res_count)
    if need < 0:
        raise KiviError(-6, "kivi_attention_workspace_bytes")
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _on_device(workspace, "workspace", q.device)
        if not workspace.is_contiguous():
            raise ValueError("workspace: expected a contiguous tensor")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().kivi_decode_attention(_cfg(cfg), ctypes.byref(cache.c), S, r, _ptr(q),
                                       float(sm_scale), _ptr(out), _ptr(workspace), ws_bytes,
                                       _stream_ptr(stream)), "kivi_decode_attention")


def kivi_decode_attention_noalloc(cfg, cache: AttnCache, q: torch.Tensor, sm_scale: float,
                                  out: torch.Tensor, stream=None):
    """:func:`kivi_decode_attention` with the split partials in the library's
    static per-device scratch (``ATTENTION_SCRATCH_BYTES``): allocates
    nothing.  Calls that overlap on one device race on that scratch."""
    S, r = _attention_io(cfg, cache, q, out)
    _check(lib().kivi_decode_attention_noalloc(_cfg(cfg), ctypes.byref(cache.c), S, r, _ptr(q),
                                               float(sm_scale), _ptr(out), _stream_ptr(stream)),
           "kivi_decode_attention_noalloc")
