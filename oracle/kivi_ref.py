"""KIVI grouped KV-cache codec -- numpy oracle tier.

TEST INFRASTRUCTURE ONLY (see the package docstring): plain, slow and
written to be checked by eye against the method statement.  No blocking, no
fusion; a Python loop over groups, numpy arithmetic inside each group.

Method (CacheForge README, "How it works"; CacheSeek PR #4 description):

* keys   -- one (scale, zero) pair per channel per group of ``G`` consecutive
  tokens (keys are quantized channel by channel);
* values -- one (scale, zero) pair per token per group of ``G`` consecutive
  channels (values are quantized token by token);
* codes of ``b`` bits (2**b levels, vLLM ``TurboQuantConfig`` docstring),
  packed into 32-bit words (CacheSeek PR #4 packs 4-bit codes into int32),
  with padding for partial groups;
* the most recent ``R`` tokens stay in fp16 (CacheForge README, "How it
  works" and the ``residual_length`` knob in "Example").

Readings where the pages are silent (each is a choice, stated once here and
applied everywhere below):

1. Statistics in float32 over the *valid* elements of a group (padding never
   enters them).  ``mn``/``mx`` are fp16 values, exact in float32; a negative
   zero is canonicalised to +0.
2. ``scale = fp16( fp32( fp32(mx - mn) / fp32(2**b - 1) ) )`` with IEEE
   round-to-nearest-even at each step; ``zero = fp16(mn)`` (exact).
3. ``q = clamp(rint(fp32(fp32(x - zero) / scale)), 0, 2**b - 1)`` with IEEE
   float32 division and ``rint`` rounding half to even; a group whose fp16
   scale is zero (constant group, or a range too small for fp16) gets
   ``q = 0`` everywhere.
4. Packing: code ``i`` of a word sits at bits ``[i*b, i*b + b)``; word ``w``
   of a group holds elements ``w*(32/b) + i`` along the group axis.  Keys are
   packed along tokens, values along channels.  Pad slots hold code 0.
5. Decode: ``xhat = fp16( fp32( fp32(q) * fp32(scale) + fp32(zero) ) )``;
   the product is exact in float32 (8-bit code times 11-bit significand).
6. Full cache of ``T`` tokens: the first ``T_q = max(T - R, 0)`` are
   quantized, the last ``min(R, T)`` stay fp16 and are not touched.
7. Streaming: after a prefill that quantizes ``floor((T - R)/G)*G`` tokens,
   each step appends one fp16 token to the residual; when the residual holds
   more than ``R`` tokens and at least ``G``, its oldest ``G`` tokens are
   quantized as one key group and ``G`` value rows.

Layouts (per slice ``s`` of ``S`` independent (layer, batch, head) slices):

* input K or V: float16 ``[S, T_alloc, D]``, token stride ``D``;
* key codes ``int32 [S, NG_k * G*b/32, D]`` (channel innermost), key stats
  ``float16 [S, NG_k, D]`` with ``NG_k = ceil(T_q / G)``;
* value codes ``int32 [S, T_q, NG_v * G*b/32]``, value stats
  ``float16 [S, T_q, NG_v]`` with ``NG_v = ceil(D / G)``.
"""

from __future__ import annotations

import numpy as np

F16 = np.float16
F32 = np.float32

VALID_BITS = (2, 4, 8)
VALID_GROUPS = (32, 64, 128)


# ---------------------------------------------------------------------------
# sizes (CacheSeek PR #4: stored payload sizes are accounted by the manager)
# ---------------------------------------------------------------------------

def n_groups(n: int, group_size: int) -> int:
    """Number of groups, the last one possibly partial (padded)."""
    return -(-n // group_size) if n > 0 else 0


def words_per_group(bits: int, group_size: int) -> int:
    """int32 words that hold one group's ``group_size`` codes of ``bits`` bits."""
    return group_size * bits // 32


def k_code_words(n_tokens: int, head_dim: int, bits: int, group_size: int) -> int:
    """int32 words of key codes per slice for ``n_tokens`` quantized tokens."""
    return n_groups(n_tokens, group_size) * words_per_group(bits, group_size) * head_dim


def k_stat_elems(n_tokens: int, head_dim: int, group_size: int) -> int:
    """fp16 elements of *one* key sidecar (scale or zero) per slice."""
    return n_groups(n_tokens, group_size) * head_dim


def v_code_words(n_tokens: int, head_dim: int, bits: int, group_size: int) -> int:
    """int32 words of value codes per slice."""
    return n_tokens * n_groups(head_dim, group_size) * words_per_group(bits, group_size)


def v_stat_elems(n_tokens: int, head_dim: int, group_size: int) -> int:
    """fp16 elements of *one* value sidecar (scale or zero) per slice."""
    return n_tokens * n_groups(head_dim, group_size)


def quantized_tokens(total_tokens: int, residual_length: int) -> int:
    """Reading 6: tokens that are quantized in a full cache of ``total_tokens``."""
    return max(total_tokens - residual_length, 0)


# ---------------------------------------------------------------------------
# one group: statistics, codes, reconstruction
# ---------------------------------------------------------------------------

def group_params(x: np.ndarray, bits: int):
    """Scale and zero of groups whose valid elements lie along the last axis.

    ``x`` holds fp16 values (any float dtype that represents them exactly);
    every group must have at least one valid element.  Returns
    ``(scale, zero)`` as float16 arrays of shape ``x.shape[:-1]``
    (readings 1 and 2).
    """
    x32 = np.asarray(x).astype(F32)
    mn = x32.min(axis=-1) + F32(0.0)      # -0 + +0 = +0 under round-to-nearest
    mx = x32.max(axis=-1) + F32(0.0)
    rng = (mx - mn).astype(F32)
    levels = F32(2 ** bits - 1)
    s32 = (rng / levels).astype(F32)
    scale = s32.astype(F16)
    zero = mn.astype(F16)
    return scale, zero


def quantize(x: np.ndarray, scale: np.ndarray, zero: np.ndarray, bits: int) -> np.ndarray:
    """Codes of fp16 values ``x`` under broadcastable fp16 ``scale``/``zero``
    (reading 3).  Returns uint32 codes in ``[0, 2**b - 1]``."""
    x32 = np.asarray(x).astype(F32)
    s32 = np.asarray(scale).astype(F32)
    z32 = np.asarray(zero).astype(F32)
    d = (x32 - z32).astype(F32)
    s_b = np.broadcast_to(s32, d.shape)
    ok = s_b != 0
    quot = np.zeros(d.shape, dtype=F32)
    np.divide(d, s_b, out=quot, where=ok)
    q = np.clip(np.rint(quot), F32(0), F32(2 ** bits - 1))
    q = np.where(ok, q, F32(0))
    return q.astype(np.uint32)


def dequantize(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """fp16 reconstruction (reading 5)."""
    q32 = np.asarray(codes).astype(F32)
    s32 = np.asarray(scale).astype(F32)
    z32 = np.asarray(zero).astype(F32)
    y = (q32 * s32).astype(F32)
    y = (y + z32).astype(F32)
    with np.errstate(over="ignore"):      # |y| >= 65520 rounds to +-inf, as IEEE says
        return y.astype(F16)


# ---------------------------------------------------------------------------
# packing (reading 4)
# ---------------------------------------------------------------------------

def pack_words(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes along the last axis (length a multiple of 32/bits) into
    uint32 words, LSB first."""
    per = 32 // bits
    c = np.asarray(codes).astype(np.uint32)
    assert c.shape[-1] % per == 0
    c = c.reshape(c.shape[:-1] + (c.shape[-1] // per, per))
    words = np.zeros(c.shape[:-1], dtype=np.uint32)
    for i in range(per):
        words |= (c[..., i] & np.uint32(2 ** bits - 1)) << np.uint32(bits * i)
    return words


def unpack_words(words: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of :func:`pack_words`: uint32 words -> codes along the last axis."""
    per = 32 // bits
    w = np.asarray(words).astype(np.uint32)
    out = np.empty(w.shape + (per,), dtype=np.uint32)
    for i in range(per):
        out[..., i] = (w >> np.uint32(bits * i)) & np.uint32(2 ** bits - 1)
    return out.reshape(w.shape[:-1] + (w.shape[-1] * per,))


# ---------------------------------------------------------------------------
# full-tensor encode / decode
# ---------------------------------------------------------------------------

def _check(bits: int, group_size: int):
    if bits not in VALID_BITS:
        raise ValueError(f"bits must be one of {VALID_BITS}, got {bits}")
    if group_size not in VALID_GROUPS:
        raise ValueError(f"group_size must be one of {VALID_GROUPS}, got {group_size}")


def encode_k(k: np.ndarray, n_tokens: int, bits: int, group_size: int):
    """Per-channel key quantization over groups of ``group_size`` tokens.

    ``k``: float16 ``[S, T_alloc, D]`` with ``T_alloc >= n_tokens``; only the
    first ``n_tokens`` tokens are read.  Returns ``(codes, scale, zero)`` in
    the key layouts of the module docstring.
    """
    _check(bits, group_size)
    k = np.asarray(k, dtype=F16)
    S, _, D = k.shape
    G = group_size
    ng = n_groups(n_tokens, G)
    codes = np.zeros((S, ng * G, D), dtype=np.uint32)
    scale = np.zeros((S, ng, D), dtype=F16)
    zero = np.zeros((S, ng, D), dtype=F16)
    for g in range(ng):
        t0, t1 = g * G, min((g + 1) * G, n_tokens)
        xg = k[:, t0:t1, :]                                  # [S, nv, D]
        sc, zr = group_params(np.moveaxis(xg, 1, 2), bits)   # [S, D]
        scale[:, g, :] = sc
        zero[:, g, :] = zr
        codes[:, t0:t1, :] = quantize(xg, sc[:, None, :], zr[:, None, :], bits)
    # pack along tokens: move tokens last, pack, move word rows back
    words = pack_words(np.moveaxis(codes, 1, 2), bits)      # [S, D, ng*W]
    words = np.ascontiguousarray(np.moveaxis(words, 2, 1))  # [S, ng*W, D]
    return words.view(np.int32), scale, zero


def encode_v(v: np.ndarray, n_tokens: int, bits: int, group_size: int):
    """Per-token value quantization over groups of ``group_size`` channels.

    ``v``: float16 ``[S, T_alloc, D]``.  Returns ``(codes, scale, zero)`` in
    the value layouts of the module docstring.
    """
    _check(bits, group_size)
    v = np.asarray(v, dtype=F16)
    S, _, D = v.shape
    G = group_size
    ng = n_groups(D, G)
    codes = np.zeros((S, n_tokens, ng * G), dtype=np.uint32)
    scale = np.zeros((S, n_tokens, ng), dtype=F16)
    zero = np.zeros((S, n_tokens, ng), dtype=F16)
    for g in range(ng):
        c0, c1 = g * G, min((g + 1) * G, D)
        xg = v[:, :n_tokens, c0:c1]                          # [S, n, nv]
        sc, zr = group_params(xg, bits)                      # [S, n]
        scale[:, :, g] = sc
        zero[:, :, g] = zr
        codes[:, :, c0:c1] = quantize(xg, sc[..., None], zr[..., None], bits)
    words = pack_words(codes, bits)                          # [S, n, ng*W]
    return np.ascontiguousarray(words).view(np.int32), scale, zero


def decode_k(codes, scale, zero, n_tokens: int, bits: int, group_size: int):
    """Inverse of :func:`encode_k` for the ``n_tokens`` valid tokens:
    returns float16 ``[S, n_tokens, D]``."""
    _check(bits, group_size)
    G = group_size
    w = np.asarray(codes).view(np.uint32)                    # [S, ng*W, D]
    q = unpack_words(np.moveaxis(w, 1, 2), bits)             # [S, D, ng*G]
    q = np.moveaxis(q, 2, 1)[:, :n_tokens, :]                # [S, n, D]
    tok_group = np.arange(n_tokens) // G
    sc = np.asarray(scale)[:, tok_group, :]
    zr = np.asarray(zero)[:, tok_group, :]
    return dequantize(q, sc, zr)


def decode_v(codes, scale, zero, n_tokens: int, bits: int, group_size: int, head_dim: int):
    """Inverse of :func:`encode_v`: returns float16 ``[S, n_tokens, D]``."""
    _check(bits, group_size)
    G = group_size
    w = np.asarray(codes).view(np.uint32)[:, :n_tokens, :]   # [S, n, ng*W]
    q = unpack_words(w, bits)[:, :, :head_dim]               # [S, n, D]
    ch_group = np.arange(head_dim) // G
    sc = np.asarray(scale)[:, :n_tokens, :][:, :, ch_group]
    zr = np.asarray(zero)[:, :n_tokens, :][:, :, ch_group]
    return dequantize(q, sc, zr)


# ---------------------------------------------------------------------------
# streaming decode phase (reading 7)
# ---------------------------------------------------------------------------

def flush_due(residual_count: int, residual_length: int, group_size: int) -> bool:
    """True when the fp16 residual must give its oldest group to the codec."""
    return residual_count > residual_length and residual_count >= group_size


class StreamRef:
    """Logical state of a streaming cache: a quantized prefix (grown one
    group at a time) and the fp16 residual in age order.

    Keys and values share ``G`` and ``R`` (the CacheForge example has one
    ``group_size`` and one ``residual_length``).
    """

    def __init__(self, k_bits, v_bits, group_size, residual_length):
        _check(k_bits, group_size)
        _check(v_bits, group_size)
        self.kb, self.vb = k_bits, v_bits
        self.G, self.R = group_size, residual_length
        self.k_groups = []   # list of (codes [S, W, D], scale [S, D], zero [S, D])
        self.v_rows = []     # list of (codes [S, G, NGv*W], scale, zero)
        self.res_k = None    # float16 [S, n_res, D], oldest first
        self.res_v = None
        self.n_quant = 0
        self.flushes = 0

    def prefill(self, k, v, total_tokens):
        """Quantize ``floor((T - R)/G)*G`` tokens; keep the rest as residual."""
        k = np.asarray(k, dtype=F16)
        v = np.asarray(v, dtype=F16)
        G = self.G
        nq = (quantized_tokens(total_tokens, self.R) // G) * G
        for g in range(nq // G):
            self._flush_tokens(k[:, g * G:(g + 1) * G], v[:, g * G:(g + 1) * G])
        self.res_k = k[:, nq:total_tokens].copy()
        self.res_v = v[:, nq:total_tokens].copy()
        self.n_quant = nq
        self.flushes = 0

    def _flush_tokens(self, kg, vg):
        G = self.G
        self.k_groups.append(encode_k(kg, G, self.kb, G))
        c, s, z = encode_v(vg, G, self.vb, G)
        self.v_rows.append((c, s, z))

    def append(self, k_new, v_new):
        """One decode step: ``k_new``/``v_new`` float16 ``[S, D]``.  Returns
        True when the step flushed a group."""
        self.res_k = np.concatenate([self.res_k, np.asarray(k_new, F16)[:, None]], axis=1)
        self.res_v = np.concatenate([self.res_v, np.asarray(v_new, F16)[:, None]], axis=1)
        if flush_due(self.res_k.shape[1], self.R, self.G):
            G = self.G
            self._flush_tokens(self.res_k[:, :G], self.res_v[:, :G])
            self.res_k = self.res_k[:, G:]
            self.res_v = self.res_v[:, G:]
            self.n_quant += G
            self.flushes += 1
            return True
        return False

    def key_arrays(self):
        """Concatenated key codes/scale/zero in the full-cache layout."""
        c = np.concatenate([g[0] for g in self.k_groups], axis=1)
        s = np.concatenate([g[1] for g in self.k_groups], axis=1)
        z = np.concatenate([g[2] for g in self.k_groups], axis=1)
        return c, s, z

    def value_arrays(self):
        c = np.concatenate([r[0] for r in self.v_rows], axis=1)
        s = np.concatenate([r[1] for r in self.v_rows], axis=1)
        z = np.concatenate([r[2] for r in self.v_rows], axis=1)
        return c, s, z
