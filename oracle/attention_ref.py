"""Decode-phase attention over a KIVI-quantized KV cache -- float64 oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain numpy, no
blocking or fusion, written to be checked by eye.

What is computed (CacheForge README: "Contribution scope" says the
inherited KIVI code brings model integrations and the kernels that consume
the quantized cache; "How it works" keeps keys quantized per channel,
values per token and the newest tokens in higher precision; the same page's
prefill/decoding flow figure is missing from the text).  The pages give no
formula for the consumer, so the reading used here is the ordinary one for
the Llama and Mistral families the page names:

* one query token per query head attends to every cached token of its KV
  head: ``out = sum_t softmax_t(sm_scale * q . k_t) * v_t``;
* grouped-query heads: ``r = q_per_kv`` consecutive query heads share one
  KV head (``r = 1`` is plain multi-head attention);
* the cached tokens are the quantized prefix, dequantized as
  ``code * scale + zero`` with the stored fp16 scale and zero, followed by
  the fp16 residual tokens in age order (the softmax does not depend on the
  order);
* the dequantized values enter at full precision: the fp16 rounding of the
  codec's decode output is a property of materialising a decoded cache, not
  of the attention (float64 holds ``code * scale`` exactly and rounds the sum
  with ``zero`` once, i.e. correctly).

Shapes: ``q`` float16 ``[S, r, D]``; key/value payloads as produced by
:mod:`oracle.kivi_ref` for ``S`` slices; residual float16 ``[S, count, D]``.
Returns float64 ``[S, r, D]``.
"""

from __future__ import annotations

import numpy as np

from . import kivi_ref as ref

F64 = np.float64


def dequantize_exact_k(codes, scale, zero, n_tokens: int, bits: int, group_size: int):
    """Keys ``code * scale + zero`` in float64 for the first ``n_tokens``
    tokens: ``[S, n_tokens, D]``.  Codes unpacked along tokens, one (scale,
    zero) pair per channel per group of ``group_size`` tokens."""
    w = np.asarray(codes).view(np.uint32)                    # [S, ng*W, D]
    q = ref.unpack_words(np.moveaxis(w, 1, 2), bits)         # [S, D, ng*G]
    q = np.moveaxis(q, 2, 1)[:, :n_tokens, :].astype(F64)    # [S, n, D]
    grp = np.arange(n_tokens) // group_size
    s = np.asarray(scale)[:, grp, :].astype(F64)
    z = np.asarray(zero)[:, grp, :].astype(F64)
    return q * s + z


def dequantize_exact_v(codes, scale, zero, n_tokens: int, bits: int, group_size: int,
                       head_dim: int):
    """Values ``code * scale + zero`` in float64: ``[S, n_tokens, D]``.
    Codes unpacked along channels, one pair per token per channel group."""
    w = np.asarray(codes).view(np.uint32)[:, :n_tokens, :]
    q = ref.unpack_words(w, bits)[:, :, :head_dim].astype(F64)
    grp = np.arange(head_dim) // group_size
    s = np.asarray(scale)[:, :n_tokens, :][:, :, grp].astype(F64)
    z = np.asarray(zero)[:, :n_tokens, :][:, :, grp].astype(F64)
    return q * s + z


def ring_tokens(ring, head: int, count: int):
    """The ``count`` residual tokens of a ring ``[S, slots, D]`` in age order,
    oldest at slot ``head``."""
    ring = np.asarray(ring)
    slots = ring.shape[1]
    idx = (head + np.arange(count)) % slots
    return ring[:, idx, :]


def softmax_attention(q, k, v, sm_scale: float):
    """``q`` ``[S, r, D]``, ``k``/``v`` ``[S, T, D]`` (T >= 1): float64
    ``softmax(sm_scale * q k^T) v`` per slice; all query heads of a slice
    attend to that slice's tokens."""
    q = np.asarray(q).astype(F64)
    k = np.asarray(k).astype(F64)
    v = np.asarray(v).astype(F64)
    logits = np.einsum("srd,std->srt", q, k) * F64(sm_scale)
    logits -= logits.max(axis=-1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=-1, keepdims=True)
    return np.einsum("srt,std->srd", p, v)


def cache_tokens(k_payload, v_payload, n_quant: int, res_k, res_v, k_bits: int, v_bits: int,
                 group_size: int, head_dim: int):
    """All cached keys and values of each slice as float64 ``[S, n_quant +
    count, D]``: the dequantized prefix followed by the residual tokens."""
    parts_k, parts_v = [], []
    if n_quant:
        parts_k.append(dequantize_exact_k(*k_payload, n_quant, k_bits, group_size))
        parts_v.append(dequantize_exact_v(*v_payload, n_quant, v_bits, group_size, head_dim))
    if res_k is not None and np.asarray(res_k).shape[1]:
        parts_k.append(np.asarray(res_k).astype(F64))
        parts_v.append(np.asarray(res_v).astype(F64))
    return np.concatenate(parts_k, axis=1), np.concatenate(parts_v, axis=1)


def decode_attention(q, k_payload, v_payload, n_quant: int, res_k, res_v, k_bits: int,
                     v_bits: int, group_size: int, sm_scale: float):
    """Attention of ``q`` ``[S, r, D]`` over the quantized prefix of
    ``n_quant`` tokens plus the residual ``res_k``/``res_v`` ``[S, count, D]``
    (fp16, age order).  At least one token must be cached."""
    D = np.asarray(q).shape[-1]
    k, v = cache_tokens(k_payload, v_payload, n_quant, res_k, res_v, k_bits, v_bits,
                        group_size, D)
    if k.shape[1] == 0:
        raise ValueError("attention over an empty cache is undefined")
    return softmax_attention(q, k, v, sm_scale)
