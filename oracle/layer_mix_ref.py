"""Per-layer bit mixes (boundary protection) -- oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

vLLM ``turboquant/config.py``, ``get_boundary_skip_layers``: a dense model
exempts its first n and its last n attention layers from an aggressive
preset.  n is first capped at half the layer count (integer division); the
two index sets are merged, so they may overlap when the model has at most
2n layers; and n <= 0, or a model with no layers, protects nothing.  The
page switches the protection off for hybrid attention/linear models, which
have no counterpart here.

Reading (the page skips the protected layers' compression altogether): for
the KIVI codec a protected layer takes a configuration of its own, normally
more bits, and the other layers share the base configuration.  The page's
plain skipping is the case where the caller keeps the protected layers in
fp16 and codes only the others.

A mixed cache is coded layer by layer, each layer by the single-configuration
codec of :mod:`oracle.kivi_ref` with that layer's bit width.
"""

from __future__ import annotations

from . import kivi_ref as ref


def boundary_layers(n_layers: int, n: int) -> list[int]:
    """Sorted indices of the protected layers of an ``n_layers`` model."""
    if n <= 0 or n_layers <= 0:
        return []
    n = min(n, n_layers // 2)
    first = set(range(n))
    last = set(range(n_layers - n, n_layers))
    return sorted(first | last)


def layer_bits(n_layers: int, n: int, base, protected) -> list:
    """Per-layer (k_bits, v_bits): ``protected`` on the boundary layers,
    ``base`` elsewhere."""
    prot = set(boundary_layers(n_layers, n))
    return [tuple(protected) if l in prot else tuple(base) for l in range(n_layers)]


def encode_layers(x, n_tokens: int, bits_per_layer, group_size: int, keys: bool):
    """``x`` fp16 ``[L, S, T, D]`` -> list of per-layer payloads (codes,
    scale, zero); layer l is coded with the key (or value) bits of
    ``bits_per_layer[l]``."""
    side = 0 if keys else 1
    enc = ref.encode_k if keys else ref.encode_v
    return [enc(x[l], n_tokens, bits[side], group_size) for l, bits in enumerate(bits_per_layer)]


def decode_layers(payloads, n_tokens: int, bits_per_layer, group_size: int, head_dim: int,
                  keys: bool):
    """Inverse of :func:`encode_layers`: list of fp16 ``[S, n_tokens, D]``."""
    out = []
    for (codes, scale, zero), bits in zip(payloads, bits_per_layer):
        if keys:
            out.append(ref.decode_k(codes, scale, zero, n_tokens, bits[0], group_size))
        else:
            out.append(ref.decode_v(codes, scale, zero, n_tokens, bits[1], group_size, head_dim))
    return out
