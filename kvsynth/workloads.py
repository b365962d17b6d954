"""Synthetic KV-cache workloads.

The pages evaluate the codec inside Llama-2-7B and Mistral-7B inference
(CacheForge README, "Example", "GSM8K example", "Evaluate CacheForge on
LongBench").  Neither weights nor datasets are used here: each workload is a
seeded fp16 cache of the same *shape* (layers x batch x KV heads x tokens x
head_dim), with value distributions chosen to stress the codec (channel
outliers in the keys, heavy tails, per-channel bias, exact rounding ties).

Layout of one layer: float16 ``[B*H, T, D]``; slice ``j`` of layer ``l`` is
global slice ``l*B*H + j`` and belongs to KV head ``j % H``.

Seeds: the bulk Gaussian / Student-t draws of layer ``l`` come from a
Philox generator on the target device seeded with
``1000*c + 2*l + (0 for K, 1 for V)`` where ``c`` is the workload number;
structural choices (outlier channels, biases) come from CPU generators with
their own fixed seeds, so they are identical on every device.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    number: int
    name: str
    layers: int
    batch: int
    heads: int
    tokens: int
    head_dim: int
    k_bits: int
    v_bits: int
    group_size: int
    residual_length: int
    steps: int = 0          # streaming decode steps (0 = full-cache encode)
    q_per_kv: int = 1       # query heads per KV head at decode (grouped-query attention)
    fp8_keys: bool = False  # k8v4 layout: FP8 keys, values with one group per head
    boundary: int = 0       # first and last `boundary` layers take `boundary_bits` (per-layer mix)
    boundary_bits: tuple = (8, 8)

    @property
    def slices_per_layer(self) -> int:
        return self.batch * self.heads

    @property
    def slices(self) -> int:
        return self.layers * self.batch * self.heads


WORKLOADS = {
    "single_layer_4bit": Workload(1, "single layer, 8 heads, 512 tokens, 4/4-bit",
                                  1, 1, 8, 512, 128, 4, 4, 32, 128),
    "llama2_7b_2bit": Workload(2, "Llama-2-7B-shaped cache, batch 8, 4096 tokens, 2/2-bit",
                               32, 8, 32, 4096, 128, 2, 2, 32, 128),
    "mistral_7b_k2v4": Workload(3, "Mistral-7B-shaped GQA cache, batch 16, 16384 tokens, K2/V4",
                                32, 16, 8, 16384, 128, 2, 4, 32, 128, q_per_kv=4),
    "llama2_7b_k8v4": Workload(5, "Llama-2-7B-shaped cache, batch 8, 4096 tokens, FP8 keys + 4-bit values",
                               32, 8, 32, 4096, 128, 8, 4, 128, 128, fp8_keys=True),
    "llama2_7b_mix": Workload(6, "Llama-2-7B-shaped cache, batch 8, 4096 tokens, 2/2-bit with the first "
                                 "and last 2 layers at 8/8-bit", 32, 8, 32, 4096, 128, 2, 2, 32, 128,
                              boundary=2, boundary_bits=(8, 8)),
    "stream_b64": Workload(4, "streaming decode, batch 64, prefill 2048 + 512 steps, 2/2-bit",
                           32, 64, 8, 2048, 128, 2, 2, 32, 128, steps=512),
}


def slice_index(w: Workload, layer: int, b: int, h: int) -> int:
    return (layer * w.batch + b) * w.heads + h


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _student_t4(shape, gen, device):
    """Student-t with 4 degrees of freedom: N(0,1) / sqrt(chi2_4 / 4)."""
    z = _normal(shape, gen, device)
    chi2 = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(4):
        chi2 += _normal(shape, gen, device).square()
    return z / torch.sqrt(chi2 / 4.0)


def _single_layer_key_outliers(w: Workload, D: int) -> torch.Tensor:
    """4 channels per head, drawn without replacement with seed 1, scaled x20."""
    g = _gen("cpu", 1)
    mult = torch.ones(w.heads, D)
    for h in range(w.heads):
        ch = torch.randperm(D, generator=g)[:4]
        mult[h, ch] = 20.0
    return mult


def _bernoulli_key_outliers(w: Workload, layer: int, D: int) -> torch.Tensor:
    """Each (layer, head, channel) is an outlier with p = 0.02, scaled x15."""
    g = _gen("cpu", 20_000 + layer)
    hit = torch.rand(w.heads, D, generator=g) < 0.02
    return torch.where(hit, torch.tensor(15.0), torch.tensor(1.0))


def _key_bias(w: Workload, layer: int, D: int) -> torch.Tensor:
    """Per-(layer, head, channel) key bias ~ N(0, sigma=3)."""
    g = _gen("cpu", 30_000 + layer)
    return torch.randn(w.heads, D, generator=g) * 3.0


def layer_kv(w: Workload, layer: int, device="cpu", tokens: int | None = None):
    """fp16 K and V of one layer, ``[B*H, T, D]`` each (T = ``tokens`` or the
    workload's prefill length)."""
    T = w.tokens if tokens is None else tokens
    D = w.head_dim
    shape = (w.batch, w.heads, T, D)
    gk = _gen(device, 1000 * w.number + 2 * layer + 0)
    gv = _gen(device, 1000 * w.number + 2 * layer + 1)
    if w.number == 3:
        k = _student_t4(shape, gk, device)
        v = _student_t4(shape, gv, device)
        k += _key_bias(w, layer, D).to(device)[None, :, None, :]
    else:
        k = _normal(shape, gk, device)
        v = _normal(shape, gv, device)
        if w.number == 1:
            k *= _single_layer_key_outliers(w, D).to(device)[None, :, None, :]
        elif w.number in (2, 6):
            k *= _bernoulli_key_outliers(w, layer, D).to(device)[None, :, None, :]
    k = k.to(torch.float16).reshape(w.batch * w.heads, T, D)
    v = v.to(torch.float16).reshape(w.batch * w.heads, T, D)
    return k, v


def decode_queries(w: Workload, device="cpu"):
    """One decode step's query vectors for every slice: fp16
    ``[L*B*H, q_per_kv, D]``, N(0,1) (seed ``1000*c + 950``)."""
    g = _gen(device, 1000 * w.number + 950)
    return _normal((w.slices, w.q_per_kv, w.head_dim), g, device).to(torch.float16)


def stream_tokens(w: Workload, steps: int, device="cpu"):
    """Tokens appended during streaming decode, for all layers at once:
    fp16 ``[steps, L*B*H, D]`` for K and for V, N(0,1)."""
    S = w.slices
    gk = _gen(device, 1000 * w.number + 900)
    gv = _gen(device, 1000 * w.number + 901)
    k = _normal((steps, S, w.head_dim), gk, device).to(torch.float16)
    v = _normal((steps, S, w.head_dim), gv, device).to(torch.float16)
    return k, v


# ---------------------------------------------------------------------------
# edge shapes: uniform[-8, 8] with exact rounding ties
# ---------------------------------------------------------------------------

def _grid_step(bits: int) -> float:
    """Largest power of two s with (2**bits - 1) * s <= 16 (the width of
    [-8, 8])."""
    levels = 2 ** bits - 1
    s = 1.0
    while levels * s > 16.0:
        s /= 2.0
    while levels * (2 * s) <= 16.0:
        s *= 2.0
    return s


def uniform_with_ties(S: int, T: int, D: int, *, axis: str, n_valid: int,
                      bits: int, group_size: int, seed: int,
                      grid_group_fraction: float = 0.08,
                      tie_fraction_in_group: float = 0.125) -> np.ndarray:
    """fp16 ``[S, T, D]`` uniform on [-8, 8], with a fraction of its groups
    rebuilt on a known grid so that some elements fall exactly half-way
    between two reconstruction levels.

    ``axis='token'`` groups run along tokens per channel (key grouping),
    ``axis='channel'`` along channels per token (value grouping); only the
    first ``n_valid`` tokens belong to groups.

    A grid group has minimum ``m`` and maximum ``m + (2**bits - 1)*s`` for a
    power of two ``s`` and a multiple ``m`` of ``s/2``; all its other
    elements lie in between, and about ``tie_fraction_in_group`` of them sit
    at ``m + (k + 1/2)*s``.  Every one of these numbers is exact in fp16 for
    the sizes used here (|x| <= 8, s/2 >= 2**-7).  With 8% grid groups and
    1/8 ties per grid group, about 1% of the elements are ties.
    """
    rng = np.random.default_rng(seed)
    x = rng.uniform(-8.0, 8.0, size=(S, T, D)).astype(np.float16)
    G = group_size
    levels = 2 ** bits - 1
    s_max = _grid_step(bits)
    if axis == "token":
        ng = -(-n_valid // G)
        groups = [(s, g, d) for s in range(S) for g in range(ng) for d in range(D)]
    elif axis == "channel":
        ng = -(-D // G)
        groups = [(s, t, g) for s in range(S) for t in range(n_valid) for g in range(ng)]
    else:
        raise ValueError(axis)
    if not groups:
        return x
    n_pick = max(1, int(round(grid_group_fraction * len(groups))))
    picks = rng.choice(len(groups), size=n_pick, replace=False)
    for p in picks:
        if axis == "token":
            s, g, d = groups[p]
            t0, t1 = g * G, min((g + 1) * G, n_valid)
            view = x[s, t0:t1, d]
        else:
            s, t, g = groups[p]
            c0, c1 = g * G, min((g + 1) * G, D)
            view = x[s, t, c0:c1]
        n = view.shape[0]
        if n < 3:
            continue
        step = s_max / (2 ** int(rng.integers(0, 3)))
        half = step / 2
        top = 8.0 - levels * step
        m = -8.0 + half * int(rng.integers(0, int((top + 8.0) / half) + 1))
        vals = (m + rng.uniform(0.0, 1.0, size=n) * levels * step).astype(np.float16)
        order = rng.permutation(n)
        vals[order[0]] = m
        vals[order[1]] = m + levels * step
        n_ties = max(1, int(round(tie_fraction_in_group * n)))
        ks = rng.integers(0, levels, size=n_ties)
        vals[order[2:2 + n_ties]] = (m + (ks + 0.5) * step).astype(np.float16)
        view[:] = vals
    return x
