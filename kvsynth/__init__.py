"""Seeded synthetic KV-cache workloads.

This module serves both sides of every comparison: the CPU oracle's tests and the GPU
library's tests and benchmark draw their inputs here. It holds none of the compression
method's arithmetic (no scoring, eviction, Hadamard rotation, lattice step or coding). It
only draws Gaussian keys and values, scales a few outlier channels, and applies the
*model's* forward split-half rotary embedding to the keys, so that the keys look like a
real prefill cache written by a Llama/Mistral/Qwen-style layer.

Workload shapes follow the page "NexusQuant：无需训练实现LLM KV缓存10-33倍压缩的技术突破"
(section "压缩效果与性能表现": Mistral-7B, Phi-3-mini, Qwen2.5-7B caches; preset table) and
"Como comprimir o KV cache do seu LLM em 33x sem treino" (section "Os números": Mistral-7B,
FP16). No dataset is used; the values are i.i.d. N(0,1) with outlier channels.

Recipe (all in numpy, layer by layer, so any one layer can be rebuilt alone):
  * ``K0, V0 = default_rng([seed, layer, kind]).standard_normal((H, T, 128), float32)``,
    kind 0 = keys, 1 = values;
  * outlier channels per (layer, head, tensor): ``default_rng([seed, layer, kind, 1])``
    draws ``choice(128, n_out, replace=False)`` once per head, in head order, and those
    channels are multiplied by the outlier factor (before the rotary embedding);
  * keys get the forward split-half rotary embedding at positions 0..T-1 with
    theta_i = base**(-i/64): for i < 64,
    k_i = x_i*cos - x_{i+64}*sin, k_{i+64} = x_{i+64}*cos + x_i*sin, in float32 with
    cos/sin rounded from float64 angles; then both tensors are rounded to float16.
  * single-token decode queries: ``default_rng([seed, 99]).standard_normal`` -> float16.
  * observation-window queries (the attention scorer's stand-in for a model's last W query
    rows): ``default_rng([seed, layer, 2]).standard_normal((Hq, W, 128), float32)``, given the
    same forward rotary embedding at positions T - W .. T - 1, then float16.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
import os

import numpy as np

HEAD_DIM = 128


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    kv_heads: int
    tokens: int
    window: int
    evict_permille: int
    bits_k: int
    bits_v: int
    rope_base: float
    k_outliers: tuple  # (channels per head, factor)
    v_outliers: tuple
    protect_boundary: int
    seed: int
    q_heads: int = 0  # >0: a single-token GQA decode step follows

    @property
    def layer_begin(self) -> int:
        return self.protect_boundary

    @property
    def layer_end(self) -> int:
        return self.layers - self.protect_boundary

    @property
    def compressed_layers(self) -> int:
        return self.layer_end - self.layer_begin

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the build: 0 is the small parity case, 1 the Mistral-7B-shaped
# balanced preset (the headline), 2 the long-context max preset, 3 the Qwen2.5-7B-shaped
# high preset with protected boundary layers, 4 the decode + GQA step over workload 2.
WORKLOADS = {
    0: Workload("small-1x8x2048-K3V2-e600-W128", 1, 8, 2048, 128, 600, 3, 2, 1e4,
                (4, 8.0), (4, 8.0), 0, 1000),
    1: Workload("mistral7b-32x8x32768-balanced-K3V2-e600-W256", 32, 8, 32768, 256, 600, 3, 2,
                1e4, (4, 8.0), (4, 8.0), 0, 1001),
    2: Workload("longctx-32x8x131072-max-K2V2-e800-W512", 32, 8, 131072, 512, 800, 2, 2, 1e4,
                (4, 8.0), (4, 8.0), 0, 1002),
    3: Workload("qwen2.5-7b-28x4x65536-high-K3V2-e350-W256-pb2", 28, 4, 65536, 256, 350, 3, 2,
                1e6, (8, 20.0), (4, 8.0), 2, 1003),
    4: Workload("decode-gqa32-of-longctx-32x8x131072", 32, 8, 131072, 512, 800, 2, 2, 1e4,
                (4, 8.0), (4, 8.0), 0, 1002, q_heads=32),
}


def workload(idx: int) -> Workload:
    return WORKLOADS[idx]


_TABLE_CACHE: dict = {}


def _rope_cos_sin(tokens: int, base: float):
    """float32 cos/sin of float64 angles p*base**(-i/64), shape [tokens, 64] each."""
    key = (tokens, float(base))
    if key not in _TABLE_CACHE:
        theta = np.power(np.float64(base), -np.arange(64, dtype=np.float64) / 64.0)
        phi = np.arange(tokens, dtype=np.float64)[:, None] * theta[None, :]
        _TABLE_CACHE.clear()
        _TABLE_CACHE[key] = (np.cos(phi).astype(np.float32), np.sin(phi).astype(np.float32))
    return _TABLE_CACHE[key]


def _draw(w: Workload, layer: int, kind: int, tokens: int) -> np.ndarray:
    rng = np.random.default_rng([w.seed, layer, kind])
    x = rng.standard_normal((w.kv_heads, tokens, HEAD_DIM), dtype=np.float32)
    n_out, factor = w.k_outliers if kind == 0 else w.v_outliers
    if n_out:
        crng = np.random.default_rng([w.seed, layer, kind, 1])
        for h in range(w.kv_heads):
            ch = crng.choice(HEAD_DIM, n_out, replace=False)
            x[h][:, ch] *= np.float32(factor)
    return x


def layer_keys(w: Workload, layer: int, tokens: int | None = None) -> np.ndarray:
    """float16 keys [H, T, 128] of one layer (rotary embedding applied)."""
    T = w.tokens if tokens is None else tokens
    x = _draw(w, layer, 0, T)
    c, s = _rope_cos_sin(T, w.rope_base)
    out = np.empty(x.shape, dtype=np.float16)
    lo, hi = x[..., :64], x[..., 64:]
    out[..., :64] = (lo * c - hi * s).astype(np.float16)
    out[..., 64:] = (hi * c + lo * s).astype(np.float16)
    return out


def layer_values(w: Workload, layer: int, tokens: int | None = None) -> np.ndarray:
    """float16 values [H, T, 128] of one layer."""
    T = w.tokens if tokens is None else tokens
    return _draw(w, layer, 1, T).astype(np.float16)


def layer_kv(w: Workload, layer: int, tokens: int | None = None):
    return layer_keys(w, layer, tokens), layer_values(w, layer, tokens)


def fill_kv(w: Workload, K: np.ndarray, V: np.ndarray, layers=None, threads: int | None = None):
    """Fill preallocated float16 arrays K, V [L, H, T, 128] layer by layer (threaded)."""
    layers = range(w.layers) if layers is None else layers
    threads = threads or min(8, os.cpu_count() or 1)
    T = K.shape[2]

    def one(l):
        K[l] = layer_keys(w, l, T)
        V[l] = layer_values(w, l, T)

    _rope_cos_sin(T, w.rope_base)  # build the shared table once, outside the threads
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, layers))


def queries(w: Workload, q_heads: int | None = None) -> np.ndarray:
    """float16 single-token queries [compressed layers, q_heads, 128]."""
    hq = q_heads or w.q_heads or 4 * w.kv_heads
    rng = np.random.default_rng([w.seed, 99])
    return rng.standard_normal((w.compressed_layers, hq, HEAD_DIM),
                               dtype=np.float32).astype(np.float16)


def window_queries(w: Workload, layer: int, q_heads: int | None = None,
                   tokens: int | None = None) -> np.ndarray:
    """float16 queries [q_heads, W, 128] of one layer's observation window: query w sits at
    position T - W + w and carries the forward rotary embedding of that position (positions
    below 0, when W > T, are left unrotated; the scorer ignores those rows)."""
    T = w.tokens if tokens is None else tokens
    hq = q_heads or w.q_heads or 4 * w.kv_heads
    W = w.window
    x = np.random.default_rng([w.seed, layer, 2]).standard_normal((hq, W, HEAD_DIM),
                                                                   dtype=np.float32)
    c, s = _rope_cos_sin(max(T, 1), w.rope_base)
    pos = T - W + np.arange(W)
    ok = pos >= 0
    cc = np.ones((W, 64), np.float32)
    ss = np.zeros((W, 64), np.float32)
    cc[ok], ss[ok] = c[pos[ok]], s[pos[ok]]
    out = np.empty(x.shape, dtype=np.float16)
    lo, hi = x[..., :64], x[..., 64:]
    out[..., :64] = (lo * cc - hi * ss).astype(np.float16)
    out[..., 64:] = (hi * cc + lo * ss).astype(np.float16)
    return out
