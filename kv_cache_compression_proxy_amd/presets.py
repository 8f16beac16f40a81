"""Quality presets of the method ("NexusQuant：无需训练实现LLM KV缓存10-33倍压缩的技术突破",
section "压缩效果与性能表现": high / asym / balanced / max; "Como comprimir o KV cache do seu LLM
em 33x sem treino", section "Os números": high / balanced / max).

The pages name the presets and their ratios but not their parameters; the values here are the
readings used for the benchmarked workloads: balanced = K3V2 with 60% eviction (the pages' 60%
eviction and K3V2 example), max = K2V2 with 80% eviction, high = K3V2 with 35% eviction and two
fp16 boundary layers on each side (the pages' K3V2-at-35% figure and protect_boundary option).
The recent-window lengths are not given by the pages. "asym" has no stated parameters and is not
provided.
"""
from __future__ import annotations

PRESETS = {
    "balanced": dict(bits_k=3, bits_v=2, evict_permille=600, window=256, protect_boundary=0),
    "max": dict(bits_k=2, bits_v=2, evict_permille=800, window=512, protect_boundary=0),
    "high": dict(bits_k=3, bits_v=2, evict_permille=350, window=256, protect_boundary=2),
}


def params_for(preset: str, layers: int, kv_heads: int, tokens: int, rope_base: float = 1e4,
               **overrides):
    from . import NqParams
    if preset not in PRESETS:
        raise ValueError(f"unknown preset {preset!r}; known: {sorted(PRESETS)}")
    cfg = dict(PRESETS[preset])
    cfg.update(overrides)
    pb = cfg.pop("protect_boundary")
    return NqParams(layers, kv_heads, tokens, 128, pb, layers - pb, cfg["window"],
                    cfg["evict_permille"], cfg["bits_k"], cfg["bits_v"], float(rope_base))
