"""CPU oracle of the attention-weight scorer -- TEST INFRASTRUCTURE ONLY (the test suite and
bench.py's CPU-baseline leg use it; the GPU library never imports it and shares no code with it).

What it computes (the page "NexusQuant：无需训练实现LLM KV缓存10-33倍压缩的技术突破", sections
"Token淘汰机制" -- tokens are scored by their attention weights, BOS and a recent window are always
kept -- and "技术实现细节" -- the scorer can be the cheap key-key proxy or a real attention scorer
that costs an extra pass): the attention weights that an observation window of W queries (one
block per query head, query w at position P_w = T - W + w) gives to every key, summed over the
window and over all query heads:

    s_t = sum_j sum_w [t <= P_w] softmax_{t' <= P_w}(q_{j,w} . k_{h(j),t'} / sqrt(128))_t

with h(j) = j // (Hq / H) (grouped-query heads share kv heads) and the causal mask t <= P_w.
Keys are used as stored (rotary embedding applied), queries as given. Evaluated in float64 from
the fp16 inputs; one matrix product per query head is the only library step.
"""
from __future__ import annotations

import numpy as np


def attn_scores(K_l: np.ndarray, Q_l: np.ndarray) -> np.ndarray:
    """K_l: fp16 [H, T, 128] keys of one layer; Q_l: fp16 [Hq, W, 128] window queries.
    Returns float64 [T]: s_t for every position t (BOS and window keys included)."""
    K = np.asarray(K_l, dtype=np.float64)
    Q = np.asarray(Q_l, dtype=np.float64)
    H, T, D = K.shape
    Hq, W, _ = Q.shape
    G = Hq // H
    s = np.zeros(T, dtype=np.float64)
    for j in range(Hq):
        Z = (Q[j] @ K[j // G].T) / np.sqrt(float(D))      # [W, T] scaled logits
        for w in range(W):
            P = T - W + w                                   # the query's position
            if P < 0:
                continue
            z = Z[w, :P + 1]                                # causal: keys 0..P only
            e = np.exp(z - z.max())
            s[:P + 1] += e / e.sum()
    return s
