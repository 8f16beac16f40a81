"""Pins of the attention-weight scorer oracle (oracle/attn_scorer.py) to facts fixed by the
mathematics, not by the oracle's own formula: each softmax row carries unit mass; zero queries
give uniform weights over the visible prefix (closed form); two visible keys give the logistic
function of the scaled logit difference; the causal mask reaches exactly the query's own
position; grouped query heads read kv head j // G; a common shift of the keys cancels."""
import numpy as np
import pytest

import kvsynth
from oracle.attn_scorer import attn_scores

rng = np.random.default_rng(11)


def rand(*shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float16)


@pytest.mark.parametrize("H,G,T,W", [(2, 4, 50, 8), (1, 1, 7, 7), (2, 2, 5, 9)])
def test_unit_mass_per_visible_query(H, G, T, W):
    K, Q = rand(H, T, 128), rand(H * G, W, 128)
    s = attn_scores(K, Q)
    rows = sum(1 for w in range(W) if T - W + w >= 0)
    assert abs(s.sum() - H * G * rows) < 1e-9


def test_zero_queries_give_uniform_weights():
    H, G, T, W = 2, 2, 40, 6
    K, Q = rand(H, T, 128), np.zeros((H * G, W, 128), np.float16)
    s = attn_scores(K, Q)
    pos = T - W + np.arange(W)
    ref = np.array([H * G * sum(1.0 / (P + 1) for P in pos if P >= t) for t in range(T)])
    assert np.max(np.abs(s - ref)) < 1e-12


def test_two_keys_is_the_logistic_of_the_scaled_difference():
    K, Q = rand(1, 2, 128), rand(1, 1, 128)
    s = attn_scores(K, Q)
    q, k0, k1 = (x.astype(np.float64) for x in (Q[0, 0], K[0, 0], K[0, 1]))
    d = (q @ k1 - q @ k0) / np.sqrt(128.0)
    assert abs(s[0] - 1.0 / (1.0 + np.exp(d))) < 1e-12
    assert abs(s[1] - 1.0 / (1.0 + np.exp(-d))) < 1e-12


def test_causal_mask_reaches_the_own_position_only():
    # the last key is strongly aligned with every query, but only the last query sees it
    H, G, T, W = 1, 3, 30, 5
    K, Q = rand(H, T, 128, scale=0.1), np.zeros((G, W, 128), np.float16)
    v = np.zeros(128, np.float32)
    v[:8] = 8.0
    K[0, T - 1] = v
    Q[:, :] = v
    s = attn_scores(K, Q)
    assert abs(s[T - 1] - G) < 1e-9      # weight ~1 from the last query of each head
    # and the next-to-last key gets (nearly) all of query W - 2's mass: it is that query's own
    # position and its largest logit is exp-dominant only through the alignment of K[T - 2]
    K2 = K.copy()
    K2[0, T - 2] = v
    s2 = attn_scores(K2, Q)
    assert abs(s2[T - 2] - G * (1.0 + 0.5)) < 1e-9   # all of query W-2, half of query W-1


def test_query_heads_read_kv_head_j_div_g():
    H, G, T, W = 2, 2, 25, 4
    K, Q = rand(H, T, 128), rand(H * G, W, 128)
    K[1] = 0.0                                       # kv head 1: all logits 0 -> uniform
    s = attn_scores(K, Q)
    pos = T - W + np.arange(W)
    uniform = np.array([G * sum(1.0 / (P + 1) for P in pos if P >= t) for t in range(T)])
    head0 = attn_scores(K[:1], Q[:G])                # query heads 0..G-1 only, on kv head 0
    assert np.max(np.abs(s - (head0 + uniform))) < 1e-12


def test_common_key_shift_cancels():
    H, G, T, W = 1, 2, 20, 4
    K, Q = rand(H, T, 128).astype(np.float64), rand(H * G, W, 128)
    c = rng.standard_normal(128)
    assert np.max(np.abs(attn_scores(K + c, Q) - attn_scores(K, Q))) < 1e-12


def test_window_queries_shape_and_rotation():
    w = kvsynth.workload(0)
    Q = kvsynth.window_queries(w, 0, q_heads=4)
    assert Q.shape == (4, w.window, 128) and Q.dtype == np.float16
    # the rotation preserves each (i, i + 64) pair's norm up to fp16 rounding
    x = np.random.default_rng([w.seed, 0, 2]).standard_normal((4, w.window, 128),
                                                              dtype=np.float32)
    n0 = x[..., :64] ** 2 + x[..., 64:] ** 2
    n1 = Q[..., :64].astype(np.float32) ** 2 + Q[..., 64:].astype(np.float32) ** 2
    assert np.max(np.abs(n1 - n0) / (n0 + 1e-3)) < 5e-3
