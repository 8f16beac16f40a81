"""Pins of the oracle's numeric building blocks against things other than itself: the binary16
format as numpy implements it, numpy/scipy library routines (cos/sin, Sylvester Hadamard
matrix), closed forms and invariants. CPU only."""
import numpy as np
import pytest
from scipy.linalg import hadamard

import oracle


# ---------------------------------------------------------------- binary16 conversions
def test_h2f_matches_numpy_all_patterns():
    L = oracle.lib()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([L.nqo_h2f(int(b)) for b in bits], np.float32)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


def test_f2h_rne_matches_numpy():
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-9, 5, 20000),
        # exact halfway points between binary16 neighbours (ties to even) and the edges
        ((np.arange(1, 4000, dtype=np.float32) + np.float32(0.5)) * np.float32(2.0 ** -24)),
        np.array([0.0, -0.0, 65504.0, 65519.0, 65520.0, 1e-8, 2.0 ** -25, 3 * 2.0 ** -26,
                  2.0 ** -14, 6.1e-5], np.float32)])
    with np.errstate(over="ignore"):                      # 65520 rounds to infinity
        ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f2h_rne(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, ref)


def test_f2h_ceil_is_smallest_binary16_not_below():
    rng = np.random.default_rng(8)
    vals = np.abs(rng.standard_normal(20000)).astype(np.float32) * np.float32(10.0) ** rng.integers(-8, 4, 20000)
    vals = np.concatenate([vals, np.float16(rng.random(2000)).astype(np.float32)])  # exact grid
    for v in vals:
        h = oracle.f2h_ceil(float(v))
        s = np.uint16(h).view(np.float16).astype(np.float32)
        assert s >= v
        if h > 0:
            below = np.uint16(h - 1).view(np.float16).astype(np.float32)
            assert below < v
    assert oracle.f2h_ceil(0.0) == 0
    assert oracle.f2h_ceil(1e9) == 0x7BFF  # saturates at 65504


# ---------------------------------------------------------------- rotary table and RoPE removal
@pytest.mark.parametrize("base", [1e4, 1e6])
def test_rope_table_against_numpy_cos_sin(base):
    T = 4096
    C, S = oracle.rope_table(T, base)
    theta = np.power(np.float64(base), -np.arange(64) / 64.0)
    phi = np.arange(T)[:, None] * theta[None, :]
    # glibc and numpy both give (nearly) correctly rounded fp64 cos/sin; after rounding to fp32
    # they agree except where the fp64 value sits within an ulp of an fp32 midpoint
    assert np.mean(C == np.cos(phi).astype(np.float32)) > 0.99999
    assert np.mean(S == np.sin(phi).astype(np.float32)) > 0.99999
    assert np.all(C[0] == 1.0) and np.all(S[0] == 0.0)      # position 0 is the identity
    assert np.max(np.abs(C.astype(np.float64) ** 2 + S.astype(np.float64) ** 2 - 1)) < 1e-6


def test_rope_undo_inverts_forward_rotation_and_keeps_norm():
    rng = np.random.default_rng(3)
    C, S = oracle.rope_table(70000, 1e4)
    for p in [0, 1, 17, 4095, 69999]:
        x = rng.standard_normal(128).astype(np.float32)
        c, s = C[p].astype(np.float64), S[p].astype(np.float64)
        # forward rotation written independently in fp64 (the model's convention)
        k = np.concatenate([x[:64] * c - x[64:] * s, x[64:] * c + x[:64] * s]).astype(np.float32)
        back = oracle.rope_undo(k, C[p], S[p])
        assert np.max(np.abs(back - x)) < 2e-6 * np.max(np.abs(x)) + 1e-7
        assert abs(np.linalg.norm(back) - np.linalg.norm(k)) < 1e-6 * np.linalg.norm(k)
        if p == 0:
            assert np.array_equal(oracle.rope_undo(k, C[0], S[0]), k)


# ---------------------------------------------------------------- Hadamard rotation
def test_fwht_is_sylvester_hadamard_over_sqrt128():
    H = hadamard(128).astype(np.float64) / np.sqrt(128.0)   # scipy's Sylvester construction
    rng = np.random.default_rng(4)
    X = rng.standard_normal((200, 128))
    for x in X:
        got = oracle.fwht_f64(x)
        assert np.max(np.abs(got - H @ x)) < 1e-12
        got32 = oracle.fwht_f32(x.astype(np.float32)).astype(np.float64)
        assert np.max(np.abs(got32 - H @ x.astype(np.float32))) < 5e-6


def test_fwht_orthonormal_involution_and_basis():
    I = np.eye(128)
    cols = np.stack([oracle.fwht_f64(e) for e in I], axis=1)   # the transform's matrix
    assert np.max(np.abs(cols @ cols.T - I)) < 1e-12             # H H^T = I
    assert np.allclose(cols[:, 0], 1 / np.sqrt(128.0), atol=0, rtol=1e-15)  # H e0 = 1/sqrt(128)
    rng = np.random.default_rng(5)
    x = rng.standard_normal(128)
    assert np.max(np.abs(oracle.fwht_f64(oracle.fwht_f64(x)) - x)) < 1e-13   # own inverse
    assert abs(np.linalg.norm(oracle.fwht_f64(x)) - np.linalg.norm(x)) < 1e-12


# ---------------------------------------------------------------- proxy score
def test_scores_equal_double_sum_over_window_and_heads():
    """The collapsed form sum_h <qbar_h, k_t> equals sum_h sum_w <k_{h,w}, k_{h,t}> (brute
    force, independent association)."""
    rng = np.random.default_rng(6)
    H, T, W = 3, 50, 7
    K = (rng.standard_normal((H, T, 128)) * 3).astype(np.float16)
    s = oracle.layer_scores(K, W)
    Kd = K.astype(np.float64)
    for t in range(T):
        if 1 <= t < T - W:
            ref = sum(float(np.dot(Kd[h, w], Kd[h, t])) for h in range(H) for w in range(T - W, T))
            assert abs(s[t] - ref) <= 1e-12 * max(1.0, abs(ref))
        else:
            assert np.isnan(s[t])


@pytest.mark.parametrize("base", [1e4, 1e6])
def test_rope_table_matches_transformers_llama_rotary(base):
    """The model convention from a library: transformers' LlamaRotaryEmbedding (split-half
    layout, inv_freq = base^(-2i/d) with d = 128, computed there in fp32). Its cos/sin over the
    first 256 positions equal the oracle's table to within that library's fp32 angle error, and
    its two halves repeat the 64 frequencies (pairs i and i + 64)."""
    transformers = pytest.importorskip("transformers")
    import torch
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding
    cfg = transformers.LlamaConfig(hidden_size=1024, num_attention_heads=8, head_dim=128,
                                   rope_theta=base, max_position_embeddings=4096)
    rot = LlamaRotaryEmbedding(config=cfg)
    P = 256
    c, s = rot(torch.zeros(1, P, 128), torch.arange(P)[None])
    c, s = c[0].double().numpy(), s[0].double().numpy()
    assert np.array_equal(c[:, :64], c[:, 64:]) and np.array_equal(s[:, :64], s[:, 64:])
    C, S = oracle.rope_table(P, base)
    # fp32 angles p * inv_freq in the library: |error| <= ~P * 2^-24
    assert np.abs(c[:, :64] - C).max() < 4e-5
    assert np.abs(s[:, :64] - S).max() < 4e-5
