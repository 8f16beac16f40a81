"""The host zstd stage (kv_cache_compression_proxy_amd.entropy): the wrapper round-trips bytes,
compresses what must compress and leaves incompressible bytes alone; and the measured
post-entropy ratio of the oracle's own compressed layer (CPU only; the GPU's delta streams are
bit-identical to the oracle's, so the same sizes follow for them)."""
import numpy as np
import pytest

import kvsynth
import oracle

entropy = pytest.importorskip("kv_cache_compression_proxy_amd.entropy")


def test_round_trip_and_known_sizes():
    rng = np.random.default_rng(3)
    x = rng.integers(-3, 4, 100_000).astype(np.int8)
    assert np.array_equal(entropy.decompress(entropy.compress(x), x.nbytes).view(np.int8), x)
    zeros = np.zeros(1 << 20, np.uint8)
    assert len(entropy.compress(zeros)) < 200                      # a run compresses away
    noise = rng.integers(0, 256, 1 << 20).astype(np.uint8)
    assert len(entropy.compress(noise)) > 0.99 * noise.nbytes      # random bytes do not shrink
    # 7 equiprobable symbols in bytes: an entropy coder lands near log2(7) = 2.81 bits/byte
    r = x.nbytes / len(entropy.compress(x, 19))
    assert 8 / 2.81 * 0.85 < r <= 8 / 2.81 * 1.01


def test_measured_ratio_of_oracle_layer():
    w = kvsynth.workload(0)
    T = w.tokens
    K, V = kvsynth.layer_kv(w, 0)
    Ct, St = oracle.rope_table(T, w.rope_base)
    enc = oracle.compress_layer(K, V, w.window, w.evict_permille, w.bits_k, w.bits_v, Ct, St)
    sizes = entropy.layer_sizes(enc["codes_k"], enc["codes_v"], enc["scales_k"].view(np.float16),
                                enc["scales_v"].view(np.float16), T)
    n = enc["positions"].size
    nominal = oracle.nominal_ratio(w.kv_heads, T, n, w.bits_k, w.bits_v)
    raw = sizes["fp16_kv"] / (sizes["codes_raw"] + sizes["scales_raw"] + sizes["keep_bitmap"])
    print(f"\n[entropy] workload 0 layer 0: zstd ratio {sizes['ratio']:.2f} "
          f"(raw int8 storage {raw:.2f}, nominal {nominal:.2f}); codes "
          f"{sizes['codes_raw'] / sizes['codes_zstd']:.2f}x under zstd, scales "
          f"{sizes['scales_raw'] / sizes['scales_zstd']:.2f}x")
    assert sizes["ratio"] > raw                 # the entropy stage gains on int8 storage
    assert sizes["codes_zstd"] < sizes["codes_raw"]
