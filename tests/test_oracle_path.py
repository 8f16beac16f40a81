"""Pins of the oracle's path-level steps: eviction (brute force, invariants, the pages' 2.5x at
60%), group scales and codes (scale rule, composition with the lattice step), delta coding,
reconstruction bounds, the attention check (torch's library attention) and the nominal ratio.
CPU only."""
import json
import os

import itertools

import numpy as np
import pytest
import torch

import kvsynth
import oracle

PAGES = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


# ---------------------------------------------------------------- eviction
@pytest.mark.parametrize("T,W,e", [(40, 5, 600), (40, 0, 600), (9, 3, 600), (5, 10, 600),
                                   (1, 0, 600), (64, 8, 0), (64, 8, 1000), (200, 16, 350)])
def test_select_brute_force(T, W, e):
    rng = np.random.default_rng(T * 1000 + W * 10 + e)
    s = np.round(rng.standard_normal(T) * 4) / 4           # coarse values: many exact ties
    pos, near, tau = oracle.select_layer(s, W, e)
    n_keep = max(T - (e * T) // 1000, min(T, 1 + W))
    assert len(pos) == n_keep
    prot = {0} | set(range(max(1, T - W), T))
    cand = [t for t in range(1, max(1, T - W))]
    m = n_keep - len(prot)
    order = sorted(cand, key=lambda t: (-s[t], t))          # score desc, position asc
    expect = sorted(prot | set(order[:m]))
    assert list(pos) == expect
    assert np.all(np.diff(pos) > 0)


def test_zero_window_scores_tie_and_lowest_positions_win():
    K = np.ones((2, 30, 128), np.float16)
    s = oracle.layer_scores(K, 0)                          # empty window: all scores zero
    assert np.all(s[1:] == 0)
    pos, _, _ = oracle.select_layer(s, 0, 600)
    assert list(pos) == list(range(len(pos)))


def test_bos_and_window_always_kept_and_60pct_gives_2_5x():
    w = kvsynth.workload(0)
    K = kvsynth.layer_keys(w, 0)
    s = oracle.layer_scores(K, w.window)
    pos, near, tau = oracle.select_layer(s, w.window, w.evict_permille)
    assert pos[0] == 0
    assert set(range(w.tokens - w.window, w.tokens)) <= set(pos.tolist())
    ref = PAGES["eviction_60pct_token_reduction"]
    assert w.evict_permille == int(1000 * ref["evict_fraction"])
    for T in (2048, 32768, 131072):
        assert abs(T / oracle.keep_count(T, 128, 600) - ref["value"]) < 2.5 ** 2 / T + 1e-9


# ---------------------------------------------------------------- scale and lattice step
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantize_row_scale_rule_and_composition(bits):
    rho = float(2 ** (bits - 1) - 1)
    rng = np.random.default_rng(20 + bits)
    for trial in range(300):
        x = (rng.standard_normal(128) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        if trial == 0:
            x[:8] = 0                                      # an all-zero group
            # groups whose a/rho exceeds the fp16 range: the scale saturates at 65504 and the
            # clamp to [-rho, rho] decides the point
            x[8:16] = [1e6, 0, 3, 0, 0, 0, 0, 0]
            x[16:24] = [-1e6, 0, 0, -5, 0, 0, 0, 0]
        s16, c, fl = oracle.quantize_row(x, bits)
        for g in range(16):
            xg = x[8 * g:8 * g + 8]
            a = np.float32(np.max(np.abs(xg)))
            if a == 0:
                assert s16[g] == 0 and np.all(c[8 * g:8 * g + 8] == 0)
                continue
            v = np.float32(a / np.float32(rho))             # IEEE fp32 division (numpy)
            s = np.uint16(s16[g]).view(np.float16).astype(np.float32)
            below = np.uint16(s16[g] - 1).view(np.float16).astype(np.float32)
            if v > 65504:
                assert s16[g] == 0x7BFF                    # saturated
            else:
                assert s >= v and below < v                # smallest binary16 >= a/rho
            u = np.clip(xg / s, -rho, rho).astype(np.float32)
            assert np.max(np.abs(u)) <= rho
            cref, _ = oracle.e8_nearest(u[None])
            assert np.array_equal(c[8 * g:8 * g + 8], cref[0])
            assert np.max(np.abs(c[8 * g:8 * g + 8])) <= 2 * rho + 2


@pytest.mark.parametrize("bits,limit", [(2, 2 ** 16), (3, 2 ** 24)])
def test_bit_budget_is_honest(bits, limit):
    """With |u| <= rho every emitted point has |y_i| <= rho + 1/2 (covering radius 1 and the
    lattice structure); the E8 points in that cube number fewer than 2^(8b)."""
    rho = 2 ** (bits - 1) - 1
    rng = np.random.default_rng(30 + bits)
    u = rng.uniform(-rho, rho, (20000, 8)).astype(np.float32)
    c, _ = oracle.e8_nearest(u)
    assert np.max(np.abs(c)) <= 2 * rho + 1
    r = rho + 0.5
    ints = np.arange(-rho, rho + 1)
    halves = np.arange(-rho - 0.5, rho + 1)
    # count lattice points in [-r, r]^8 by parity classes of the coordinate sum
    def count(vals, offset):
        ways = {0: 1}
        for _ in range(8):
            nxt = {}
            for par, n in ways.items():
                for v in vals:
                    p = (par + int(round(v - offset))) % 2
                    nxt[p] = nxt.get(p, 0) + n
            ways = nxt
        return ways[0]
    total = count(ints, 0.0) + count(halves, 0.5)
    assert total < limit


# ---------------------------------------------------------------- delta coding and reconstruction
def test_constant_values_give_zero_deltas_and_roundtrip():
    rng = np.random.default_rng(40)
    H, T = 2, 64
    K = rng.standard_normal((H, T, 128)).astype(np.float16)
    V = np.broadcast_to(rng.standard_normal((H, 1, 128)), (H, T, 128)).astype(np.float16).copy()
    Ct, St = oracle.rope_table(T, 1e4)
    pos = np.arange(0, T, 3, dtype=np.int32)
    enc = oracle.encode_layer(K, V, pos, Ct, St, 3, 2)
    assert np.all(enc["codes_v"][:, 1:] == 0)
    # the prefix sum of the deltas restores the absolute codes of every token
    absk = np.cumsum(enc["codes_k"].astype(np.int64), axis=1)
    absk = ((absk + 128) % 256 - 128).astype(np.int8)
    for h in range(H):
        for j, p in enumerate(pos):
            x = oracle.fwht_f32(oracle.rope_undo(K[h, p].astype(np.float32), Ct[p], St[p]))
            _, c, _ = oracle.quantize_row(x, 3)
            assert np.array_equal(absk[h, j], c)


def test_running_sum_wraps_mod_256():
    """Decode's running sum is taken mod 256 as int8, whatever the byte stream: deltas of 100
    give the codes 100, -56, 44, -112 (values decode to H(s*c/2), and H is its own inverse)."""
    H, n = 1, 4
    d = np.full((H, n, 128), 100, np.int8)
    sc = np.full((H, n, 16), oracle.f2h_rne(1.0), np.uint16)
    Ct, St = oracle.rope_table(4, 1e4)
    pos = np.arange(n, dtype=np.int32)
    _, Vh = oracle.decode_layer(d, d, sc, sc, pos, Ct, St)
    want = ((np.cumsum(d.astype(np.int64), axis=1) + 128) % 256 - 128).astype(np.float64)
    assert list(want[0, :, 0]) == [100, -56, 44, -112]
    for j in range(n):
        assert np.allclose(2.0 * oracle.fwht_f64(Vh[0, j]), want[0, j], atol=1e-9)


def test_lattice_exact_rows_roundtrip():
    """Rows built as s*y with y on E8 are reconstructed to fp64 rounding."""
    rng = np.random.default_rng(41)
    H, n = 2, 16
    codes = np.zeros((H, n, 128), np.int8)
    absc = np.zeros((H, n, 128), np.int64)
    for h in range(H):
        for j in range(n):
            u = rng.uniform(-3, 3, (16, 8)).astype(np.float32)
            c, _ = oracle.e8_nearest(u)
            absc[h, j] = c.reshape(-1)
    codes[:, 0] = absc[:, 0]
    codes[:, 1:] = ((absc[:, 1:] - absc[:, :-1]) % 256).astype(np.uint8).view(np.int8)
    scales = np.float16(rng.uniform(0.01, 2, (H, n, 16))).view(np.uint16)
    pos = np.arange(n, dtype=np.int32) * 5
    Ct, St = oracle.rope_table(100, 1e4)
    Kh, Vh = oracle.decode_layer(codes, codes, scales, scales, pos, Ct, St)
    x = scales.view(np.float16).astype(np.float64).repeat(8, axis=-1) * absc / 2.0
    from scipy.linalg import hadamard
    Hm = hadamard(128) / np.sqrt(128.0)
    xr = x @ Hm.T
    assert np.max(np.abs(Vh - xr)) < 1e-12
    c, s = Ct[pos].astype(np.float64), St[pos].astype(np.float64)
    kr = np.concatenate([xr[..., :64] * c - xr[..., 64:] * s, xr[..., 64:] * c + xr[..., :64] * s], -1)
    assert np.max(np.abs(Kh - kr)) < 1e-12


def test_reconstruction_error_within_covering_bound():
    w = kvsynth.workload(0)
    K, V = kvsynth.layer_kv(w, 0, tokens=400)
    Ct, St = oracle.rope_table(400, w.rope_base)
    enc = oracle.compress_layer(K, V, 32, 600, 3, 2, Ct, St)
    Kh, Vh = oracle.decode_layer(enc["codes_k"], enc["codes_v"], enc["scales_k"],
                                 enc["scales_v"], enc["positions"], Ct, St)
    for X, Xh, sc in ((K, Kh, enc["scales_k"]), (V, Vh, enc["scales_v"])):
        Xk = X[:, enc["positions"]].astype(np.float64)
        err = np.linalg.norm(Xk - Xh, axis=-1)
        s = sc.view(np.float16).astype(np.float64)
        bound = np.sqrt(np.sum(s ** 2, axis=-1))           # per group |u - y| <= 1
        assert np.all(err <= bound * (1 + 1e-5) + 1e-4)


# ---------------------------------------------------------------- attention check
def test_attend_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(50)
    Hq, H, n = 8, 2, 37
    q = rng.standard_normal((Hq, 128)).astype(np.float16)
    K = rng.standard_normal((H, n, 128))
    V = rng.standard_normal((H, n, 128))
    out = oracle.attend_layer(q, K, V)
    qt = torch.from_numpy(q.astype(np.float64)).view(1, Hq, 1, 128)
    kt = torch.from_numpy(K).repeat_interleave(Hq // H, 0).view(1, Hq, n, 128)
    vt = torch.from_numpy(V).repeat_interleave(Hq // H, 0).view(1, Hq, n, 128)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).view(Hq, 128).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12


def test_attend_special_cases():
    q = np.zeros((4, 128), np.float16)                     # zero query: uniform weights
    V = np.random.default_rng(51).standard_normal((1, 9, 128))
    out = oracle.attend_layer(q, np.ones((1, 9, 128)), V)
    assert np.allclose(out, V[0].mean(0)[None], atol=1e-14)
    one = oracle.attend_layer(np.ones((4, 128), np.float16), np.ones((1, 1, 128)), V[:, :1])
    assert np.allclose(one, V[0, 0][None], atol=0)
    # logits far beyond exp's range: with the maximum subtracted the weights are one-hot on the
    # largest logit (the textbook softmax, not inf / inf)
    qb = np.zeros((1, 128), np.float16)
    qb[0, 0] = 60000
    Kb = np.zeros((1, 3, 128))
    Kb[0, :, 0] = [0.0, 1000.0, 2000.0]
    big = oracle.attend_layer(qb, Kb, V[:, :3])
    assert np.all(np.isfinite(big)) and np.allclose(big[0], V[0, 2], atol=0)


# ---------------------------------------------------------------- nominal ratio
def test_nominal_ratio_closed_form():
    """Bits per kept token per layer: H*(128*(bK+bV) + 2*16*16) + 32 (scales and positions
    counted, as the pages count overhead); compared with 2*H*128*16 bits of fp16."""
    w = kvsynth.workload(1)
    n = oracle.keep_count(w.tokens, w.window, w.evict_permille)
    assert n == 13108
    r = oracle.nominal_ratio(w.kv_heads, w.tokens, n, w.bits_k, w.bits_v)
    bits_out = n * (w.kv_heads * (128 * (w.bits_k + w.bits_v) + 16 * 16 * 2) + 32)
    assert r == pytest.approx(2 * w.kv_heads * 128 * 16 * w.tokens / bits_out, rel=1e-12)
    assert r == pytest.approx(8.858, abs=1e-3)
    # with no eviction and no overhead the pattern reduces to the pages' 16/b (3 bits: 5.33x)
    b = PAGES["three_bit_theoretical_ratio"]
    assert 16 / b["bits"] == pytest.approx(b["value"], abs=5e-3)
    bare = (2 * 128 * 16) / (128 * 2 * b["bits"])
    assert bare == pytest.approx(b["value"], abs=5e-3)


def _codebook_size(bits: int) -> int:
    """E8 points y with |y_i| <= rho + 1/2 (every point the quantizer can emit), counted by
    brute force over the integer and half-integer cubes for b = 2, and by the parity generating
    function otherwise: n integer vectors in [-rho, rho]^8 with even sum plus half-integer ones
    whose sum of (y_i - 1/2) is even."""
    rho = (1 << (bits - 1)) - 1
    if bits == 2:
        ints = np.array(list(itertools.product(range(-rho, rho + 1), repeat=8)))
        halves = np.array(list(itertools.product(range(-rho - 1, rho + 1), repeat=8)))
        return int(np.sum(ints.sum(1) % 2 == 0) + np.sum(halves.sum(1) % 2 == 0))
    n_int = 2 * rho + 1                       # values -rho..rho; sum of (-1)^v over them is -1
    n_half = 2 * rho + 2                      # z = y - 1/2 in -rho-1..rho; sum of (-1)^z is 0
    return (n_int ** 8 + 1) // 2 + n_half ** 8 // 2


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_size_fits_the_budget(bits):
    n = _codebook_size(bits)
    assert 2 ** (8 * bits - 1) < n <= 2 ** (8 * bits)        # 8b bits index a group, no fewer
    if bits == 2:
        assert n == 36049
    if bits == 3:
        assert n == 11271009


def test_nominal_ratio_counted_from_the_oracle_output():
    """The nominal ratio from what the oracle actually emits for a layer: each 8-float group as
    a fixed-length index into its codebook (ceil(log2 size) bits, the size counted above), the
    fp16 scale arrays and the int32 positions, in bytes as produced; against the fp16 cache's
    2 * H * T * 128 * 16 bits."""
    w = kvsynth.workload(0).with_(tokens=600)
    K, V = kvsynth.layer_kv(w, 0)
    C, S = oracle.rope_table(w.tokens, w.rope_base)
    enc = oracle.compress_layer(K, V, w.window, w.evict_permille, w.bits_k, w.bits_v, C, S)
    H, n = w.kv_heads, enc["positions"].size
    groups = H * n * 16                                          # per tensor
    code_bits = groups * sum(int(np.ceil(np.log2(_codebook_size(b))))
                             for b in (w.bits_k, w.bits_v))
    other_bits = 8 * (enc["scales_k"].nbytes + enc["scales_v"].nbytes + enc["positions"].nbytes)
    assert enc["positions"].dtype == np.int32 and enc["scales_k"].dtype == np.uint16
    ratio = (2 * H * w.tokens * 128 * 16) / (code_bits + other_bits)
    assert oracle.nominal_ratio(H, w.tokens, n, w.bits_k, w.bits_v) == pytest.approx(ratio,
                                                                                       rel=1e-12)
