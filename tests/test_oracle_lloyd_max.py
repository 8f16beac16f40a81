"""Pins of the scalar-baseline oracle (oracle/lloyd_max.py): the Lloyd-Max tables of N(0, 1)
against the 1-bit closed form and against Max's published 2- and 3-bit tables (J. Max,
"Quantizing for minimum distortion", IRE Trans. Inf. Theory 6(1), 1960, Table I; 4 printed
digits); the centroid condition by numerical integration; the closed-form distortion against a
Monte Carlo estimate; and group quantization on inputs whose answer is known."""
import math

import numpy as np
import pytest
from scipy import integrate

import oracle
from oracle.lloyd_max import (decode_layer, gaussian_mse, lloyd_max_gaussian, quantize_group,
                              tables_f32)


def test_one_bit_closed_form():
    y, t = lloyd_max_gaussian(1)
    assert abs(y[1] - math.sqrt(2 / math.pi)) < 1e-12 and abs(y[0] + y[1]) < 1e-15
    assert abs(t[0]) < 1e-15
    assert abs(gaussian_mse(y, t) - (1 - 2 / math.pi)) < 1e-12


@pytest.mark.parametrize("bits,levels,thresholds,mse", [
    (2, [0.4528, 1.510], [0.0, 0.9816], 0.1175),
    (3, [0.2451, 0.7560, 1.344, 2.152], [0.0, 0.5006, 1.050, 1.748], 0.03454),
])
def test_published_tables(bits, levels, thresholds, mse):
    y, t = lloyd_max_gaussian(bits)
    n = 1 << bits
    assert np.allclose(y[n // 2:], levels, atol=6e-4) and np.allclose(y, -y[::-1], atol=1e-14)
    assert np.allclose(t[n // 2 - 1:], thresholds, atol=6e-4)
    assert abs(gaussian_mse(y, t) - mse) < 1e-4


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_centroid_and_midpoint_conditions(bits):
    y, t = lloyd_max_gaussian(bits)
    edges = [-np.inf, *t, np.inf]
    pdf = lambda x: math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)
    for k in range(len(y)):
        a, b = edges[k], edges[k + 1]
        m0 = integrate.quad(pdf, a, b, epsabs=1e-14)[0]
        m1 = integrate.quad(lambda x: x * pdf(x), a, b, epsabs=1e-14)[0]
        assert abs(m1 / m0 - y[k]) < 1e-8
    assert np.allclose(t, 0.5 * (y[:-1] + y[1:]), atol=1e-15)


@pytest.mark.parametrize("bits", [2, 3])
def test_distortion_matches_monte_carlo(bits):
    y, t = lloyd_max_gaussian(bits)
    x = np.random.default_rng(5).standard_normal(2_000_000)
    q = y[np.searchsorted(t, x)]
    assert abs(np.mean((x - q) ** 2) / gaussian_mse(y, t) - 1) < 0.01


def test_group_quantization_known_answers():
    y32, t32 = tables_f32(3)
    # levels whose RMS is r = 0.989: every level / r' for r' in [0.9, 1.1] stays inside its own
    # cell of the 3-bit table (cells: 0 | 0.5006 | 1.050 | 1.748, mirrored), so a group
    # c * levels[idx] must come back as idx with scale c * r
    idx = np.array([0, 6, 2, 5, 3, 4, 3, 4])
    r = math.sqrt(np.mean(y32[idx].astype(np.float64) ** 2))
    assert 0.95 < r < 1.05
    c = 3.7
    x = (y32[idx] * np.float32(c)).astype(np.float32)
    s_got, i_got, _ = quantize_group(x, 3)
    assert abs(oracle.h2f(s_got) / (c * r) - 1) < 1e-3     # fp16 rounding of the RMS
    assert np.array_equal(i_got, idx)
    z16, z_idx, _ = quantize_group(np.zeros(8, np.float32), 2)
    assert z16 == 0 and np.all(z_idx == 2)
    # a coordinate exactly on a threshold takes the lower cell: u = 0 sits on the middle
    # threshold, which is exactly 0 (the tables are antisymmetric)
    for bits in (2, 3, 4):
        _, on_idx, _ = quantize_group(np.array([0, 1, -1, 1, -1, 1, -1, 1], np.float32), bits)
        assert on_idx[0] == (1 << (bits - 1)) - 1
    # an RMS beyond the fp16 range keeps the largest finite scale; u then lies beyond every
    # threshold in magnitude, so the indices are the outermost cells
    big = np.array([2e5, -2e5, 2e5, -2e5, 2e5, -2e5, 2e5, -2e5], np.float32)
    b16, b_idx, _ = quantize_group(big, 3)
    assert b16 == 0x7BFF and list(b_idx) == [7, 0, 7, 0, 7, 0, 7, 0]


def test_decode_inverts_the_rotation():
    # indices and scales chosen directly: decode must equal the inverse Hadamard (its own
    # inverse) of s * level, computed here with the oracle's fp64 transform
    rng = np.random.default_rng(9)
    idx = rng.integers(0, 8, (1, 1, 128)).astype(np.uint8)
    sc = np.full((1, 1, 16), oracle.f2h_rne(0.5), np.uint16)
    y32, _ = tables_f32(3)
    Ct, St = oracle.rope_table(4, 1e4)
    Kh, Vh = decode_layer(idx, idx, sc, sc, np.array([2]), Ct, St, 3, 3)
    ref = oracle.fwht_f64(0.5 * y32.astype(np.float64)[idx[0, 0]])
    assert np.max(np.abs(Vh[0, 0] - ref)) < 1e-15
    # keys get the rotary embedding of their position back: removing it with the pinned
    # RoPE removal of the codec (fp32) returns the rotated-back row
    back = oracle.rope_undo(Kh[0, 0].astype(np.float32), Ct[2], St[2]).astype(np.float64)
    assert np.max(np.abs(back - ref)) < 1e-6 * np.max(np.abs(ref))
