"""Pins of the oracle's E8 nearest-point step: brute force over enumerated lattice
neighbourhoods, the textbook kissing number and second moment, lattice membership, the
covering radius and idempotence. CPU only."""
import itertools
import json
import os

import numpy as np

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "e8_textbook.json")))
OFFS = np.array(list(itertools.product((-1, 0, 1), repeat=8)), np.float64)   # 6561 x 8


def e8_candidates(u):
    """All E8 points within 1 of u in every coordinate (the covering radius is 1, so the
    nearest point is among them): integer points round(u)+{-1,0,1}^8 with even sum and
    half-integer points floor(u)+1/2+{-1,0,1}^8 with sum(y - 1/2) even."""
    u = np.asarray(u, np.float64)
    ci = np.round(u) + OFFS
    ci = ci[np.sum(ci, axis=1) % 2 == 0]
    ch = np.floor(u) + 0.5 + OFFS
    ch = ch[np.sum(ch - 0.5, axis=1) % 2 == 0]
    return np.concatenate([ci, ch])


def in_e8(y):
    y = np.asarray(y, np.float64)
    two = 2 * y
    if not np.all(two == np.round(two)):
        return False
    ints = np.all(y == np.round(y))
    halves = np.all(y - 0.5 == np.round(y - 0.5))
    if not (ints or halves):
        return False
    return (np.sum(y - (0.0 if ints else 0.5)) % 2) == 0


def test_enumerator_finds_240_minimal_vectors():
    pts = e8_candidates(np.zeros(8))
    n2 = np.sum(pts ** 2, axis=1)
    assert np.sum(n2 == 2.0) == GOLD["kissing_number"]["value"]
    assert np.min(n2[n2 > 0]) == 2.0


def test_oracle_matches_brute_force():
    rng = np.random.default_rng(11)
    U = np.concatenate([
        rng.uniform(-7.2, 7.2, (1500, 8)),
        rng.uniform(-1.0, 1.0, (1500, 8)),
        rng.standard_normal((500, 8)) * 3,
        # structured points: near lattice points, deep holes, half-integers
        np.round(rng.uniform(-3, 3, (200, 8))) + rng.normal(0, 1e-3, (200, 8)),
        np.tile([1.0, 0, 0, 0, 0, 0, 0, 0], (1, 1)),          # deep hole of E8
        np.full((1, 8), 0.25),
    ]).astype(np.float32)
    codes, margin = oracle.e8_nearest(U)
    for u, c, m in zip(U, codes, margin):
        y = c.astype(np.float64) / 2
        assert in_e8(y)
        cand = e8_candidates(u)
        d = np.sum((cand - u.astype(np.float64)) ** 2, axis=1)
        dy = np.sum((y - u.astype(np.float64)) ** 2)
        assert dy <= d.min() + 1e-12                       # y is a nearest point
        assert dy <= 1.0 + 1e-12                           # covering radius 1
        assert m >= -1e-12                                 # Voronoi certificate holds
        if m > 1e-9:                                       # away from a facet: unique argmin
            assert np.sum(d <= dy + 1e-9) == 1


def test_certificate_detects_non_nearest_points():
    """A D8-only decoder is often wrong; the facet distance must then be negative."""
    rng = np.random.default_rng(12)
    U = rng.uniform(-3, 3, (2000, 8)).astype(np.float32)
    wrong = 0
    for u in U:
        f = np.round(u.astype(np.float64))
        if np.sum(f) % 2:
            j = np.argmax(np.abs(u - f))
            f[j] += 1.0 if u[j] > f[j] else -1.0
        m = oracle.e8_margin(u, (2 * f).astype(np.int8))
        best = np.min(np.sum((e8_candidates(u) - u) ** 2, axis=1))
        if np.sum((f - u) ** 2) > best + 1e-9:
            wrong += 1
            assert m < 0
        else:
            assert m >= -1e-12
    assert wrong > 100


def test_idempotent_on_lattice_points():
    rng = np.random.default_rng(13)
    z = rng.integers(-5, 6, (3000, 8)).astype(np.float64)
    z[:, 0] += np.sum(z, axis=1) % 2                       # even sum: D8
    half = rng.random(3000) < 0.5
    z[half] += 0.5                                         # sum(z+1/2 - 1/2) even: D8 + 1/2
    codes, margin = oracle.e8_nearest(z.astype(np.float32))
    assert np.array_equal(codes.astype(np.float64) / 2, z)
    assert np.allclose(margin, 1 / np.sqrt(2.0))


def test_normalized_second_moment():
    rng = np.random.default_rng(14)
    U = rng.uniform(-4, 4, (200000, 8)).astype(np.float32)
    codes, _ = oracle.e8_nearest(U)
    e = U.astype(np.float64) - codes / 2.0
    G = np.mean(np.sum(e ** 2, axis=1)) / 8
    assert abs(G - GOLD["normalized_second_moment"]["value"]) < 4e-4
    # a Z^8 quantizer would give 1/12; D8-only decoding also lands well above E8's value
    assert G < 0.074


def test_exact_tie_rules():
    """The oracle's rules on exact ties (measure zero; the readings of the nearest-point step):
    the integer coset wins a distance tie, rint rounds ties to even, and a coordinate with zero
    error moves toward zero when the parity fix falls on it."""
    cases = [
        ([0.25] * 8, [0] * 8),                     # both cosets at squared distance 1/2
        ([2.5, 0.5, 0, 0, 0, 0, 0, 0], [4, 0, 0, 0, 0, 0, 0, 0]),   # ties to even: (2, 0, ...)
        ([1, 0, 0, 0, 0, 0, 0, 0], [0] * 8),       # odd sum, all errors 0: index 0 moves to 0
        ([-1, 0, 0, 0, 0, 0, 0, 0], [0] * 8),
    ]
    for u, want in cases:
        c, _ = oracle.e8_nearest(np.array([u], np.float32))
        assert list(c[0]) == want, (u, list(c[0]))
