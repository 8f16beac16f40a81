"""Pins of the oracle's near-tie classification, the part of the tolerance rule that decides
which GPU results may differ from the oracle's (lattice codes and keep-sets are compared bit
for bit except inside these bands):
- Voronoi near-tie: u's distance to the nearest facet of its E8 Voronoi cell is below
  1e-6 * max(1, |u|_inf);
- scale near-tie: fp32(a / rho) lies within 1e-6 relative of a binary16 value at which the
  rounded-up scale changes;
- eviction near-tie: a candidate's score lies within 1e-6 relative of the m-th best score;
- for the equal-bit Lloyd-Max baseline: a coordinate within 1e-6 * max(1, |t|) of a threshold
  t, or the fp32 RMS within 1e-6 relative of a binary16 rounding boundary.
Every input is built at a known distance from its band's edge: half the band (must be flagged)
and twice the band (must not be), so a rule that flags everything, nothing, or uses a band a
thousand times too wide fails here. The facet distance is measured independently of the
oracle, over the 240 enumerated roots of E8. CPU only.
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle import lloyd_max as lm


def e8_roots() -> np.ndarray:
    """The 240 minimal vectors of E8: the 112 permutations of (+-1, +-1, 0^6) and the 128
    vectors (+-1/2)^8 with an even number of minus signs."""
    r = []
    for i, j in itertools.combinations(range(8), 2):
        for si in (-1.0, 1.0):
            for sj in (-1.0, 1.0):
                v = np.zeros(8)
                v[i], v[j] = si, sj
                r.append(v)
    for signs in itertools.product((-0.5, 0.5), repeat=8):
        if sum(s < 0 for s in signs) % 2 == 0:
            r.append(np.array(signs))
    return np.array(r)


ROOTS = e8_roots()


def facet_distance(u, y) -> float:
    """Distance of u to the nearest facet of the Voronoi cell of the lattice point y:
    min over roots r of (|r|^2/2 - (u - y).r) / |r| (negative: u is outside the cell)."""
    e = np.asarray(u, np.float64) - np.asarray(y, np.float64)
    return float(np.min((1.0 - ROOTS @ e) / np.sqrt(2.0)))


def test_root_enumeration():
    assert ROOTS.shape == (240, 8)
    assert np.all(np.sum(ROOTS ** 2, axis=1) == 2.0)
    assert len({tuple(r) for r in ROOTS}) == 240


def facet_group(rho: int, d: float, kind: str):
    """A rotated 8-float group whose scale is exactly 1 (so u = x) and whose nearest E8 point
    y lies at facet distance d from u. Coordinates 6 and 7 hold the group's largest value
    A = rho (1 - 2^-12), so a / rho = 1 - 2^-12 is far from every binary16 step (no scale
    near-tie) and |u|_inf = A. kind 'root2': the facet toward y + (1, 1, 0^6) (both points in
    D8); kind 'root8': the facet toward y + (1/2^6, -1/2, -1/2), a point of D8 + 1/2."""
    A = np.float32(rho * (1.0 - 2.0 ** -12))
    lam = 1.0 - np.sqrt(2.0) * d          # e.r for the facet's root: facet distance (1-lam)/sqrt2
    y = np.array([0, 0, 0, 0, 0, 0, rho, rho], np.float64)
    if kind == "root2":
        h = lam / 2
        u = np.array([h, h, 0, 0, 0, 0, A, A])
    else:
        c = (lam - rho * 2.0 ** -12) / 3   # e.r = 3c - (A - rho) = lam
        u = np.array([c, c, c, c, c, c, A, A])
    return u.astype(np.float32), y


def band(umax: float) -> float:
    return 1e-6 * max(1.0, umax)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("kind", ["root2", "root8"])
@pytest.mark.parametrize("factor", [0.0, 0.5, 2.0])
def test_voronoi_near_tie_band(bits, kind, factor):
    rho = (1 << (bits - 1)) - 1
    A = float(np.float32(rho * (1.0 - 2.0 ** -12)))
    u, y = facet_group(rho, factor * band(A), kind)
    d = facet_distance(u, y)
    assert abs(d - factor * band(A)) <= 0.05 * band(A), d          # built where intended
    row = np.zeros(128, np.float32)
    row[:8] = u
    s16, c, flags = oracle.quantize_row(row, bits)
    assert s16[0] == 0x3C00                                          # scale exactly 1: u = x
    gu, umax = oracle.group_u(row[:8], s16[0], bits)
    assert np.array_equal(gu, u) and umax == A
    if factor > 0:
        assert np.array_equal(c[:8] / 2.0, y)                        # y is the nearest point
    # the facet distance of the oracle's own point, measured independently
    assert abs(facet_distance(u, c[:8] / 2.0) - d) <= 1e-9 or factor == 0.0
    want = factor < 1.0
    assert bool(flags[0] & 1) == want, (bits, kind, factor, d, flags[0])
    assert oracle.voronoi_near_tie(u, c[:8]) == want
    assert not flags[0] & 2                                          # no scale near-tie
    assert not np.any(flags[1:])                                     # all-zero groups


def test_voronoi_band_grows_with_the_largest_coordinate():
    """At |u|_inf = 7 the band is 7e-6: facet distance 3.5e-6 is flagged, though it is far
    outside a fixed 1e-6 band."""
    A = float(np.float32(7 * (1.0 - 2.0 ** -12)))
    u, y = facet_group(7, 3.5e-6, "root2")
    assert facet_distance(u, y) > 3e-6
    row = np.zeros(128, np.float32)
    row[:8] = u
    _, _, flags = oracle.quantize_row(row, 4)
    assert flags[0] & 1
    assert band(A) > 6.9e-6


def scale_group(rho: int, v: float, delta: float) -> np.ndarray:
    """A group with a / rho = v (1 + delta) and u near (rho, 1, 0^6), a lattice point deep
    inside its Voronoi cell (no Voronoi near-tie)."""
    w = np.float32(v * (1.0 + delta))
    x = np.zeros(8, np.float32)
    x[0] = np.float32(rho * np.float64(w))
    x[1] = w
    return x


STEPS = [
    (0x3E00, 1.5),               # a normal binary16 value
    (0x3A00, 0.75),
    (0x0010, 16 * 2.0 ** -24),    # a subnormal binary16 value (steps 2^-24 apart)
    (0x63D0, 1000.0),
]


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("h,v", STEPS)
@pytest.mark.parametrize("delta,want", [(0.0, True), (0.5e-6, True), (-0.5e-6, True),
                                        (2e-6, False), (-2e-6, False)])
def test_scale_near_tie_band(bits, h, v, delta, want):
    rho = (1 << (bits - 1)) - 1
    assert oracle.h2f(h) == v
    row = np.zeros(128, np.float32)
    row[:8] = scale_group(rho, v, delta)
    s16, c, flags = oracle.quantize_row(row, bits)
    # the rounded-up scale: v itself unless a / rho lies above it
    assert s16[0] == (h + 1 if delta > 0 else h)
    assert bool(flags[0] & 2) == want, (bits, v, delta, flags[0])
    assert not flags[0] & 1


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("v,delta,want,s16", [
    # just above the step below the largest binary16: the scale saturates at 65504, and a
    # slightly smaller a / rho would give 65472
    (65472.0, 0.5e-6, True, 0x7BFF),
    (65472.0, 2e-6, False, 0x7BFF),
    # at or above 65504 every nearby a / rho keeps the saturated scale
    (65504.0, 0.0, False, 0x7BFF),
    (65504.0, 0.5e-6, False, 0x7BFF),
    (65504.0, 1e-3, False, 0x7BFF),
])
def test_scale_near_tie_at_saturation(bits, v, delta, want, s16):
    rho = (1 << (bits - 1)) - 1
    row = np.zeros(128, np.float32)
    row[:8] = scale_group(rho, v, delta)
    got_s16, c, flags = oracle.quantize_row(row, bits)
    assert got_s16[0] == s16
    assert bool(flags[0] & 2) == want, (bits, v, delta, flags[0])


@pytest.mark.parametrize("tau", [3.75, -2.5, 1234.5])
def test_eviction_near_tie_band(tau):
    """m = 10 candidates are kept; the 10th best score is tau. Candidates at tau(1 +- 0.5e-6)
    (relative to |tau|) are flagged, at tau(1 +- 2e-6) are not, and nothing else is."""
    W, T, e = 4, 25, 400
    assert oracle.keep_count(T, W, e) - (W + 1) == 10
    a = abs(tau)
    cands = ([tau + 10 * a + k for k in range(7)] +
             [tau + 2e-6 * a, tau + 0.5e-6 * a, tau, tau - 0.5e-6 * a, tau - 2e-6 * a] +
             [tau - 5 * a - k for k in range(8)])
    near_want = [False] * 7 + [False, True, True, True, False] + [False] * 8
    rng = np.random.default_rng(5)
    order = rng.permutation(20)                       # candidate slots 1..20, scrambled
    s = np.full(T, np.nan)
    want = np.zeros(T, bool)
    for k, slot in enumerate(order):
        s[1 + slot] = cands[k]
        want[1 + slot] = near_want[k]
    pos, near, th = oracle.select_layer(s, W, e)
    assert th == tau
    assert np.array_equal(near.astype(bool), want), (np.nonzero(near)[0], np.nonzero(want)[0])
    kept = set(pos.tolist())
    assert all((1 + order[k]) in kept for k in range(10))


def test_eviction_no_threshold_no_flags():
    """With nothing evicted (or nothing kept among the candidates) there is no threshold and
    no candidate is a near-tie."""
    s = np.concatenate([[np.nan], np.linspace(1, 2, 40), [np.nan] * 4])
    for e in (0, 1000):
        _, near, th = oracle.select_layer(s, 4, e)
        assert not near.any()
        assert np.isnan(th)


# ---- the equal-bit Lloyd-Max baseline's bands --------------------------------------------------
def lm_threshold_group(u0: float) -> np.ndarray:
    """A group whose RMS is 1 to within a few ulps (scale 1: u = x) with u_0 = u0."""
    c = np.float32(np.sqrt((8.0 - np.float64(np.float32(u0)) ** 2) / 7.0))
    x = np.full(8, c, np.float32)
    x[0] = np.float32(u0)
    return x


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("factor,want", [(0.5, True), (-0.5, True), (2.0, False),
                                         (-2.0, False)])
def test_lloyd_max_threshold_band(bits, factor, want):
    _, t32 = lm.tables_f32(bits)
    for t in t32:
        u0 = float(t) + factor * 1e-6 * max(1.0, abs(float(t)))
        x = lm_threshold_group(u0)
        s16, idx, near = lm.quantize_group(x, bits)
        assert s16 == 0x3C00
        # the other coordinates sit far from every threshold
        assert np.min(np.abs(np.float64(x[1]) - t32.astype(np.float64))) > 1e-3
        assert near == want, (bits, float(t), factor)


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("delta,want", [(0.3e-6, True), (-0.3e-6, True), (3e-6, False),
                                        (-3e-6, False)])
def test_lloyd_max_scale_band(bits, delta, want):
    """The RMS near the binary16 rounding boundary 1 + 2^-11 (halfway between 1 and 1 + 2^-10);
    every coordinate is ~1, far from the thresholds."""
    m = 1.0 + 2.0 ** -11
    x = np.full(8, np.float32(m * (1.0 + delta)), np.float32)
    s16, idx, near = lm.quantize_group(x, bits)
    assert s16 in (0x3C00, 0x3C01)
    assert near == want, (bits, delta)
