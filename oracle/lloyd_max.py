"""CPU oracle of the equal-bit scalar baseline -- TEST INFRASTRUCTURE ONLY (the test suite and
bench.py use it; the GPU library never imports it and shares no code with it).

The baseline keeps the lattice codec's front end (rotary embedding removed from keys, the
normalised 128-point Hadamard rotation, one fp16 scale per 8-float group) and replaces the E8
step by a per-coordinate Lloyd-Max quantizer for the unit Gaussian at the same bit budget
(3 bits for keys, 2 for values in the balanced preset). The page "Lloyd-Max量化" (sections
"从均匀量化到非均匀量化" and "量化过程详解") describes the quantizer: alternate nearest-level
assignment and centroid updates until they converge, then quantize by table lookup; its
"3-bit量化的设计选择" section fixes the 3-bit budget. After the rotation the coordinates are
close to Gaussian, so the tables are those of N(0, 1) and need no data.

Readings (the pages leave them open): the group scale is the fp16 (round to nearest even,
saturating at 65504 so that it stays finite) of the group's RMS, s = sqrt(sum(x_i^2) / 8) in
fp32 with the squares added in dim order; a
coordinate's index is the number of thresholds strictly below u = x / s (fp32 division, fp32
thresholds), so a value on a threshold takes the lower cell; an all-zero group (s = 0) takes
index 2^(b-1) everywhere (its reconstruction is 0 whatever the index).
"""
from __future__ import annotations

import functools
import math

import numpy as np

from . import fwht_f32, h2f, f2h_rne, rope_undo


def _phi(x: float) -> float:
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi) if math.isfinite(x) else 0.0


def _Phi(x: float) -> float:
    if x == math.inf:
        return 1.0
    if x == -math.inf:
        return 0.0
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def lloyd_max_gaussian(bits: int, tol: float = 1e-15, max_iter: int = 200000):
    """Lloyd-Max quantizer of N(0, 1) with 2^bits levels: alternate the two optimality
    conditions -- each threshold is the midpoint of its two levels (nearest-level assignment),
    each level is the mean of N(0, 1) over its cell (centroid) -- from uniform levels until the
    levels move less than tol. Returns (levels [2^b], thresholds [2^b - 1]) in float64."""
    n = 1 << bits
    y = np.linspace(-2.0, 2.0, n) if n > 1 else np.zeros(1)
    for _ in range(max_iter):
        t = 0.5 * (y[:-1] + y[1:])
        edges = [-math.inf, *t.tolist(), math.inf]
        y_new = np.array([(_phi(a) - _phi(b)) / (_Phi(b) - _Phi(a))
                          for a, b in zip(edges[:-1], edges[1:])])
        if np.max(np.abs(y_new - y)) < tol:
            y = y_new
            break
        y = y_new
    # N(0, 1) is symmetric: make the table exactly antisymmetric, so that the middle
    # threshold is exactly 0 (rounding noise of order 1e-17 would otherwise decide the side of 0)
    y = 0.5 * (y - y[::-1])
    return y, 0.5 * (y[:-1] + y[1:])


def gaussian_mse(levels: np.ndarray, thresholds: np.ndarray) -> float:
    """E[(X - Q(X))^2] for X ~ N(0, 1) in closed form (sum over cells of the second moment
    about the cell's level)."""
    edges = [-math.inf, *thresholds.tolist(), math.inf]
    d = 0.0
    for y, a, b in zip(levels.tolist(), edges[:-1], edges[1:]):
        P = _Phi(b) - _Phi(a)
        m1 = _phi(a) - _phi(b)                                       # int x phi
        am = a * _phi(a) if math.isfinite(a) else 0.0
        bm = b * _phi(b) if math.isfinite(b) else 0.0
        m2 = P + am - bm                                             # int x^2 phi
        d += m2 - 2.0 * y * m1 + y * y * P
    return d


@functools.lru_cache(maxsize=None)
def _tables_f32_cached(bits: int):
    y, t = lloyd_max_gaussian(bits)
    return y.astype(np.float32), t.astype(np.float32)


def tables_f32(bits: int):
    """The fp32 tables the quantizer compares and reconstructs with (copies of a cached pair)."""
    y, t = _tables_f32_cached(bits)
    return y.copy(), t.copy()


def quantize_group(x8: np.ndarray, bits: int):
    """x8: float32 [8] of the rotated row -> (scale fp16 bits, indices uint8 [8], near-tie)."""
    y32, t32 = tables_f32(bits)
    ss = np.float32(0.0)
    for v in x8.astype(np.float32):
        ss = np.float32(ss + np.float32(v * v))
    s32 = np.float32(np.sqrt(np.float32(ss * np.float32(0.125))))
    s16 = min(f2h_rne(float(s32)), 0x7BFF)   # saturating: an RMS above 65504 keeps 65504
    s = np.float32(h2f(s16))
    near = False
    # scale near-tie: fp32 RMS within 1e-6 relative of an fp16 rounding boundary
    if s32 > 0:
        lo, hi = h2f(max(s16 - 1, 0)), h2f(min(s16 + 1, 0x7bff))
        for b in ((lo + float(s)) / 2, (hi + float(s)) / 2):
            near |= abs(float(s32) - b) <= 1e-6 * float(s32)
    if s == 0:
        return s16, np.full(8, 1 << (bits - 1), np.uint8), near
    idx, u = indices_at(x8, s16, bits)
    for ui in u:
        near |= bool(np.any(np.abs(ui - t32) <= 1e-6 * np.maximum(1.0, np.abs(t32))))
    return s16, idx, near


def indices_at(x8: np.ndarray, s16: int, bits: int):
    """The quantizer step of one group at the fp16 scale bits s16 (nonzero): u = x / s in fp32,
    index = number of fp32 thresholds strictly below u. -> (indices uint8 [8], u float32 [8])."""
    _, t32 = tables_f32(bits)
    s = np.float32(h2f(int(s16)))
    u = (x8.astype(np.float32) / s).astype(np.float32)
    idx = np.array([int(np.sum(t32 < ui)) for ui in u], np.uint8)
    return idx, u


def encode_layer(K_l, V_l, positions, Ctab, Stab, bits_k: int, bits_v: int):
    """-> dict(idx_k, idx_v uint8 [H, n, 128], scales_k, scales_v fp16 bits [H, n, 16],
    near_k, near_v bool [H, n, 16])."""
    H = K_l.shape[0]
    n = len(positions)
    out = {k: None for k in ("idx_k", "idx_v", "scales_k", "scales_v", "near_k", "near_v")}
    for name, X, bits, is_key in (("k", K_l, bits_k, True), ("v", V_l, bits_v, False)):
        idx = np.zeros((H, n, 128), np.uint8)
        sc = np.zeros((H, n, 16), np.uint16)
        nr = np.zeros((H, n, 16), bool)
        for h in range(H):
            for j, p in enumerate(positions):
                row = X[h, p].astype(np.float32)
                x = rope_undo(row, Ctab[p], Stab[p]) if is_key else row
                x = fwht_f32(x)
                for g in range(16):
                    sc[h, j, g], idx[h, j, 8 * g:8 * g + 8], nr[h, j, g] = \
                        quantize_group(x[8 * g:8 * g + 8], bits)
        out["idx_" + name], out["scales_" + name], out["near_" + name] = idx, sc, nr
    return out


def decode_layer(idx_k, idx_v, scales_k, scales_v, positions, Ctab, Stab, bits_k, bits_v):
    """-> (K_hat, V_hat) float64 [H, n, 128]: x = s * level[index] per coordinate, the inverse
    normalised Hadamard transform (the transform is its own inverse), the rotary embedding at
    each kept position for keys. fp64 throughout."""
    outs = []
    for idx, sc, bits, is_key in ((idx_k, scales_k, bits_k, True),
                                  (idx_v, scales_v, bits_v, False)):
        y32, _ = tables_f32(bits)
        H, n, _ = idx.shape
        s = np.vectorize(h2f)(sc.astype(np.int64)).astype(np.float64)     # [H, n, 16]
        x = y32.astype(np.float64)[idx] * np.repeat(s, 8, axis=2)         # [H, n, 128]
        # inverse normalised Hadamard (Sylvester order), fp64
        x = x.copy()
        hlen = 1
        while hlen < 128:
            x = x.reshape(H, n, 128 // (2 * hlen), 2, hlen)
            a, b = x[..., 0, :].copy(), x[..., 1, :].copy()
            x[..., 0, :], x[..., 1, :] = a + b, a - b
            x = x.reshape(H, n, 128)
            hlen *= 2
        x = x / math.sqrt(128.0)
        if is_key:
            C = Ctab[np.asarray(positions)].astype(np.float64)[None]      # [1, n, 64]
            S = Stab[np.asarray(positions)].astype(np.float64)[None]
            lo, hi = x[..., :64].copy(), x[..., 64:].copy()
            x[..., :64] = lo * C - hi * S
            x[..., 64:] = hi * C + lo * S
        outs.append(x)
    return outs[0], outs[1]
