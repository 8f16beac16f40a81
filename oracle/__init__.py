"""CPU oracle for the KV-cache compression hot path (ctypes wrapper over nq_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` use it. The GPU library never imports it and shares no code with it.

Every function here is marshalling only; the arithmetic lives in nq_oracle.c, which cites the
pages' passages step by step. Arrays are numpy; fp16 data travels as uint16 bit patterns. Two
numpy modules sit beside it: attn_scorer.py (the attention-weight scorer) and lloyd_max.py (the
equal-bit scalar baseline).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None

_P = np.ctypeslib.ndpointer
_u16 = _P(np.uint16, flags="C_CONTIGUOUS")
_i8 = _P(np.int8, flags="C_CONTIGUOUS")
_u8 = _P(np.uint8, flags="C_CONTIGUOUS")
_i32 = _P(np.int32, flags="C_CONTIGUOUS")
_f32 = _P(np.float32, flags="C_CONTIGUOUS")
_f64 = _P(np.float64, flags="C_CONTIGUOUS")


def lib():
    global _lib
    if _lib is None:
        # NQ_ORACLE_LIB names another build of nq_oracle.c to load (the pin tests' mutants)
        path = os.environ.get("NQ_ORACLE_LIB")
        if path is None:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        L = C.CDLL(path)
        sig = {
            "nqo_h2f": (C.c_float, [C.c_uint16]),
            "nqo_f2h_rne": (C.c_uint16, [C.c_float]),
            "nqo_f2h_ceil": (C.c_uint16, [C.c_float]),
            "nqo_rope_table": (None, [C.c_int32, C.c_double, _f32, _f32]),
            "nqo_layer_scores": (None, [_u16, C.c_int32, C.c_int32, C.c_int32, _f64]),
            "nqo_keep_count": (C.c_int32, [C.c_int32, C.c_int32, C.c_int32]),
            "nqo_select_layer": (C.c_int32, [_f64, C.c_int32, C.c_int32, C.c_int32, _i32, _u8,
                                             C.POINTER(C.c_double)]),
            "nqo_rope_undo": (None, [_f32, _f32, _f32, _f32]),
            "nqo_fwht_f32": (None, [_f32]),
            "nqo_fwht_f64": (None, [_f64]),
            "nqo_e8_nearest_many": (None, [_f32, C.c_int64, _i8, _f64]),
            "nqo_e8_margin": (C.c_double, [_f32, _i8]),
            "nqo_quantize_row": (None, [_f32, C.c_int32, _u16, _i8, _u8]),
            "nqo_group_u": (C.c_float, [_f32, C.c_uint16, C.c_int32, _f32]),
            "nqo_voronoi_near_tie": (C.c_int, [_f32, _i8, C.c_float]),
            "nqo_scale_near_tie": (C.c_int, [C.c_float, C.c_uint16]),
            "nqo_encode_layer": (None, [_u16, _u16, C.c_int32, C.c_int32, _i32, C.c_int32, _f32,
                                        _f32, C.c_int32, C.c_int32, _i8, _i8, _u16, _u16, _u8,
                                        _u8]),
            "nqo_decode_layer": (None, [_i8, _i8, _u16, _u16, _i32, C.c_int32, C.c_int32, _f32,
                                        _f32, _f64, _f64]),
            "nqo_attend_layer": (None, [_u16, C.c_int32, _f64, _f64, C.c_int32, C.c_int32,
                                        _f64]),
            "nqo_nominal_ratio": (C.c_double, [C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                              C.c_int32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _bits(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return a


# --- scalar / small helpers (used by the pins) ----------------------------------------------
def h2f(h: int) -> float:
    return lib().nqo_h2f(h)


def f2h_rne(f: float) -> int:
    return lib().nqo_f2h_rne(f)


def f2h_ceil(f: float) -> int:
    return lib().nqo_f2h_ceil(f)


def keep_count(T: int, W: int, evict_permille: int) -> int:
    return lib().nqo_keep_count(T, W, evict_permille)


def rope_table(T: int, base: float):
    Cc = np.empty((T, 64), np.float32)
    Ss = np.empty((T, 64), np.float32)
    lib().nqo_rope_table(T, base, Cc, Ss)
    return Cc, Ss


def rope_undo(k: np.ndarray, Crow: np.ndarray, Srow: np.ndarray) -> np.ndarray:
    x = np.empty(128, np.float32)
    lib().nqo_rope_undo(np.ascontiguousarray(k, np.float32), np.ascontiguousarray(Crow, np.float32),
                        np.ascontiguousarray(Srow, np.float32), x)
    return x


def fwht_f32(x: np.ndarray) -> np.ndarray:
    y = np.array(x, np.float32, copy=True)
    lib().nqo_fwht_f32(y)
    return y


def fwht_f64(x: np.ndarray) -> np.ndarray:
    y = np.array(x, np.float64, copy=True)
    lib().nqo_fwht_f64(y)
    return y


def e8_nearest(u: np.ndarray):
    """u: float32 [..., 8] -> (codes int8 [..., 8] = 2y, Voronoi facet distance float64 [...])."""
    u = np.ascontiguousarray(u, np.float32)
    n = u.size // 8
    c = np.empty(u.shape, np.int8)
    m = np.empty(u.shape[:-1], np.float64)
    lib().nqo_e8_nearest_many(u.reshape(-1), n, c.reshape(-1), m.reshape(-1))
    return c, m


def e8_margin(u: np.ndarray, c: np.ndarray) -> float:
    """Distance of u - c/2 to the nearest facet of E8's Voronoi cell (negative: not nearest)."""
    return lib().nqo_e8_margin(np.ascontiguousarray(u, np.float32), np.ascontiguousarray(c, np.int8))


def quantize_row(x: np.ndarray, bits: int):
    """x: float32 [128] (already rotated) -> (scales fp16 bits [16], codes int8 [128], flags)."""
    s = np.empty(16, np.uint16)
    c = np.empty(128, np.int8)
    f = np.empty(16, np.uint8)
    lib().nqo_quantize_row(np.ascontiguousarray(x, np.float32), bits, s, c, f)
    return s, c, f


def group_u(xg: np.ndarray, s16: int, bits: int):
    """The lattice-step input of one rotated 8-float group at the fp16 scale bits s16:
    -> (u float32 [8], max |u|)."""
    u = np.empty(8, np.float32)
    m = lib().nqo_group_u(np.ascontiguousarray(xg, np.float32), int(s16), bits, u)
    return u, m


def voronoi_near_tie(u: np.ndarray, c: np.ndarray) -> bool:
    u = np.ascontiguousarray(u, np.float32)
    return bool(lib().nqo_voronoi_near_tie(u, np.ascontiguousarray(c, np.int8),
                                           float(np.abs(u).max())))


def scale_near_tie(v: float, s16: int) -> bool:
    """v = fp32(a / rho), s16 = its rounded-up fp16 scale bits."""
    return bool(lib().nqo_scale_near_tie(float(np.float32(v)), int(s16)))


def rotated_row(row16: np.ndarray, is_key: bool, Crow=None, Srow=None) -> np.ndarray:
    """The codec's front end for one stored fp16 row: RoPE removal (keys, at the row's
    position) then the normalised Hadamard rotation -> float32 [128]."""
    k = np.asarray(row16).view(np.float16).astype(np.float32) if np.asarray(row16).dtype == np.uint16 \
        else np.asarray(row16, np.float16).astype(np.float32)
    x = rope_undo(k, Crow, Srow) if is_key else k
    return fwht_f32(x)


# --- per-layer path --------------------------------------------------------------------------
def layer_scores(K_l, W: int) -> np.ndarray:
    K_l = _bits(K_l)
    H, T, D = K_l.shape
    s = np.empty(T, np.float64)
    lib().nqo_layer_scores(K_l, H, T, W, s)
    return s


def select_layer(s: np.ndarray, W: int, evict_permille: int):
    """-> (positions int32 [n_keep], eviction near-tie mask uint8 [T], tau)."""
    T = s.shape[0]
    n_keep = keep_count(T, W, evict_permille)
    pos = np.empty(max(n_keep, 1), np.int32)
    near = np.empty(max(T, 1), np.uint8)
    tau = C.c_double()
    n = lib().nqo_select_layer(np.ascontiguousarray(s, np.float64), T, W, evict_permille, pos,
                               near, C.byref(tau))
    assert n == n_keep
    return pos[:n_keep], near[:T], tau.value


def encode_layer(K_l, V_l, positions, Ctab, Stab, bits_k: int, bits_v: int):
    """-> dict(codes_k, codes_v (delta-coded int8 [H,n,128]), scales_k, scales_v (fp16 bits
    [H,n,16]), flags_k, flags_v (uint8 [H,n,16]))."""
    K_l, V_l = _bits(K_l), _bits(V_l)
    H, T, _ = K_l.shape
    pos = np.ascontiguousarray(positions, np.int32)
    n = pos.shape[0]
    out = dict(
        codes_k=np.empty((H, n, 128), np.int8), codes_v=np.empty((H, n, 128), np.int8),
        scales_k=np.empty((H, n, 16), np.uint16), scales_v=np.empty((H, n, 16), np.uint16),
        flags_k=np.empty((H, n, 16), np.uint8), flags_v=np.empty((H, n, 16), np.uint8))
    if n == 0:
        return out
    lib().nqo_encode_layer(K_l, V_l, H, T, pos, n, np.ascontiguousarray(Ctab, np.float32),
                           np.ascontiguousarray(Stab, np.float32), bits_k, bits_v,
                           out["codes_k"], out["codes_v"], out["scales_k"], out["scales_v"],
                           out["flags_k"], out["flags_v"])
    return out


def decode_layer(codes_k, codes_v, scales_k, scales_v, positions, Ctab, Stab):
    """-> (K_hat, V_hat) float64 [H, n, 128]."""
    H, n, _ = codes_k.shape
    Ko = np.empty((H, n, 128), np.float64)
    Vo = np.empty((H, n, 128), np.float64)
    if n == 0:
        return Ko, Vo
    lib().nqo_decode_layer(np.ascontiguousarray(codes_k), np.ascontiguousarray(codes_v),
                           _bits(scales_k), _bits(scales_v),
                           np.ascontiguousarray(positions, np.int32), n, H,
                           np.ascontiguousarray(Ctab, np.float32),
                           np.ascontiguousarray(Stab, np.float32), Ko, Vo)
    return Ko, Vo


def attend_layer(q, K_hat, V_hat) -> np.ndarray:
    """q: fp16 [Hq,128]; K_hat, V_hat: float64 [H,n,128] -> float64 [Hq,128]."""
    q = _bits(q)
    Hq = q.shape[0]
    H, n, _ = K_hat.shape
    out = np.empty((Hq, 128), np.float64)
    lib().nqo_attend_layer(q, Hq, np.ascontiguousarray(K_hat, np.float64),
                           np.ascontiguousarray(V_hat, np.float64), H, n, out)
    return out


def nominal_ratio(H: int, T: int, n_keep: int, bits_k: int, bits_v: int) -> float:
    return lib().nqo_nominal_ratio(H, T, n_keep, bits_k, bits_v)


def compress_layer(K_l, V_l, W: int, evict_permille: int, bits_k: int, bits_v: int,
                   Ctab, Stab):
    """Whole encode chain for one layer: scores -> keep-set -> codes."""
    s = layer_scores(K_l, W)
    pos, near, tau = select_layer(s, W, evict_permille)
    enc = encode_layer(K_l, V_l, pos, Ctab, Stab, bits_k, bits_v)
    enc.update(positions=pos, scores=s, evict_near=near, tau=tau)
    return enc
