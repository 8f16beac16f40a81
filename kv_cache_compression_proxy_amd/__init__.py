"""Python binding of libnq, the MI355X (gfx950) KV-cache compression hot path.

Argument marshalling only: every step runs in the HIP kernels of ``libnq.so`` (built in-tree by
``python kv_cache_compression_proxy_amd/build.py``). PyTorch supplies device memory and streams.
Importing this package without the built library raises ImportError -- there is no fallback.

Low-level functions carry the C names of ``include/nq.h`` (``nq_score_evict``, ``nq_encode``,
``nq_decode``, ...) and take torch tensors. ``compress`` / ``decompress`` chain them with the
pages' quality presets.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

from .presets import PRESETS, params_for

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      f"`python kv_cache_compression_proxy_amd/build.py` (no CPU fallback exists)")

# torch ships its own HIP runtime; importing it first makes libnq's libamdhip64.so.7 dependency
# resolve (by soname) to that same, already loaded runtime, so both share one device context.
import torch  # noqa: E402,F401

_lib = C.CDLL(LIB_PATH)

NQ_OK, NQ_ERR_INVALID_ARG, NQ_ERR_UNSUPPORTED, NQ_ERR_WORKSPACE, NQ_ERR_HIP = 0, -1, -2, -3, -4
NQ_OUT_F16, NQ_OUT_F32 = 0, 1
EXPORTED = ("nq_keep_count", "nq_check_params", "nq_score_evict_workspace_bytes",
            "nq_decode_workspace_bytes", "nq_attend_workspace_bytes", "nq_rope_table",
            "nq_score_evict", "nq_encode", "nq_decode", "nq_attend_decode",
            "nq_decode_attend_workspace_bytes", "nq_decode_attend",
            "nq_score_evict_attn_workspace_bytes", "nq_score_evict_attn", "nq_lloyd_max_table",
            "nq_encode_scalar", "nq_decode_scalar", "nq_decode_static", "nq_status_string")


class NqParams(C.Structure):
    _fields_ = [("layers", C.c_int32), ("kv_heads", C.c_int32), ("tokens", C.c_int32),
                ("head_dim", C.c_int32), ("layer_begin", C.c_int32), ("layer_end", C.c_int32),
                ("window", C.c_int32), ("evict_permille", C.c_int32), ("bits_k", C.c_int32),
                ("bits_v", C.c_int32), ("rope_base", C.c_double)]

    def __repr__(self):
        return "NqParams(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


_P = C.POINTER(NqParams)
_v = C.c_void_p
_sig = {
    "nq_keep_count": (C.c_int32, [_P]),
    "nq_check_params": (C.c_int, [_P]),
    "nq_score_evict_workspace_bytes": (C.c_size_t, [_P]),
    "nq_decode_workspace_bytes": (C.c_size_t, [_P]),
    "nq_attend_workspace_bytes": (C.c_size_t, [_P, C.c_int32, C.c_int32]),
    "nq_rope_table": (C.c_int, [_P, _v, _v, _v]),
    "nq_score_evict": (C.c_int, [_P, _v, _v, _v, _v, C.c_size_t, _v]),
    "nq_encode": (C.c_int, [_P, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v]),
    "nq_decode": (C.c_int, [_P, _v, _v, _v, _v, _v, _v, _v, _v, _v, C.c_int, _v, C.c_size_t, _v]),
    "nq_attend_decode": (C.c_int, [_P, _v, C.c_int32, _v, _v, C.c_int32, _v, _v, C.c_size_t,
                                   _v]),
    "nq_decode_attend_workspace_bytes": (C.c_size_t, [_P, C.c_int32]),
    "nq_decode_attend": (C.c_int, [_P, _v, _v, _v, _v, _v, _v, _v, _v, C.c_int32, _v, _v,
                                   C.c_size_t, _v]),
    "nq_score_evict_attn_workspace_bytes": (C.c_size_t, [_P, C.c_int32]),
    "nq_score_evict_attn": (C.c_int, [_P, _v, _v, C.c_int32, _v, _v, _v, C.c_size_t, _v]),
    "nq_lloyd_max_table": (C.c_int, [C.c_int32, _v, _v]),
    "nq_encode_scalar": (C.c_int, [_P, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v]),
    "nq_decode_scalar": (C.c_int, [_P, _v, _v, _v, _v, _v, _v, _v, _v, _v, C.c_int, _v]),
    "nq_decode_static": (C.c_int, [_P, _v, _v, _v, _v, _v, _v, _v, _v, _v, C.c_int, _v]),
    "nq_status_string": (C.c_char_p, [C.c_int]),
}
# bytes of the static scratch array behind nq_decode_static (NQ_DECODE_STATIC_MAX_BYTES)
NQ_DECODE_STATIC_MAX_BYTES = 64 << 20
for _name, (_res, _args) in _sig.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class NqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {_lib.nq_status_string(status).decode()} ({status})")
        self.status = status


def _ok(fn: str, status: int):
    if status != NQ_OK:
        raise NqError(fn, status)


def _ptr(t):
    """Device (or host) address of a tensor, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _torch_stream(stream):
    """The torch stream object for a stream argument (None: the current stream; an int: a raw
    HIP stream handle)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


def _need(t, name: str, dtype, numel: int, device=None):
    """Host check of a tensor argument before its address goes to the library: dtype,
    contiguity, device and at least the element count the call will access. Raw integer
    addresses (and None, which the library rejects itself) pass unchecked."""
    import torch
    if t is None or isinstance(t, int):
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor or an address, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, the call accesses {numel}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _dev(t):
    import torch
    return t.device if isinstance(t, torch.Tensor) else None


def _sizes(p: NqParams):
    """(compressed layers, kv heads, tokens, kept tokens) of p (kept = 0 if p is invalid)."""
    Lc = max(p.layer_end - p.layer_begin, 0)
    return Lc, p.kv_heads, max(p.tokens, 0), max(_lib.nq_keep_count(C.byref(p)), 0)


def make_params(layers, kv_heads, tokens, window, evict_permille, bits_k, bits_v, rope_base,
                layer_begin=0, layer_end=None, head_dim=128) -> NqParams:
    return NqParams(layers, kv_heads, tokens, head_dim, layer_begin,
                    layers if layer_end is None else layer_end, window, evict_permille, bits_k,
                    bits_v, float(rope_base))


# ---------------------------------------------------------------- C entry points (same names)
def nq_keep_count(p: NqParams) -> int:
    return _lib.nq_keep_count(C.byref(p))


def nq_check_params(p: NqParams) -> int:
    return _lib.nq_check_params(C.byref(p))


def nq_score_evict_workspace_bytes(p: NqParams) -> int:
    return _lib.nq_score_evict_workspace_bytes(C.byref(p))


def nq_decode_workspace_bytes(p: NqParams) -> int:
    return _lib.nq_decode_workspace_bytes(C.byref(p))


def nq_attend_workspace_bytes(p: NqParams, q_heads: int, n_tok: int) -> int:
    return _lib.nq_attend_workspace_bytes(C.byref(p), q_heads, n_tok)


def nq_rope_table(p, cos, sin, stream=None):
    import torch
    T = max(p.tokens, 0)
    _need(cos, "cos", torch.float32, T * 64)
    _need(sin, "sin", torch.float32, T * 64, _dev(cos))
    _ok("nq_rope_table", _lib.nq_rope_table(C.byref(p), _ptr(cos), _ptr(sin), _stream(stream)))


def nq_score_evict(p, K, positions, workspace, scores=None, stream=None):
    import torch
    Lc, H, T, n = _sizes(p)
    d = _dev(K)
    _need(K, "K", torch.float16, p.layers * H * T * 128)
    _need(positions, "positions", torch.int32, Lc * n, d)
    _need(scores, "scores", torch.float64, Lc * T, d)
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _ok("nq_score_evict", _lib.nq_score_evict(C.byref(p), _ptr(K), _ptr(positions), _ptr(scores),
                                              _ptr(workspace), ws, _stream(stream)))


def nq_encode(p, K, V, positions, rope_cos, rope_sin, codes_k, codes_v, scales_k, scales_v,
              stream=None):
    import torch
    Lc, H, T, n = _sizes(p)
    d = _dev(K)
    for name, t, dt, k in (("K", K, torch.float16, p.layers * H * T * 128),
                           ("V", V, torch.float16, p.layers * H * T * 128),
                           ("positions", positions, torch.int32, Lc * n),
                           ("rope_cos", rope_cos, torch.float32, T * 64),
                           ("rope_sin", rope_sin, torch.float32, T * 64),
                           ("codes_k", codes_k, torch.int8, Lc * H * n * 128),
                           ("codes_v", codes_v, torch.int8, Lc * H * n * 128),
                           ("scales_k", scales_k, torch.float16, Lc * H * n * 16),
                           ("scales_v", scales_v, torch.float16, Lc * H * n * 16)):
        _need(t, name, dt, k, d)
    _ok("nq_encode", _lib.nq_encode(C.byref(p), _ptr(K), _ptr(V), _ptr(positions), _ptr(rope_cos),
                                    _ptr(rope_sin), _ptr(codes_k), _ptr(codes_v), _ptr(scales_k),
                                    _ptr(scales_v), _stream(stream)))


def nq_decode(p, codes_k, codes_v, scales_k, scales_v, positions, rope_cos, rope_sin, K_out,
              V_out, out_dtype, workspace, stream=None):
    import torch
    Lc, H, T, n = _sizes(p)
    d = _dev(codes_k)
    odt = torch.float32 if out_dtype == NQ_OUT_F32 else torch.float16
    for name, t, dt, k in (("codes_k", codes_k, torch.int8, Lc * H * n * 128),
                           ("codes_v", codes_v, torch.int8, Lc * H * n * 128),
                           ("scales_k", scales_k, torch.float16, Lc * H * n * 16),
                           ("scales_v", scales_v, torch.float16, Lc * H * n * 16),
                           ("positions", positions, torch.int32, Lc * n),
                           ("rope_cos", rope_cos, torch.float32, T * 64),
                           ("rope_sin", rope_sin, torch.float32, T * 64),
                           ("K_out", K_out, odt, Lc * H * n * 128),
                           ("V_out", V_out, odt, Lc * H * n * 128)):
        _need(t, name, dt, k, d)
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _ok("nq_decode", _lib.nq_decode(C.byref(p), _ptr(codes_k), _ptr(codes_v), _ptr(scales_k),
                                    _ptr(scales_v), _ptr(positions), _ptr(rope_cos),
                                    _ptr(rope_sin), _ptr(K_out), _ptr(V_out), out_dtype,
                                    _ptr(workspace), ws, _stream(stream)))


def nq_decode_static(p, codes_k, codes_v, scales_k, scales_v, positions, rope_cos, rope_sin,
                     K_out, V_out, out_dtype, stream=None):
    """nq_decode without a workspace: the library's static device scratch (for callers that
    cannot allocate; calls on one GPU must not overlap)."""
    import torch
    Lc, H, T, n = _sizes(p)
    d = _dev(codes_k)
    odt = torch.float32 if out_dtype == NQ_OUT_F32 else torch.float16
    for name, t, dt, k in (("codes_k", codes_k, torch.int8, Lc * H * n * 128),
                           ("codes_v", codes_v, torch.int8, Lc * H * n * 128),
                           ("scales_k", scales_k, torch.float16, Lc * H * n * 16),
                           ("scales_v", scales_v, torch.float16, Lc * H * n * 16),
                           ("positions", positions, torch.int32, Lc * n),
                           ("rope_cos", rope_cos, torch.float32, T * 64),
                           ("rope_sin", rope_sin, torch.float32, T * 64),
                           ("K_out", K_out, odt, Lc * H * n * 128),
                           ("V_out", V_out, odt, Lc * H * n * 128)):
        _need(t, name, dt, k, d)
    _ok("nq_decode_static", _lib.nq_decode_static(
        C.byref(p), _ptr(codes_k), _ptr(codes_v), _ptr(scales_k), _ptr(scales_v),
        _ptr(positions), _ptr(rope_cos), _ptr(rope_sin), _ptr(K_out), _ptr(V_out), out_dtype,
        _stream(stream)))


def nq_attend_decode(p, Q, q_heads, K, V, n_tok, out, workspace, stream=None):
    import torch
    Lc, H, _, _ = _sizes(p)
    d = _dev(Q)
    _need(Q, "Q", torch.float16, Lc * q_heads * 128)
    _need(K, "K", torch.float16, Lc * H * max(n_tok, 0) * 128, d)
    _need(V, "V", torch.float16, Lc * H * max(n_tok, 0) * 128, d)
    _need(out, "out", torch.float32, Lc * q_heads * 128, d)
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _ok("nq_attend_decode", _lib.nq_attend_decode(C.byref(p), _ptr(Q), q_heads, _ptr(K), _ptr(V),
                                                  n_tok, _ptr(out), _ptr(workspace), ws,
                                                  _stream(stream)))


def nq_score_evict_attn_workspace_bytes(p: NqParams, q_heads: int) -> int:
    return _lib.nq_score_evict_attn_workspace_bytes(C.byref(p), q_heads)


def nq_score_evict_attn(p, K, Q_obs, q_heads, positions, workspace, scores=None, stream=None):
    import torch
    Lc, H, T, n = _sizes(p)
    d = _dev(K)
    _need(K, "K", torch.float16, p.layers * H * T * 128)
    _need(Q_obs, "Q_obs", torch.float16, Lc * q_heads * max(p.window, 0) * 128, d)
    _need(positions, "positions", torch.int32, Lc * n, d)
    _need(scores, "scores", torch.float64, Lc * T, d)
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _ok("nq_score_evict_attn", _lib.nq_score_evict_attn(
        C.byref(p), _ptr(K), _ptr(Q_obs), q_heads, _ptr(positions), _ptr(scores),
        _ptr(workspace), ws, _stream(stream)))


def nq_decode_attend_workspace_bytes(p: NqParams, q_heads: int) -> int:
    return _lib.nq_decode_attend_workspace_bytes(C.byref(p), q_heads)


def nq_decode_attend(p, codes_k, codes_v, scales_k, scales_v, positions, rope_cos, rope_sin, Q,
                     q_heads, out, workspace, stream=None):
    import torch
    Lc, H, T, n = _sizes(p)
    d = _dev(Q)
    for name, t, dt, k in (("codes_k", codes_k, torch.int8, Lc * H * n * 128),
                           ("codes_v", codes_v, torch.int8, Lc * H * n * 128),
                           ("scales_k", scales_k, torch.float16, Lc * H * n * 16),
                           ("scales_v", scales_v, torch.float16, Lc * H * n * 16),
                           ("positions", positions, torch.int32, Lc * n),
                           ("rope_cos", rope_cos, torch.float32, T * 64),
                           ("rope_sin", rope_sin, torch.float32, T * 64),
                           ("Q", Q, torch.float16, Lc * q_heads * 128),
                           ("out", out, torch.float32, Lc * q_heads * 128)):
        _need(t, name, dt, k, d)
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _ok("nq_decode_attend", _lib.nq_decode_attend(
        C.byref(p), _ptr(codes_k), _ptr(codes_v), _ptr(scales_k), _ptr(scales_v), _ptr(positions),
        _ptr(rope_cos), _ptr(rope_sin), _ptr(Q), q_heads, _ptr(out), _ptr(workspace), ws,
        _stream(stream)))


def nq_lloyd_max_table(bits: int):
    """-> (levels, thresholds) float64 numpy arrays of the library's Lloyd-Max table."""
    import numpy as np
    y = np.zeros(1 << bits, np.float64)
    t = np.zeros(max((1 << bits) - 1, 1), np.float64)
    _ok("nq_lloyd_max_table", _lib.nq_lloyd_max_table(bits, y.ctypes.data, t.ctypes.data))
    return y, t[:(1 << bits) - 1]


def nq_encode_scalar(p, K, V, positions, rope_cos, rope_sin, idx_k, idx_v, scales_k, scales_v,
                     stream=None):
    import torch
    Lc, H, T, n = _sizes(p)
    d = _dev(K)
    for name, t, dt, k in (("K", K, torch.float16, p.layers * H * T * 128),
                           ("V", V, torch.float16, p.layers * H * T * 128),
                           ("positions", positions, torch.int32, Lc * n),
                           ("rope_cos", rope_cos, torch.float32, T * 64),
                           ("rope_sin", rope_sin, torch.float32, T * 64),
                           ("idx_k", idx_k, torch.uint8, Lc * H * n * 128),
                           ("idx_v", idx_v, torch.uint8, Lc * H * n * 128),
                           ("scales_k", scales_k, torch.float16, Lc * H * n * 16),
                           ("scales_v", scales_v, torch.float16, Lc * H * n * 16)):
        _need(t, name, dt, k, d)
    _ok("nq_encode_scalar", _lib.nq_encode_scalar(
        C.byref(p), _ptr(K), _ptr(V), _ptr(positions), _ptr(rope_cos), _ptr(rope_sin),
        _ptr(idx_k), _ptr(idx_v), _ptr(scales_k), _ptr(scales_v), _stream(stream)))


def nq_decode_scalar(p, idx_k, idx_v, scales_k, scales_v, positions, rope_cos, rope_sin, K_out,
                     V_out, out_dtype, stream=None):
    import torch
    Lc, H, T, n = _sizes(p)
    d = _dev(idx_k)
    odt = torch.float32 if out_dtype == NQ_OUT_F32 else torch.float16
    for name, t, dt, k in (("idx_k", idx_k, torch.uint8, Lc * H * n * 128),
                           ("idx_v", idx_v, torch.uint8, Lc * H * n * 128),
                           ("scales_k", scales_k, torch.float16, Lc * H * n * 16),
                           ("scales_v", scales_v, torch.float16, Lc * H * n * 16),
                           ("positions", positions, torch.int32, Lc * n),
                           ("rope_cos", rope_cos, torch.float32, T * 64),
                           ("rope_sin", rope_sin, torch.float32, T * 64),
                           ("K_out", K_out, odt, Lc * H * n * 128),
                           ("V_out", V_out, odt, Lc * H * n * 128)):
        _need(t, name, dt, k, d)
    _ok("nq_decode_scalar", _lib.nq_decode_scalar(
        C.byref(p), _ptr(idx_k), _ptr(idx_v), _ptr(scales_k), _ptr(scales_v), _ptr(positions),
        _ptr(rope_cos), _ptr(rope_sin), _ptr(K_out), _ptr(V_out), out_dtype, _stream(stream)))


def nq_status_string(status: int) -> str:
    return _lib.nq_status_string(status).decode()


# ---------------------------------------------------------------- convenience chain
@dataclass
class Compressed:
    params: NqParams
    positions: "object"   # int32 [Lc, n_keep]
    codes_k: "object"     # int8 [Lc, H, n_keep, 128] (delta-coded)
    codes_v: "object"
    scales_k: "object"    # fp16 [Lc, H, n_keep, 16]
    scales_v: "object"
    rope_cos: "object"    # fp32 [T, 64]
    rope_sin: "object"

    @property
    def n_keep(self) -> int:
        return self.positions.shape[1]


def workspace(nbytes: int, device="cuda"):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def lookback_timed_out(ws) -> bool:
    """True if the nq_decode / nq_decode_attend call that last used the workspace `ws` gave up
    a wait for a predecessor tile's prefix (its uint32 word 1, see nq.h; never expected, the
    outputs are then invalid). Reads the word back, so it waits for that call to finish."""
    import torch
    return int(ws[4:8].view(torch.int32).item()) != 0


def _check_lookback(fn: str, ws):
    if lookback_timed_out(ws):
        raise RuntimeError(f"{fn}: a look-back wait exceeded the spin limit; outputs are invalid")


def rope_table(p: NqParams, device="cuda", stream=None):
    import torch
    with torch.cuda.stream(_torch_stream(stream)):
        cos = torch.empty((max(p.tokens, 1), 64), dtype=torch.float32, device=device)
        sin = torch.empty_like(cos)
    nq_rope_table(p, cos, sin, stream)
    return cos, sin


def _check_kv(K, V):
    import torch
    for name, t in (("K", K), ("V", V)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{name}: expected a [layers, kv_heads, tokens, 128] tensor")
        if t.dtype != torch.float16 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name}: must be a contiguous fp16 tensor on a GPU")
    if K.shape != V.shape or K.device != V.device:
        raise ValueError(f"K {tuple(K.shape)} and V {tuple(V.shape)} must match")
    if K.shape[3] != 128:
        raise ValueError(f"head_dim {K.shape[3]}: only 128 is supported")


def _check_q(Q, Lc: int, H: int, name="Q", window=None):
    """Q: fp16 [Lc, Hq, 128] (window None) or [Lc, Hq, window, 128]; returns Hq."""
    import torch
    shape = (Lc, None, 128) if window is None else (Lc, None, window, 128)
    if (not isinstance(Q, torch.Tensor) or Q.dim() != len(shape) or Q.dtype != torch.float16
            or not Q.is_contiguous() or not Q.is_cuda
            or any(want is not None and got != want for got, want in zip(Q.shape, shape))):
        raise ValueError(f"{name}: expected a contiguous fp16 GPU tensor of shape "
                         f"{tuple('Hq' if d is None else d for d in shape)}")
    if Q.shape[1] < 1 or Q.shape[1] % H:
        raise ValueError(f"{name}: {Q.shape[1]} query heads is not a multiple of {H} kv heads")
    return Q.shape[1]


# Stream use of the convenience chains: every tensor they allocate, workspaces included, is
# allocated with the call's stream current, so torch's caching allocator hands a workspace
# back to that stream only after the kernels queued on it; the outputs belong to that stream
# too (use them on another stream after the usual synchronisation or record_stream).


def compress(K, V, preset: str = "balanced", rope=None, stream=None, window_queries=None,
             **overrides) -> Compressed:
    """K, V: contiguous fp16 GPU tensors [L, H, T, 128]. Runs scoring + eviction + encode on the
    GPU. window_queries: None for the key-key proxy scorer, or fp16 [Lc, Hq, window, 128]
    queries of the observation window for the attention-weight scorer."""
    import torch
    _check_kv(K, V)
    L, H, T, D = K.shape
    p = params_for(preset, L, H, T, **overrides)
    _ok("nq_check_params", nq_check_params(p))
    n_keep = nq_keep_count(p)
    Lc = p.layer_end - p.layer_begin
    dev = K.device
    hq = None if window_queries is None else _check_q(window_queries, Lc, H, "window_queries",
                                                      p.window)
    s = _torch_stream(stream)
    with torch.cuda.stream(s):
        cos, sin = rope if rope is not None else rope_table(p, dev, s)
        positions = torch.empty((Lc, n_keep), dtype=torch.int32, device=dev)
        if hq is None:
            ws = workspace(nq_score_evict_workspace_bytes(p), dev)
            nq_score_evict(p, K, positions, ws, stream=s)
        else:
            ws = workspace(nq_score_evict_attn_workspace_bytes(p, hq), dev)
            nq_score_evict_attn(p, K, window_queries, hq, positions, ws, stream=s)
        ck = torch.empty((Lc, H, n_keep, 128), dtype=torch.int8, device=dev)
        cv = torch.empty_like(ck)
        sk = torch.empty((Lc, H, n_keep, 16), dtype=torch.float16, device=dev)
        sv = torch.empty_like(sk)
        nq_encode(p, K, V, positions, cos, sin, ck, cv, sk, sv, s)
    return Compressed(p, positions, ck, cv, sk, sv, cos, sin)


def decompress(c: Compressed, out_dtype=None, stream=None, check: bool = False):
    """-> (K_hat, V_hat) [Lc, H, n_keep, 128] in fp16 (default) or fp32. check: wait for the
    call and raise if a look-back wait timed out."""
    import torch
    out_dtype = out_dtype or torch.float16
    if out_dtype not in (torch.float16, torch.float32):
        raise ValueError(f"out_dtype {out_dtype}: fp16 or fp32")
    Lc, H, n, _ = c.codes_k.shape
    s = _torch_stream(stream)
    with torch.cuda.stream(s):
        Ko = torch.empty((Lc, H, n, 128), dtype=out_dtype, device=c.codes_k.device)
        Vo = torch.empty_like(Ko)
        ws = workspace(nq_decode_workspace_bytes(c.params), c.codes_k.device)
        nq_decode(c.params, c.codes_k, c.codes_v, c.scales_k, c.scales_v, c.positions,
                  c.rope_cos, c.rope_sin, Ko, Vo,
                  NQ_OUT_F32 if out_dtype == torch.float32 else NQ_OUT_F16, ws, s)
        if check:
            _check_lookback("nq_decode", ws)
    return Ko, Vo


def attend(c_params: NqParams, Q, K_hat, V_hat, stream=None):
    """One-token GQA over a reconstructed cache: Q fp16 [Lc, Hq, 128], K_hat/V_hat fp16
    [Lc, H, n, 128] -> fp32 [Lc, Hq, 128]."""
    import torch
    Lc = c_params.layer_end - c_params.layer_begin
    Hq = _check_q(Q, Lc, c_params.kv_heads)
    if (K_hat.dtype != torch.float16 or V_hat.shape != K_hat.shape or K_hat.dim() != 4
            or tuple(K_hat.shape[:2]) != (Lc, c_params.kv_heads) or K_hat.shape[3] != 128):
        raise ValueError("K_hat, V_hat: fp16 [Lc, kv_heads, n, 128] of equal shape")
    n = K_hat.shape[2]
    s = _torch_stream(stream)
    with torch.cuda.stream(s):
        out = torch.empty((Lc, Hq, 128), dtype=torch.float32, device=Q.device)
        ws = workspace(nq_attend_workspace_bytes(c_params, Hq, n), Q.device)
        nq_attend_decode(c_params, Q, Hq, K_hat, V_hat, n, out, ws, s)
    return out


def attend_compressed(c: Compressed, Q, stream=None, check: bool = False):
    """One-token GQA straight from the compressed cache (no K_hat/V_hat written):
    Q fp16 [Lc, Hq, 128] -> fp32 [Lc, Hq, 128]. check: as for decompress."""
    import torch
    Lc = c.params.layer_end - c.params.layer_begin
    Hq = _check_q(Q, Lc, c.params.kv_heads)
    s = _torch_stream(stream)
    with torch.cuda.stream(s):
        out = torch.empty((Lc, Hq, 128), dtype=torch.float32, device=Q.device)
        ws = workspace(nq_decode_attend_workspace_bytes(c.params, Hq), Q.device)
        nq_decode_attend(c.params, c.codes_k, c.codes_v, c.scales_k, c.scales_v, c.positions,
                         c.rope_cos, c.rope_sin, Q, Hq, out, ws, s)
        if check:
            _check_lookback("nq_decode_attend", ws)
    return out


__all__ = ["NqParams", "NqError", "Compressed", "PRESETS", "params_for", "make_params",
           "compress", "decompress", "attend", "attend_compressed", "rope_table", "workspace",
           "lookback_timed_out",
           *EXPORTED]
