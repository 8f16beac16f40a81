"""Host entropy stage: zstd over the delta-coded lattice codes, and the measured compression
ratio it yields.

The pages follow the delta coding with zstd: consecutive tokens give similar lattice indices,
so their deltas compress a further 2-3x ("NexusQuant：无需训练实现LLM KV缓存10-33倍压缩的技术突破",
section "E8格点量化"; "Como comprimir o KV cache do seu LLM em 33x sem treino", "Como funciona"
step 6 and "Os números"). That stage runs on the host, off the GPU path: the device arrays of a
``Compressed`` cache are copied out and compressed with the system libzstd (loaded with ctypes,
no headers needed). Nothing here is on the timed path.

Stored size counted per compressed layer: zstd of the K and V delta streams, zstd of the K and V
fp16 scales, and the keep-set as a bitmap of T bits. The ratio is fp16 K+V bytes of the layer
over that size.
"""
from __future__ import annotations

import ctypes as C
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_z = None


def _lib():
    global _z
    if _z is None:
        try:
            z = C.CDLL("libzstd.so.1")
        except OSError as e:
            raise ImportError("libzstd.so.1 is not available on this host") from e
        z.ZSTD_compressBound.restype = C.c_size_t
        z.ZSTD_compressBound.argtypes = [C.c_size_t]
        z.ZSTD_compress.restype = C.c_size_t
        z.ZSTD_compress.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_size_t, C.c_int]
        z.ZSTD_decompress.restype = C.c_size_t
        z.ZSTD_decompress.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_size_t]
        z.ZSTD_isError.restype = C.c_uint
        z.ZSTD_isError.argtypes = [C.c_size_t]
        z.ZSTD_versionNumber.restype = C.c_uint
        _z = z
    return _z


def zstd_version() -> int:
    return int(_lib().ZSTD_versionNumber())


def compress(data: np.ndarray, level: int = 3) -> bytes:
    """One zstd frame of the array's bytes."""
    z = _lib()
    src = np.ascontiguousarray(data).view(np.uint8).reshape(-1)
    cap = z.ZSTD_compressBound(src.size)
    dst = np.empty(cap, np.uint8)
    n = z.ZSTD_compress(dst.ctypes.data, cap, src.ctypes.data, src.size, level)
    if z.ZSTD_isError(n):
        raise RuntimeError("ZSTD_compress failed")
    return dst[:n].tobytes()


def decompress(frame: bytes, nbytes: int) -> np.ndarray:
    """The nbytes bytes of one zstd frame, as uint8."""
    z = _lib()
    dst = np.empty(max(nbytes, 1), np.uint8)
    n = z.ZSTD_decompress(dst.ctypes.data, nbytes, frame, len(frame))
    if z.ZSTD_isError(n) or n != nbytes:
        raise RuntimeError("ZSTD_decompress failed")
    return dst[:nbytes]


def zstd_size(data: np.ndarray, level: int = 3, chunk: int = 1 << 24, threads: int = 8) -> int:
    """Compressed size of the array's bytes, as independent frames of `chunk` bytes compressed
    in parallel (a frame per chunk is how a streaming store would write them)."""
    src = np.ascontiguousarray(data).view(np.uint8).reshape(-1)
    parts = [src[i:i + chunk] for i in range(0, src.size, chunk)] or [src]
    with ThreadPoolExecutor(threads) as ex:
        return int(sum(ex.map(lambda p: len(compress(p, level)), parts)))


def layer_sizes(codes_k, codes_v, scales_k, scales_v, T: int, level: int = 3) -> dict:
    """Stored bytes of one compressed layer (host arrays: codes int8 [H, n, 128], scales fp16
    [H, n, 16]) and the parts they come from."""
    H, n, _ = codes_k.shape
    out = {
        "fp16_kv": 2 * H * T * 128 * 2,
        "codes_raw": codes_k.nbytes + codes_v.nbytes,
        "codes_zstd": zstd_size(codes_k, level) + zstd_size(codes_v, level),
        "scales_raw": scales_k.nbytes + scales_v.nbytes,
        "scales_zstd": zstd_size(scales_k, level) + zstd_size(scales_v, level),
        "keep_bitmap": (T + 7) // 8,
    }
    out["stored"] = out["codes_zstd"] + out["scales_zstd"] + out["keep_bitmap"]
    out["ratio"] = out["fp16_kv"] / out["stored"]
    return out


def cache_ratio(c, level: int = 3, layers=None) -> dict:
    """Measured post-entropy compression of a ``Compressed`` cache (device arrays are copied to
    the host layer by layer): per-layer sizes summed over the chosen compressed layers."""
    Lc = c.codes_k.shape[0]
    T = c.params.tokens
    tot: dict = {}
    for lc in (range(Lc) if layers is None else layers):
        s = layer_sizes(c.codes_k[lc].cpu().numpy(), c.codes_v[lc].cpu().numpy(),
                        c.scales_k[lc].cpu().numpy(), c.scales_v[lc].cpu().numpy(), T, level)
        for k, v in s.items():
            if k != "ratio":
                tot[k] = tot.get(k, 0) + v
    tot["ratio"] = tot["fp16_kv"] / tot["stored"]
    tot["codes_ratio_zstd"] = tot["codes_raw"] / tot["codes_zstd"]
    return tot
