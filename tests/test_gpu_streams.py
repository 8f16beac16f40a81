"""Calls on two streams at once, with separate buffers and workspaces, give the same bytes as
the same calls one after another. Every entry point keeps its state (decode tile tickets,
look-back words, partial sums) in the caller's workspace, so concurrent calls that share no
buffer cannot interact; this checks it for the whole chain (score + evict, encode, decode,
fused decode-attention) with kernels of both calls resident on the GPU together."""
import pytest
import torch

import kv_cache_compression_proxy_amd as nq
import kvsynth
from gpu_helpers import params_of, say, upload

pytestmark = pytest.mark.gpu


def chain(p, K, V, Q, cos, sin, stream):
    """Score + evict, encode, fp16 decode and fused decode-attention on `stream`; returns the
    output tensors (allocated here, before the calls are queued)."""
    Lc, H, n = p.layer_end - p.layer_begin, p.kv_heads, nq.nq_keep_count(p)
    dev = K.device
    o = {
        "positions": torch.empty((Lc, n), dtype=torch.int32, device=dev),
        "codes_k": torch.empty((Lc, H, n, 128), dtype=torch.int8, device=dev),
        "codes_v": torch.empty((Lc, H, n, 128), dtype=torch.int8, device=dev),
        "scales_k": torch.empty((Lc, H, n, 16), dtype=torch.float16, device=dev),
        "scales_v": torch.empty((Lc, H, n, 16), dtype=torch.float16, device=dev),
        "K_hat": torch.empty((Lc, H, n, 128), dtype=torch.float16, device=dev),
        "V_hat": torch.empty((Lc, H, n, 128), dtype=torch.float16, device=dev),
        "att": torch.empty((Lc, Q.shape[1], 128), dtype=torch.float32, device=dev),
    }
    ws_s = nq.workspace(nq.nq_score_evict_workspace_bytes(p), dev)
    ws_d = nq.workspace(nq.nq_decode_workspace_bytes(p), dev)
    ws_a = nq.workspace(nq.nq_decode_attend_workspace_bytes(p, Q.shape[1]), dev)
    nq.nq_score_evict(p, K, o["positions"], ws_s, stream=stream)
    nq.nq_encode(p, K, V, o["positions"], cos, sin, o["codes_k"], o["codes_v"], o["scales_k"],
                 o["scales_v"], stream)
    nq.nq_decode(p, o["codes_k"], o["codes_v"], o["scales_k"], o["scales_v"], o["positions"],
                 cos, sin, o["K_hat"], o["V_hat"], nq.NQ_OUT_F16, ws_d, stream)
    nq.nq_decode_attend(p, o["codes_k"], o["codes_v"], o["scales_k"], o["scales_v"],
                        o["positions"], cos, sin, Q, Q.shape[1], o["att"], ws_a, stream)
    o["_ws"] = (ws_s, ws_d, ws_a)
    return o


def test_two_streams_bitwise():
    w = kvsynth.workload(1).with_(layers=4, tokens=8192)
    p = params_of(w)
    K, V = upload(w)
    Q = torch.randn((w.compressed_layers, 4 * w.kv_heads, 128), device="cuda",
                    generator=torch.Generator(device="cuda").manual_seed(3)).half()
    cos, sin = nq.rope_table(p, "cuda")
    torch.cuda.synchronize()
    say("[streams] reference chain on the current stream")
    ref = chain(p, K, V, Q, cos, sin, torch.cuda.current_stream())
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()      # default priority
    for rep in range(3):
        say(f"[streams] two chains at once, repetition {rep}")
        a = chain(p, K, V, Q, cos, sin, s1)
        b = chain(p, K, V, Q, cos, sin, s2)
        torch.cuda.synchronize()
        for name, r in ref.items():
            if name.startswith("_"):
                continue
            assert torch.equal(a[name], r), f"stream 1, {name}"
            assert torch.equal(b[name], r), f"stream 2, {name}"
        for ws in (a["_ws"][1], a["_ws"][2], b["_ws"][1], b["_ws"][2]):
            assert not nq.lookback_timed_out(ws)
