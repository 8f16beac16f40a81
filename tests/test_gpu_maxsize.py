"""GPU parity at the largest supported token count: 2^23 - 1 tokens in one layer and one head.

The encode addresses a chain's rows, the rotary table and the chain's codes with 32-bit byte
offsets (position * 256 plus the lane's part), which reach their maximum here, and the selection
runs on 8.4M candidates (the kernel that re-reads the scores). Checked against the oracle on the
same host bytes: every score; the keep-set as the exact top m of the GPU's own scores and as the
oracle's keep-set up to eviction near-ties; codes, scales and fp16 reconstructions of sampled
kept tokens -- the first and last ones of the chain (the largest offsets), tokens at tile
boundaries and random ones -- under the same rules as the other parity tests.

Inputs: seeded standard-normal K and V drawn on the device and rounded to fp16 (the host
generator would take minutes for 2 x 2^30 values); the oracle reads the same bytes.
"""
import numpy as np
import pytest
import torch

import kv_cache_compression_proxy_amd as nq
import kvsynth
import oracle
from gpu_helpers import (GpuRun, absolute_codes, compare_codes, compare_keep, fp16_recon_ratio,
                         gpu_keep_set, params_of, rotated_rows, say)

pytestmark = pytest.mark.gpu

T_MAX = (1 << 23) - 1


def sampled_indices(n: int, seed: int = 5) -> np.ndarray:
    rng = np.random.default_rng(seed)
    edges = np.arange(0, n, 256)
    picks = [np.arange(min(n, 64)), np.arange(max(0, n - 64), n),
             rng.choice(edges, min(len(edges), 48), replace=False),
             np.clip(rng.choice(edges, min(len(edges), 48), replace=False) - 1, 0, n - 1),
             rng.integers(0, n, 256)]
    return np.unique(np.concatenate(picks))


def gpu_abs_codes(codes: torch.Tensor, idx: np.ndarray) -> np.ndarray:
    """Absolute codes of chain rows idx from a device delta-coded chain [n, 128]."""
    c = torch.cumsum(codes.to(torch.int32), dim=0)
    c = ((c + 128) % 256 - 128).to(torch.int8)
    return c[torch.from_numpy(idx).to(codes.device)].cpu().numpy()


def test_max_token_count():
    w = kvsynth.workload(0).with_(layers=1, kv_heads=1, tokens=T_MAX, window=256,
                                  evict_permille=600)
    p = params_of(w)
    assert nq.nq_check_params(p) == nq.NQ_OK
    T, W = T_MAX, w.window
    say(f"[maxsize] drawing 1x1x{T} fp16 K/V on the device")
    gen = torch.Generator(device="cuda").manual_seed(2 ** 23 - 1)
    K = torch.randn((1, 1, T, 128), generator=gen, device="cuda").half()
    V = torch.randn((1, 1, T, 128), generator=gen, device="cuda").half()
    K_l, V_l = K[0].cpu().numpy(), V[0].cpu().numpy()
    say("[maxsize] score/evict/encode/decode on the GPU")
    run = GpuRun(p, K, V, out_f32=False)
    assert run.lookback_error() == 0
    n = run.n_keep
    del K, V

    say("[maxsize] scores and keep-set")
    sg = run.scores[0].cpu().numpy()
    so = oracle.layer_scores(K_l, W)
    cand = slice(1, T - W)   # the scored candidates (the window and BOS are always kept)
    err = np.abs(sg[cand] - so[cand]).max() / max(1.0, float(np.abs(so[cand]).max()))
    say(f"[maxsize] score error / max score {err:.3g}")
    assert err < 1e-12
    pos_g = run.positions[0].cpu().numpy()[:n]
    assert np.all(np.diff(pos_g) > 0)
    assert np.array_equal(pos_g, gpu_keep_set(sg, T, W, n)), \
        "keep-set is not the top-m of the GPU's own scores"
    pos_o, near, _ = oracle.select_layer(so, W, w.evict_permille)
    nd, only_near = compare_keep(pos_g, pos_o, near)
    say(f"[maxsize] keep-set: {nd} positions differ from the oracle's (near-ties only: {only_near})")
    assert only_near
    assert pos_g[-1] == T - 1   # the last window token: the largest row offset

    idx = sampled_indices(n)
    say(f"[maxsize] oracle encode/decode of {idx.size} sampled kept tokens (last position {pos_g[idx[-1]]})")
    Ct, St = oracle.rope_table(T, w.rope_base)
    enc = oracle.encode_layer(K_l, V_l, pos_g[idx], Ct, St, w.bits_k, w.bits_v)
    Kh, Vh = oracle.decode_layer(enc["codes_k"], enc["codes_v"], enc["scales_k"],
                                 enc["scales_v"], pos_g[idx], Ct, St)
    for tensor, X, bits, codes, scales, hat, ohat in (
            ("K", K_l, w.bits_k, run.codes_k, run.scales_k, run.K_hat, Kh),
            ("V", V_l, w.bits_v, run.codes_v, run.scales_v, run.V_hat, Vh)):
        key = tensor.lower()
        gc = gpu_abs_codes(codes[0, 0, :n], idx)[None]
        gs = scales[0, 0, :n][torch.from_numpy(idx).to(scales.device)].cpu().numpy()[None]
        oc = absolute_codes(enc[f"codes_{key}"])
        x_of = rotated_rows(X, tensor == "K", pos_g[idx], Ct, St)
        mism, bad, vor = compare_codes(gc, gs, oc, enc[f"scales_{key}"], enc[f"flags_{key}"],
                                       x_of, bits)
        say(f"[maxsize] {tensor}: {mism} groups differ ({vor} Voronoi near-ties flagged)")
        assert bad == 0
        g16 = hat[0, 0, :n][torch.from_numpy(idx).to(hat.device)].cpu().numpy()[None]
        r = fp16_recon_ratio(g16, ohat, enc[f"scales_{key}"], enc[f"flags_{key}"])
        say(f"[maxsize] {tensor}: fp16 reconstruction error / group scale {r:.3g}")
        assert r <= 1e-3
