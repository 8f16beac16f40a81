"""Quality of the E8 lattice step against the equal-bit scalar baseline (both oracles, CPU):
the same keep-set, the same front end and the same fp16 scale per 8 dims, then E8 at b bits per
dim (absmax scaling to radius 2^(b-1) - 1) or a Lloyd-Max quantizer of N(0, 1) at b bits per dim
(RMS scaling). Reported: SNR and mean cosine of the reconstructed rows against the original
kept rows. Sanity bars only: which one is better is a measurement, not a pin."""
import numpy as np

import kvsynth
import oracle
from oracle import lloyd_max as lm


def metrics(X, Xh):
    err = np.sum((X - Xh) ** 2)
    snr = 10 * np.log10(np.sum(X ** 2) / err)
    cos = np.sum(X * Xh, -1) / (np.linalg.norm(X, axis=-1) * np.linalg.norm(Xh, axis=-1) + 1e-30)
    return float(snr), float(cos.mean())


def test_e8_vs_scalar_equal_bits():
    w = kvsynth.workload(0)
    T = w.tokens
    K_l, V_l = kvsynth.layer_kv(w, 0)
    Ct, St = oracle.rope_table(T, w.rope_base)
    e8 = oracle.compress_layer(K_l, V_l, w.window, w.evict_permille, w.bits_k, w.bits_v, Ct, St)
    pos = e8["positions"]
    Kh, Vh = oracle.decode_layer(e8["codes_k"], e8["codes_v"], e8["scales_k"], e8["scales_v"],
                                 pos, Ct, St)
    sc = lm.encode_layer(K_l, V_l, pos, Ct, St, w.bits_k, w.bits_v)
    Ks, Vs = lm.decode_layer(sc["idx_k"], sc["idx_v"], sc["scales_k"], sc["scales_v"], pos, Ct,
                             St, w.bits_k, w.bits_v)
    K0 = K_l[:, pos].astype(np.float64)
    V0 = V_l[:, pos].astype(np.float64)
    res = {"E8": (metrics(K0, Kh), metrics(V0, Vh)), "LloydMax": (metrics(K0, Ks), metrics(V0, Vs))}
    for name, ((sk, ck), (sv, cv)) in res.items():
        print(f"\n[quality] {name:8s} K{w.bits_k}: SNR {sk:5.2f} dB cos {ck:.4f} | "
              f"V{w.bits_v}: SNR {sv:5.2f} dB cos {cv:.4f}")
    for (sk, ck), (sv, cv) in res.values():
        assert sk > 5 and sv > 3 and ck > 0.9 and cv > 0.8
