"""Host-side argument checks of the Python binding (no GPU): tensors of the wrong dtype, too few
elements or a non-contiguous layout are rejected with ValueError before any address reaches
the library, so a short or strided buffer can never send a kernel past its end. The
convenience chains also reject tensors that are not on a GPU and mismatched K/V shapes."""
import pytest
import torch

import kv_cache_compression_proxy_amd as nq

P = nq.make_params(2, 2, 64, 8, 600, 3, 2, 1e4)
N = nq.nq_keep_count(P)


def args_encode(**bad):
    L, H, T = 2, 2, 64
    a = dict(K=torch.zeros((L, H, T, 128), dtype=torch.float16),
             V=torch.zeros((L, H, T, 128), dtype=torch.float16),
             positions=torch.zeros((L, N), dtype=torch.int32),
             rope_cos=torch.zeros((T, 64)), rope_sin=torch.zeros((T, 64)),
             codes_k=torch.zeros((L, H, N, 128), dtype=torch.int8),
             codes_v=torch.zeros((L, H, N, 128), dtype=torch.int8),
             scales_k=torch.zeros((L, H, N, 16), dtype=torch.float16),
             scales_v=torch.zeros((L, H, N, 16), dtype=torch.float16))
    a.update(bad)
    return a


@pytest.mark.parametrize("name,bad", [
    ("K", torch.zeros((2, 2, 64, 128), dtype=torch.float32)),          # wrong dtype
    ("V", torch.zeros((2, 2, 63, 128), dtype=torch.float16)),          # one token short
    ("K", torch.zeros((2, 2, 128, 64), dtype=torch.float16).transpose(2, 3)),   # strided
    ("positions", torch.zeros((2, N - 1), dtype=torch.int32)),
    ("codes_v", torch.zeros((2, 2, N, 127), dtype=torch.int8)),
    ("scales_k", torch.zeros((2, 2, N, 16), dtype=torch.float32)),
    ("rope_sin", torch.zeros((64, 64), dtype=torch.float64)),
])
def test_encode_rejects_bad_tensors(name, bad):
    a = args_encode(**{name: bad})
    with pytest.raises(ValueError) as ei:
        nq.nq_encode(P, **a, stream=0)
    assert name in str(ei.value)


def test_decode_checks_output_dtype_against_the_mode():
    L, H, T = 2, 2, 64
    a = args_encode()
    out16 = torch.zeros((L, H, N, 128), dtype=torch.float16)
    with pytest.raises(ValueError) as ei:
        nq.nq_decode(P, a["codes_k"], a["codes_v"], a["scales_k"], a["scales_v"],
                     a["positions"], a["rope_cos"], a["rope_sin"], out16, out16, nq.NQ_OUT_F32,
                     None, stream=0)
    assert "K_out" in str(ei.value)


def test_attention_checks():
    Q = torch.zeros((2, 8, 128), dtype=torch.float16)
    out = torch.zeros((2, 8, 128), dtype=torch.float32)
    short = torch.zeros((2, 2, 10, 128), dtype=torch.float16)
    with pytest.raises(ValueError) as ei:
        nq.nq_attend_decode(P, Q, 8, short, short, 11, out, None, stream=0)
    assert "K" in str(ei.value)
    with pytest.raises(ValueError):
        nq.nq_decode_attend(P, torch.zeros(1, dtype=torch.int8), None, None, None, None, None,
                            None, Q, 8, out, None, stream=0)


def test_convenience_chains_reject_bad_inputs():
    K = torch.zeros((2, 2, 64, 128), dtype=torch.float16)
    with pytest.raises(ValueError):                      # not on a GPU
        nq.compress(K, K.clone())
    with pytest.raises(ValueError):
        nq.compress(K, K[:, :, :32].contiguous())
    with pytest.raises(ValueError):
        nq._check_q(torch.zeros((2, 6, 128), dtype=torch.float16), 2, 4)


def test_raw_addresses_pass_unchecked():
    """Integer addresses go straight to the library, which validates what it can (null,
    alignment) and returns its own status."""
    with pytest.raises(nq.NqError) as ei:
        nq.nq_encode(P, 2, 0, 0, 0, 0, 0, 0, 0, 0, stream=0)
    assert ei.value.status == nq.NQ_ERR_INVALID_ARG
