"""Pins of the oracle's attention over an uncompressed fp16 cache.

Pages: hotdry page (blog.hotdry.top), section on the deployment parameters
(throughput is compared with an FP16 baseline); deep-dive page
(vatt-ghern.pages.dev), section on where the memory of a 16K-context
inference goes (each decode step reads the whole cache, so decode is bound by
memory bandwidth).  The baseline is plain softmax attention over the binary16
values.

Pins: torch's scaled_dot_product_attention in float64 on the CPU (an
independent library routine) with the GQA group expanded; two closed forms
(equal keys give the mean of the values; one dominant key gives its value);
the empty sequence.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_bit_token_amd import synthetic


def _sdpa(q16, k16, v16):
    B, Hq, d0 = q16.shape
    hkv = k16.shape[1]
    q = torch.from_numpy(q16.astype(np.float64)).reshape(B, Hq, 1, d0)
    K = torch.from_numpy(k16.astype(np.float64)).repeat_interleave(Hq // hkv, dim=1)
    V = torch.from_numpy(v16.astype(np.float64)).repeat_interleave(Hq // hkv, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=1.0 / np.sqrt(d0))
    return o.reshape(B, Hq, d0).numpy()


@pytest.mark.parametrize("B,hkv,hq,T,d0", [(2, 2, 8, 512, 128), (1, 1, 1, 200, 96),
                                           (3, 2, 6, 77, 64), (1, 1, 16, 300, 256)])
def test_fp16_attention_is_sdpa(B, hkv, hq, T, d0):
    k, v = synthetic.outlier_kv_host(13, B * hkv, T, d0)
    k, v = k.reshape(B, hkv, T, d0), v.reshape(B, hkv, T, d0)
    q = synthetic.query_host(13, B, hq, d0)
    o = oracle.decode_attention_fp16(q, k, v)
    assert np.allclose(o, _sdpa(q, k, v), rtol=0, atol=1e-12)


def test_fp16_attention_equal_keys_give_mean_value():
    rng = np.random.default_rng(3)
    T, d0 = 129, 64
    k = np.broadcast_to(rng.standard_normal(d0).astype(np.float16), (1, 1, T, d0)).copy()
    v = rng.standard_normal((1, 1, T, d0)).astype(np.float16)
    q = rng.standard_normal((1, 4, d0)).astype(np.float16)
    o = oracle.decode_attention_fp16(q, k, v)
    mean = v[0, 0].astype(np.float64).mean(0)
    for h in range(4):
        assert np.allclose(o[0, h], mean, rtol=0, atol=1e-13)


def test_fp16_attention_dominant_key_gives_its_value():
    rng = np.random.default_rng(4)
    T, d0 = 64, 64
    q = np.zeros((1, 1, d0), np.float16)
    q[0, 0, 0] = 1.0
    k = np.zeros((1, 1, T, d0), np.float16)
    k[0, 0, 37, 0] = 1000.0          # score 125 above the rest
    v = rng.standard_normal((1, 1, T, d0)).astype(np.float16)
    o = oracle.decode_attention_fp16(q, k, v)
    assert np.allclose(o[0, 0], v[0, 0, 37].astype(np.float64), rtol=0, atol=1e-40)


def test_fp16_attention_empty_sequence_is_zero():
    q = synthetic.query_host(1, 2, 4, 128)
    k = np.zeros((2, 1, 0, 128), np.float16)
    o = oracle.decode_attention_fp16(q, k, k.copy())
    assert np.array_equal(o, np.zeros_like(o))
