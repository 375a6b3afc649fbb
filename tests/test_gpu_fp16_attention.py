"""GPU parity of kvarn_decode_attention_fp16, the uncompressed-cache baseline.

Expected values come from the oracle's fp16-cache attention alone.  Shapes
cover several token steps and a ragged last step, every head_dim class
(64, padded 96 -> 128, 128, 256, and 40 -> 64), GQA groups of 1, 3, 4 and 16
heads, a single token, and the empty sequence.
"""
import numpy as np
import pytest
import torch

import kv_cache_bit_token_amd as kv
import oracle
from kv_cache_bit_token_amd import synthetic
from parity import compare_attention

pytestmark = pytest.mark.gpu


def _case(seed, B, hkv, hq, T, d0):
    k, v = synthetic.outlier_kv_host(seed, B * hkv, T, d0)
    k, v = k.reshape(B, hkv, T, d0), v.reshape(B, hkv, T, d0)
    q = synthetic.query_host(seed, B, hq, d0)
    return q, k, v


@pytest.mark.parametrize("B,hkv,hq,T,d0", [
    (2, 2, 8, 512, 128),     # G = 4, whole steps
    (2, 2, 8, 1000, 128),    # ragged last step
    (1, 1, 1, 200, 96),      # G = 1, padded head_dim
    (3, 2, 6, 77, 64),       # G = 3
    (1, 1, 16, 300, 256),    # G = 16
    (2, 1, 4, 129, 40),      # head_dim 40 -> 64
    (1, 2, 8, 1, 128),       # one token
    (1, 8, 32, 4096, 128),   # many splits per sequence
])
def test_fp16_attention_matches_oracle(B, hkv, hq, T, d0):
    q, k, v = _case(B * 100 + T, B, hkv, hq, T, d0)
    out = kv.decode_attention_fp16(torch.from_numpy(q).cuda(), torch.from_numpy(k).cuda(),
                                   torch.from_numpy(v).cuda())
    torch.cuda.synchronize()
    ref = oracle.decode_attention_fp16(q, k, v)
    print(compare_attention(out.cpu().numpy(), ref))


def test_fp16_attention_empty_sequence_is_zero():
    q = torch.from_numpy(synthetic.query_host(2, 2, 4, 128)).cuda()
    k = torch.zeros((2, 1, 0, 128), dtype=torch.float16, device="cuda")
    out = kv.decode_attention_fp16(q, k, k.clone())
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), torch.zeros((2, 4, 128)))


def test_fp16_attention_scale_argument():
    q, k, v = _case(5, 1, 2, 8, 300, 128)
    out = kv.decode_attention_fp16(torch.from_numpy(q).cuda(), torch.from_numpy(k).cuda(),
                                   torch.from_numpy(v).cuda(), sm_scale=0.05)
    torch.cuda.synchronize()
    ref = oracle.decode_attention_fp16(q, k, v, sm_scale=0.05)
    print(compare_attention(out.cpu().numpy(), ref))


@pytest.mark.parametrize("B,hkv,hq,T,d0", [
    (2, 2, 8, 1000, 128),    # ragged last step of 8 of 32 tokens
    (2, 1, 4, 129, 40),      # head_dim 40 -> 64: 1 of 64 tokens
    (1, 1, 16, 300, 256),    # 12 of 16 tokens
])
def test_fp16_attention_ignores_memory_past_the_cache(B, hkv, hq, T, d0):
    """K and V are the front of larger buffers whose tail is fp16 NaN: rows
    past the sequence end must never be read (a stray NaN V row would turn
    the output NaN through 0 x NaN in p.V)."""
    q, k, v = _case(B * 100 + T + 7, B, hkv, hq, T, d0)
    n = k.size
    spare = 256 * d0   # more than a step of rows
    bufs = []
    for x in (k, v):
        buf = torch.full((n + spare,), float("nan"), dtype=torch.float16, device="cuda")
        buf[:n] = torch.from_numpy(x.reshape(-1)).cuda()
        bufs.append(buf[:n].view(B, hkv, T, d0))
    out = kv.decode_attention_fp16(torch.from_numpy(q).cuda(), bufs[0], bufs[1])
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.isfinite(o).all()
    print(compare_attention(o, oracle.decode_attention_fp16(q, k, v)))
