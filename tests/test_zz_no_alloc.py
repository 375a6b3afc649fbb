"""kvarn_decode_attention_noalloc: the attention entry point that allocates
nothing (its scratch is the library's static device array).

Two calls in a row through the C ABI, the second with a smaller input, each
checked against kvarn_decode_attention (the caller-workspace entry point) on
the same oracle-packed cache, and the first against the oracle too.  A shape
whose workspace exceeds the static buffer is refused before any launch.
"""
import numpy as np
import pytest
import torch

import kv_cache_bit_token_amd as kv
import oracle
from kv_cache_bit_token_amd import synthetic
from parity import compare_attention, record

pytestmark = pytest.mark.gpu


def _case(seed, B, n_kv, Hq, T, d0):
    k, v = synthetic.outlier_kv_host(seed, B * n_kv, T, d0)
    qk = oracle.quantize_tiles(synthetic.as_tiles(k), 4, 5, True)
    qv = oracle.quantize_tiles(synthetic.as_tiles(v), 2, 5, False)
    q = synthetic.query_host(seed, B, Hq, d0)
    return q, qk, qv


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_noalloc_matches_workspace_entry_point_twice():
    shapes = [(4, 2, 8, 1024, 128), (2, 1, 4, 256, 64)]   # second call smaller
    for i, (B, n_kv, Hq, T, d0) in enumerate(shapes):
        q, qk, qv = _case(40 + i, B, n_kv, Hq, T, d0)
        args = [_cuda(x) for x in (q, qk["codes"], qv["codes"], qk["meta"], qv["meta"])]
        tps = T // 128
        out_s = torch.full((B, Hq, d0), float("nan"), dtype=torch.float32, device="cuda")
        kv.decode_attention_noalloc(*args, out_s, n_kv_heads=n_kv, tiles_per_seq=tps)
        out_w = kv.decode_attention(*args, n_kv_heads=n_kv, tiles_per_seq=tps)
        torch.cuda.synchronize()
        a, b = out_s.cpu().numpy(), out_w.cpu().numpy()
        stats = compare_attention(a, b)
        stats["identical"] = bool(np.array_equal(a, b))
        if i == 0:
            ref = oracle.decode_attention(q, qk["codes"], qv["codes"], qk["meta"], qv["meta"],
                                          n_kv_heads=n_kv, tiles_per_seq=tps)
            stats["vs_oracle"] = compare_attention(a, ref)["attn_abs"]
        record("noalloc attention call %d %s" % (i + 1, (B, n_kv, Hq, T, d0)), stats)
        assert stats["identical"], stats


def test_noalloc_refuses_shapes_beyond_the_static_scratch():
    # G = 16 at head_dim 256 with 8192 (sequence, KV head) pairs needs
    # 8192 * 16 * 258 * 4 bytes of split partials: above 64 MiB
    q = torch.zeros((8192, 16, 256), dtype=torch.float16, device="cuda")
    c = torch.zeros((8192, 16384), dtype=torch.uint8, device="cuda")
    vc = torch.zeros((8192, 8192), dtype=torch.uint8, device="cuda")
    km = torch.zeros((8192, 640), dtype=torch.float16, device="cuda")
    vm = torch.zeros((8192, 512), dtype=torch.float16, device="cuda")
    out = torch.zeros((8192, 16, 256), dtype=torch.float32, device="cuda")
    with pytest.raises(kv.KvarnError, match="KVARN_E_WORKSPACE"):
        kv.decode_attention_noalloc(q, c, vc, km, vm, out, n_kv_heads=1, tiles_per_seq=1)
