"""GPU parity of kvarn_dequantize_tiles and kvarn_decode_attention.

Both kernels read packed caches written by the oracle's quantiser (or drawn
at random), never by the GPU quantiser, so every expected value comes from
the oracle alone.
"""
import numpy as np
import pytest
import torch

import kv_cache_bit_token_amd as kv
import oracle
from kv_cache_bit_token_amd import synthetic
from parity import compare_attention, compare_dequant, packed_cache, record

pytestmark = pytest.mark.gpu


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _oracle_cache(seed, heads, tokens, d0, kb=4, vb=2, n_iters=5):
    k, v = synthetic.outlier_kv_host(seed, heads, tokens, d0)
    kt, vt = synthetic.as_tiles(k), synthetic.as_tiles(v)
    qk = oracle.quantize_tiles(kt, kb, n_iters, True)
    qv = oracle.quantize_tiles(vt, vb, n_iters, False)
    return k, v, qk, qv


def _gpu_dequant(qk, qv, d0, kb, vb):
    ko, vo = kv.dequantize_tiles(_cuda(qk["codes"]), _cuda(qv["codes"]), _cuda(qk["meta"]),
                                 _cuda(qv["meta"]), head_dim=d0, k_bits=kb, v_bits=vb)
    torch.cuda.synchronize()
    return ko.cpu().numpy(), vo.cpu().numpy()


@pytest.mark.parametrize("d0,kb,vb", [(128, 4, 2), (128, 4, 4), (128, 2, 2), (128, 2, 4),
                                      (64, 4, 2), (96, 4, 2), (256, 4, 2), (40, 4, 2),
                                      (200, 4, 2), (64, 2, 4), (256, 4, 4), (96, 2, 2),
                                      (256, 2, 4)])
def test_dequantize_oracle_packed(d0, kb, vb):
    _, _, qk, qv = _oracle_cache(6, 2, 384, d0, kb, vb)
    ko, vo = _gpu_dequant(qk, qv, d0, kb, vb)
    rk, _ = oracle.dequantize_tiles(qk["codes"], qk["meta"], d0, kb, True)
    rv, _ = oracle.dequantize_tiles(qv["codes"], qv["meta"], d0, vb, False)
    print(compare_dequant(ko, rk), compare_dequant(vo, rv))


@pytest.mark.parametrize("d0", [128, 64, 256])
def test_dequantize_random_packed(d0):
    rng = np.random.default_rng(d0)
    n = 5
    D = oracle.padded_dim(d0)
    kc = rng.integers(0, 256, size=(n, oracle.code_bytes(D, 4)), dtype=np.uint8)
    vc = rng.integers(0, 256, size=(n, oracle.code_bytes(D, 2)), dtype=np.uint8)
    km = np.concatenate([rng.uniform(0.01, 2.0, (n, D)), rng.uniform(-10, 10, (n, D)),
                         rng.uniform(0.1, 5.0, (n, 128))], axis=1).astype(np.float16)
    vm = np.concatenate([rng.uniform(0.01, 2.0, (n, 128)), rng.uniform(-3, 3, (n, 128)),
                         rng.uniform(0.1, 5.0, (n, D))], axis=1).astype(np.float16)
    qk, qv = {"codes": kc, "meta": km}, {"codes": vc, "meta": vm}
    ko, vo = _gpu_dequant(qk, qv, d0, 4, 2)
    rk, _ = oracle.dequantize_tiles(kc, km, d0, 4, True)
    rv, _ = oracle.dequantize_tiles(vc, vm, d0, 2, False)
    print(compare_dequant(ko, rk), compare_dequant(vo, rv))



@pytest.mark.parametrize("d0,kb,vb", [(128, 4, 2), (96, 2, 4), (256, 4, 4)])
def test_dequantize_skipping_one_tensor(d0, kb, vb):
    """K alone and V alone give the same bytes as both in one call: the grid
    then covers only the tensor given, and every tile is dequantised by a
    workgroup of its own either way."""
    _, _, qk, qv = _oracle_cache(9, 2, 384, d0, kb, vb)
    kc, vc, km, vm = (_cuda(x) for x in (qk["codes"], qv["codes"], qk["meta"], qv["meta"]))
    ko, vo = kv.dequantize_tiles(kc, vc, km, vm, head_dim=d0, k_bits=kb, v_bits=vb)
    ko1, none_v = kv.dequantize_tiles(kc, None, km, None, head_dim=d0, k_bits=kb, v_bits=vb)
    none_k, vo1 = kv.dequantize_tiles(None, vc, None, vm, head_dim=d0, k_bits=kb, v_bits=vb)
    torch.cuda.synchronize()
    assert none_v is None and none_k is None
    assert torch.equal(ko, ko1) and torch.equal(vo, vo1)
    rk, _ = oracle.dequantize_tiles(qk["codes"], qk["meta"], d0, kb, True)
    rv, _ = oracle.dequantize_tiles(qv["codes"], qv["meta"], d0, vb, False)
    record("dequantize one tensor at a time %s" % ((d0, kb, vb),),
           {"k": compare_dequant(ko1.cpu().numpy(), rk), "v": compare_dequant(vo1.cpu().numpy(), rv)})

def _attention_case(B, n_kv, Hq, T, d0, seed, kb=4, vb=2):
    k, v, qk, qv = _oracle_cache(seed, B * n_kv, T, d0, kb, vb)
    q = synthetic.query_host(seed, B, Hq, d0)
    out = kv.decode_attention(_cuda(q), _cuda(qk["codes"]), _cuda(qv["codes"]), _cuda(qk["meta"]),
                              _cuda(qv["meta"]), n_kv_heads=n_kv, tiles_per_seq=T // 128,
                              k_bits=kb, v_bits=vb)
    torch.cuda.synchronize()
    ref = oracle.decode_attention(q, qk["codes"], qv["codes"], qk["meta"], qv["meta"],
                                  n_kv_heads=n_kv, tiles_per_seq=T // 128, k_bits=kb, v_bits=vb)
    return out.cpu().numpy(), ref


@pytest.mark.parametrize("B,n_kv,Hq,T,d0", [(2, 2, 8, 512, 128), (1, 1, 1, 128, 128),
                                            (2, 1, 8, 384, 128), (1, 2, 32, 256, 128),
                                            (1, 2, 8, 512, 96), (2, 2, 4, 256, 64),
                                            (1, 1, 4, 256, 256)])
def test_attention_oracle_packed(B, n_kv, Hq, T, d0):
    out, ref = _attention_case(B, n_kv, Hq, T, d0, seed=B * 100 + Hq + d0)
    print(compare_attention(out, ref))


@pytest.mark.parametrize("B,n_kv,Hq,T,d0", [(1, 2, 12, 384, 64), (2, 1, 6, 256, 256),
                                            (1, 1, 16, 640, 256), (1, 3, 48, 256, 200),
                                            (2, 2, 10, 128, 72)])
def test_attention_group_sizes_and_widths(B, n_kv, Hq, T, d0):
    # groups of 6, 10, 12 and 16 query heads (the wide-group kernel) at the
    # other padded widths, ragged head_dims included
    out, ref = _attention_case(B, n_kv, Hq, T, d0, seed=B * 1000 + Hq * 7 + d0)
    print(compare_attention(out, ref))


@pytest.mark.parametrize("B,n_kv,Hq,tiles,d0", [(1, 1, 4, 150, 128), (2, 1, 8, 100, 64)])
def test_attention_more_than_64_splits(B, n_kv, Hq, tiles, d0):
    """Few (sequence, KV head) pairs over many tiles: one tile per split, so
    the combine kernel merges more than 64 splits per head and walks its
    weights in several chunks of 64."""
    wsb = kv.decode_attention_workspace(batch=B, n_q_heads=Hq, n_kv_heads=n_kv, tiles_per_seq=tiles,
                                        head_dim=d0)
    D = oracle.padded_dim(d0)
    assert wsb >= B * Hq * 65 * (D + 2) * 4, "fewer than 65 splits: the case would not span two chunks"
    out, ref = _attention_case(B, n_kv, Hq, tiles * 128, d0, seed=tiles + d0)
    record("attention, more than 64 splits %s" % ((B, n_kv, Hq, tiles, d0),), compare_attention(out, ref))


@pytest.mark.parametrize("tiles,d0", [(16, 128), (17, 128), (16, 256), (17, 64)])
def test_attention_combine_part_counts(tiles, d0):
    """16 and 17 splits per head (one tile each): the combine kernel reads up
    to 16 parts in a single round of loads and more in its loop over chunks;
    both sides of that boundary match the oracle."""
    wsb = kv.decode_attention_workspace(batch=1, n_q_heads=4, n_kv_heads=1, tiles_per_seq=tiles,
                                        head_dim=d0)
    D = oracle.padded_dim(d0)
    assert wsb == 4 * tiles * (D + 2) * 4, "expected one split per tile"
    out, ref = _attention_case(1, 1, 4, tiles * 128, d0, seed=tiles * 7 + d0)
    record("attention, %d parts per head, head_dim %d" % (tiles, d0), compare_attention(out, ref))


def test_attention_other_presets():
    for kb, vb in ((4, 4), (2, 2), (2, 4)):
        out, ref = _attention_case(1, 2, 8, 256, 128, seed=3, kb=kb, vb=vb)
        print(kb, vb, compare_attention(out, ref))


def test_attention_empty_cache_is_zero():
    q = _cuda(synthetic.query_host(0, 2, 8, 128))
    c = torch.zeros((1, 16), dtype=torch.uint8, device="cuda")
    m = torch.zeros((1, 8), dtype=torch.float16, device="cuda")
    out = kv.decode_attention(q, c, c, m, m, n_kv_heads=2, tiles_per_seq=0)
    torch.cuda.synchronize()
    assert not out.cpu().numpy().any()


@pytest.mark.parametrize("B,n_kv,Hq,tps,d0", [(128, 8, 32, 13, 128), (256, 4, 32, 9, 64)])
def test_attention_several_tiles_per_split(B, n_kv, Hq, tps, d0):
    """Enough (sequence, KV head) pairs that each split runs several tiles
    (1024 pairs -> 2 splits per pair, split s taking every other tile from
    tile s: 7 + 6 and 5 + 4 tiles), so the online softmax rescales across a
    split's tiles, the next-tile prefetch runs inside a split, and the combine
    merges interleaved splits.  The cache is assembled from 256 oracle-quantised tiles of
    the config-1 recipe, drawn at random per position; the host checks that a
    later tile of a split often holds a head's largest score, so the running
    maximum really moves inside splits."""
    D = oracle.padded_dim(d0)
    wsb = kv.decode_attention_workspace(batch=B, n_q_heads=Hq, n_kv_heads=n_kv, tiles_per_seq=tps,
                                        head_dim=d0)
    assert wsb == B * Hq * 2 * (D + 2) * 4, "expected two splits per (sequence, KV head)"
    rng = np.random.default_rng(B + d0)
    k, v = synthetic.outlier_kv_host(B + tps, 2, 128 * 128, d0)
    kt, vt = synthetic.as_tiles(k), synthetic.as_tiles(v)      # 256 tiles each
    qk = oracle.quantize_tiles(kt, 4, 5, True)
    qv = oracle.quantize_tiles(vt, 2, 5, False)
    idx = rng.integers(0, kt.shape[0], size=B * n_kv * tps)
    kc, km = qk["codes"][idx], qk["meta"][idx]
    vc, vm = qv["codes"][idx], qv["meta"][idx]
    q = synthetic.query_host(B * 3 + d0, B, Hq, d0)
    out = kv.decode_attention(_cuda(q), _cuda(kc), _cuda(vc), _cuda(km), _cuda(vm),
                              n_kv_heads=n_kv, tiles_per_seq=tps)
    torch.cuda.synchronize()
    ref = oracle.decode_attention(q, kc, vc, km, vm, n_kv_heads=n_kv, tiles_per_seq=tps)
    record("attention, several tiles per split %s" % ((B, n_kv, Hq, tps, d0),),
           compare_attention(out.cpu().numpy(), ref,
                             packed_cache(q, kc, vc, km, vm, n_kv, tps)))
    # the first split (tiles 0, 2, 4, ...) of each of the first 8 sequences'
    # (KV head, query head): in how many does the largest score sit past the
    # split's first tile?
    kd, _ = oracle.dequantize_tiles(qk["codes"], qk["meta"], d0, 4, True)    # [256][128][d0]
    G = Hq // n_kv
    later = total = 0
    for b in range(8):
        for g in range(n_kv):
            tiles = idx[(b * n_kv + g) * tps + np.arange(0, tps, 2)]
            keys = kd[tiles].reshape(-1, d0)
            s = q[b, g * G:(g + 1) * G].astype(np.float64) @ keys.T
            later += int((s.argmax(axis=1) >= 128).sum())
            total += G
    assert later >= 0.5 * total, (later, total)
