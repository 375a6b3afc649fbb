"""GPU parity of the paged-cache entry points: kvarn_quantize_tiles_to and
kvarn_decode_attention_paged (deep page, running inside vLLM's
PagedAttention: a 128-token page is one tile whose scales travel with it,
and the unfilled page stays in fp16 in a decode workspace).

The attention tests read pools packed by the oracle's quantiser; expected
values come from oracle.decode_attention_paged.  The block layouts (empty
sequences, tail-only ones, full ones, shuffled physical blocks) come from
kv_cache_bit_token_amd.paged.
"""
import numpy as np
import pytest
import torch

import kv_cache_bit_token_amd as kv
import oracle
from kv_cache_bit_token_amd import synthetic
from kv_cache_bit_token_amd.paged import paged_layout
from parity import compare_attention, compare_codes, compare_meta

pytestmark = pytest.mark.gpu


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_quantize_tiles_to_scatters_and_skips():
    d0, n_in, pool = 128, 6, 9
    k, v = synthetic.outlier_kv_host(51, n_in, 128, d0)
    kt, vt = synthetic.as_tiles(k), synthetic.as_tiles(v)
    dst = np.array([7, 2, -1, 5, 9, 0], np.int64)      # -1 and 9 fall outside the pool
    lay = kv.get_layout(d0, 4, 2, 5)
    kc = torch.full((pool, lay["k_code_bytes"]), 0xAB, dtype=torch.uint8, device="cuda")
    vc = torch.full((pool, lay["v_code_bytes"]), 0xAB, dtype=torch.uint8, device="cuda")
    km = torch.full((pool, lay["k_meta_bytes"] // 2), 7.0, dtype=torch.float16, device="cuda")
    vm = torch.full((pool, lay["v_meta_bytes"] // 2), 7.0, dtype=torch.float16, device="cuda")
    kv.quantize_tiles_to(_cuda(kt), _cuda(vt), _cuda(dst), kc, vc, km, vm)
    torch.cuda.synchronize()
    kc, vc, km, vm = (t.cpu().numpy() for t in (kc, vc, km, vm))
    live = [(i, int(s)) for i, s in enumerate(dst) if 0 <= s < pool]
    src = [i for i, _ in live]
    slots = [s for _, s in live]
    qk = oracle.quantize_tiles(kt[src], 4, 5, True, diag=True)
    qv = oracle.quantize_tiles(vt[src], 2, 5, False, diag=True)
    print(compare_codes(kc[slots], qk, 128, 4, True), compare_codes(vc[slots], qv, 128, 2, False))
    compare_meta(km[slots], qk["meta"], 128, True)
    compare_meta(vm[slots], qv["meta"], 128, False)
    untouched = [s for s in range(pool) if s not in slots]
    assert np.all(kc[untouched] == 0xAB) and np.all(vc[untouched] == 0xAB)
    assert np.all(km[untouched] == 7.0) and np.all(vm[untouched] == 7.0)


def _oracle_pool(seed, pool_blocks, n_kv, d0, kb=4, vb=2):
    k, v = synthetic.outlier_kv_host(seed, pool_blocks * n_kv, 128, d0)
    qk = oracle.quantize_tiles(synthetic.as_tiles(k), kb, 5, True)
    qv = oracle.quantize_tiles(synthetic.as_tiles(v), vb, 5, False)
    return qk, qv


@pytest.mark.parametrize("B,n_kv,Hq,max_blocks,d0", [(6, 2, 8, 4, 128), (3, 1, 1, 2, 96),
                                                     (4, 4, 64, 3, 64), (4, 8, 32, 3, 256),
                                                     (5, 2, 4, 1, 128), (3, 1, 16, 2, 256)])
def test_paged_attention_oracle_packed(B, n_kv, Hq, max_blocks, d0):
    table, nb, tl, pool = paged_layout(60 + B, B, max_blocks)
    qk, qv = _oracle_pool(61 + B, pool, n_kv, d0)
    kt, vt = synthetic.outlier_kv_host(62 + B, B * n_kv, 128, d0)
    kt, vt = kt.reshape(B, n_kv, 128, d0), vt.reshape(B, n_kv, 128, d0)
    q = synthetic.query_host(63 + B, B, Hq, d0)
    ref = oracle.decode_attention_paged(q, qk["codes"], qv["codes"], qk["meta"], qv["meta"], table,
                                        nb, tl, kt, vt, n_kv_heads=n_kv)
    out = kv.decode_attention_paged(_cuda(q), _cuda(qk["codes"]), _cuda(qv["codes"]),
                                    _cuda(qk["meta"]), _cuda(qv["meta"]), _cuda(table), _cuda(nb),
                                    _cuda(tl), _cuda(kt), _cuda(vt), n_kv_heads=n_kv)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    print(table.tolist(), nb.tolist(), tl.tolist(), compare_attention(o, ref))
    for b in range(B):
        if nb[b] == 0 and tl[b] == 0:
            assert np.all(o[b] == 0.0)


def test_paged_attention_other_presets():
    B, n_kv, Hq, max_blocks, d0 = 4, 2, 8, 3, 128
    table, nb, tl, pool = paged_layout(70, B, max_blocks)
    kt, vt = synthetic.outlier_kv_host(71, B * n_kv, 128, d0)
    kt, vt = kt.reshape(B, n_kv, 128, d0), vt.reshape(B, n_kv, 128, d0)
    q = synthetic.query_host(72, B, Hq, d0)
    for kb, vb in ((4, 4), (2, 2), (2, 4)):
        qk, qv = _oracle_pool(73, pool, n_kv, d0, kb, vb)
        ref = oracle.decode_attention_paged(q, qk["codes"], qv["codes"], qk["meta"], qv["meta"],
                                            table, nb, tl, kt, vt, n_kv_heads=n_kv, k_bits=kb,
                                            v_bits=vb)
        out = kv.decode_attention_paged(_cuda(q), _cuda(qk["codes"]), _cuda(qv["codes"]),
                                        _cuda(qk["meta"]), _cuda(qv["meta"]), _cuda(table),
                                        _cuda(nb), _cuda(tl), _cuda(kt), _cuda(vt),
                                        n_kv_heads=n_kv, k_bits=kb, v_bits=vb)
        torch.cuda.synchronize()
        print(kb, vb, compare_attention(out.cpu().numpy(), ref))


def test_paged_attention_without_pool_is_tail_attention():
    """No packed blocks at all (pool of zero tiles): only the fp16 tails."""
    B, n_kv, Hq, d0 = 3, 2, 8, 128
    kt, vt = synthetic.outlier_kv_host(80, B * n_kv, 128, d0)
    kt, vt = kt.reshape(B, n_kv, 128, d0), vt.reshape(B, n_kv, 128, d0)
    q = synthetic.query_host(81, B, Hq, d0)
    tl = np.array([128, 0, 33], np.int32)
    nb = np.zeros(B, np.int32)
    table = np.zeros((B, 2), np.int32)
    empty_c = np.zeros((0, 8192), np.uint8)
    empty_m = np.zeros((0, 384), np.float16)
    ref = oracle.decode_attention_paged(q, empty_c, empty_c, empty_m, empty_m, table, nb, tl, kt, vt,
                                        n_kv_heads=n_kv)
    ec = torch.empty((0, 8192), dtype=torch.uint8, device="cuda")
    em = torch.empty((0, 384), dtype=torch.float16, device="cuda")
    out = kv.decode_attention_paged(_cuda(q), ec, torch.empty((0, 4096), dtype=torch.uint8,
                                                              device="cuda"),
                                    em, em, _cuda(table), _cuda(nb), _cuda(tl), _cuda(kt),
                                    _cuda(vt), n_kv_heads=n_kv)
    torch.cuda.synchronize()
    print(compare_attention(out.cpu().numpy(), ref))
    assert np.all(out[1].cpu().numpy() == 0.0)


def test_paged_attention_bad_table_entries_stay_in_bounds():
    """Entries outside the pool are read as block 0: finite output, no fault."""
    B, n_kv, Hq, max_blocks, d0 = 2, 2, 8, 3, 128
    table, nb, tl, pool = paged_layout(90, B, max_blocks, full=True)
    qk, qv = _oracle_pool(91, pool, n_kv, d0)
    table[0, 1] = -7
    table[1, 2] = pool + 100
    kt, vt = synthetic.outlier_kv_host(92, B * n_kv, 128, d0)
    kt, vt = kt.reshape(B, n_kv, 128, d0), vt.reshape(B, n_kv, 128, d0)
    q = synthetic.query_host(93, B, Hq, d0)
    out = kv.decode_attention_paged(_cuda(q), _cuda(qk["codes"]), _cuda(qv["codes"]),
                                    _cuda(qk["meta"]), _cuda(qv["meta"]), _cuda(table), _cuda(nb),
                                    _cuda(tl), _cuda(kt), _cuda(vt), n_kv_heads=n_kv)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    # entries read as block 0 give the oracle's answer for that reading
    t2 = np.where((table < 0) | (table >= pool), 0, table).astype(np.int32)
    ref = oracle.decode_attention_paged(q, qk["codes"], qv["codes"], qk["meta"], qv["meta"], t2,
                                        nb, tl, kt, vt, n_kv_heads=n_kv)
    print(compare_attention(out.cpu().numpy(), ref))


def test_decode_append_flow():
    """Tokens arrive one decode step at a time: the tail fills, a full tail is
    quantised into a fresh pool block (kvarn_quantize_tiles_to), attention
    runs over blocks + tail after every step.  At checkpoints: the GPU-written
    pool blocks match the oracle's quantisation of the same tokens (quantiser
    parity), and attention over the oracle's pool in the GPU's state (table,
    counts, tails) matches the oracle (attention parity); the attention the
    flow itself computed over its own pool agrees with that to the scales'
    tolerance (relative L2 <= 1e-3)."""
    B, n_kv, Hq, d0 = 2, 2, 8, 128
    steps = 140                                  # crosses one block boundary
    k_all, v_all = synthetic.outlier_kv_host(95, B * n_kv, 256, d0)
    k_all = k_all.reshape(B, n_kv, 256, d0)
    v_all = v_all.reshape(B, n_kv, 256, d0)
    q_all = np.stack([synthetic.query_host(96 + s, B, Hq, d0) for s in range(steps)])
    max_blocks, pool_blocks = 2, 4
    lay = kv.get_layout(d0, 4, 2, 5)
    shapes = [(lay["k_code_bytes"], torch.uint8), (lay["v_code_bytes"], torch.uint8),
              (lay["k_meta_bytes"] // 2, torch.float16), (lay["v_meta_bytes"] // 2, torch.float16)]
    kc, vc, km, vm = (torch.zeros((pool_blocks * n_kv, w), dtype=dt, device="cuda") for w, dt in shapes)
    ktail = torch.zeros((B, n_kv, 128, d0), dtype=torch.float16, device="cuda")
    vtail = torch.zeros_like(ktail)
    table = np.zeros((B, max_blocks), np.int32)
    nb = np.zeros(B, np.int32)
    tl = np.zeros(B, np.int32)
    free = [3, 1, 0, 2]                          # pool blocks handed out in this order
    for s in range(steps):
        for b in range(B):                        # append token s of every sequence
            ktail[b, :, tl[b]] = torch.from_numpy(k_all[b, :, s]).cuda()
            vtail[b, :, tl[b]] = torch.from_numpy(v_all[b, :, s]).cuda()
            tl[b] += 1
            if tl[b] == 128:                      # full page: quantise it into a new block
                blk = free.pop(0)
                dst = torch.tensor([blk * n_kv + g for g in range(n_kv)], dtype=torch.int64,
                                   device="cuda")
                kv.quantize_tiles_to(ktail[b], vtail[b], dst, kc, vc, km, vm)
                table[b, nb[b]] = blk
                nb[b] += 1
                tl[b] = 0
        out = kv.decode_attention_paged(_cuda(q_all[s]), kc, vc, km, vm, _cuda(table), _cuda(nb),
                                        _cuda(tl), ktail, vtail, n_kv_heads=n_kv)
        if s not in (0, 126, 127, 128, steps - 1):
            continue
        torch.cuda.synchronize()
        pool_np = [t.cpu().numpy() for t in (kc, vc, km, vm)]
        okc, ovc, okm, ovm = (np.zeros_like(a) for a in pool_np)
        for b in range(B):
            for i in range(nb[b]):
                blk = table[b, i]
                rows = slice(blk * n_kv, (blk + 1) * n_kv)
                qk = oracle.quantize_tiles(k_all[b, :, 128 * i:128 * (i + 1)], 4, 5, True, diag=True)
                qv = oracle.quantize_tiles(v_all[b, :, 128 * i:128 * (i + 1)], 2, 5, False, diag=True)
                compare_codes(pool_np[0][rows], qk, 128, 4, True)
                compare_codes(pool_np[1][rows], qv, 128, 2, False)
                compare_meta(pool_np[2][rows], qk["meta"], 128, True)
                compare_meta(pool_np[3][rows], qv["meta"], 128, False)
                okc[rows], ovc[rows], okm[rows], ovm[rows] = qk["codes"], qv["codes"], qk["meta"], qv["meta"]
        kt_np, vt_np = ktail.cpu().numpy(), vtail.cpu().numpy()
        ref = oracle.decode_attention_paged(q_all[s], okc, ovc, okm, ovm, table, nb, tl, kt_np,
                                            vt_np, n_kv_heads=n_kv)
        on_oracle_pool = kv.decode_attention_paged(
            _cuda(q_all[s]), _cuda(okc), _cuda(ovc), _cuda(okm), _cuda(ovm), _cuda(table),
            _cuda(nb), _cuda(tl), ktail, vtail, n_kv_heads=n_kv)
        torch.cuda.synchronize()
        r = compare_attention(on_oracle_pool.cpu().numpy(), ref)
        o = out.cpu().numpy()
        rel = float(np.linalg.norm(o - ref) / np.linalg.norm(ref))
        print("step", s, "blocks", nb.tolist(), "tail", tl.tolist(), r, "flow rel L2 %.2e" % rel)
        assert rel <= 1e-3
