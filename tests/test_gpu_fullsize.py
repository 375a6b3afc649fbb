"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (one launch over every tile).

The oracle cannot redo multi-GB workloads, so each test checks a seeded
sample of tiles (or sequences) element by element, and checks on every tile
properties that hold at any size.  Packed inputs of the dequantiser and the
attention kernel at the sampled positions are written by the oracle's
quantiser, never by the GPU's.

  prefill quantize   64 layers x 8 KV heads x 16384 tokens x 128, K4V2, 5 it
  dequantize         256 seq x 8 KV heads x 8192 tokens x 128
  head_dim sweep     8 KV heads x 32768 tokens, head_dim 64 / 96 / 256, 3 and 5 it
                     (all 2048 tiles per tensor checked)
  decode attention   64 seq x 8 KV heads x 32768 tokens, GQA 32/8
"""
import gc

import numpy as np
import pytest
import torch

import kv_cache_bit_token_amd as kv
import oracle
from kv_cache_bit_token_amd import synthetic
from parity import compare_attention, compare_codes, compare_dequant, compare_meta

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _unpack_gpu(codes, D, bits, is_key):
    """Packed tiles -> int8 codes [n][128][D] on the GPU (bit ops only)."""
    n = codes.shape[0]
    per = 8 // bits
    parts = [(codes >> (bits * i)) & ((1 << bits) - 1) for i in range(per)]
    c = torch.stack(parts, dim=-1).reshape(n, -1)       # element order
    if is_key:
        return c.reshape(n, 128, D)
    return c.reshape(n, D, 128).transpose(1, 2)


def _coverage(codes, D, bits, is_key, chunk=4096):
    """Every non-flat group spans codes 0 .. 2^b - 1 (min -> 0, max -> top)."""
    L = (1 << bits) - 1
    bad = 0
    for i in range(0, codes.shape[0], chunk):
        c = _unpack_gpu(codes[i:i + chunk], D, bits, is_key)
        ax = 1 if is_key else 2
        lo = c.amin(dim=ax)
        hi = c.amax(dim=ax)
        flat = hi == 0
        bad += int(((lo != 0) | ((hi != L) & ~flat)).sum())
    return bad


def _sample(n, k, seed):
    idx = np.sort(np.random.default_rng(seed).choice(n, k, replace=False))
    return np.unique(np.concatenate([[0, n - 1], idx]))


def _check_quant_sample(kt, vt, kc, vc, km, vm, idx, kb, vb, n_iters):
    d0 = kt.shape[-1]
    D = oracle.padded_dim(d0)
    it = torch.from_numpy(idx).to(kt.device)
    xk, xv = kt[it].cpu().numpy(), vt[it].cpu().numpy()
    qk = oracle.quantize_tiles(xk, kb, n_iters, True, diag=True)
    qv = oracle.quantize_tiles(xv, vb, n_iters, False, diag=True)
    return {
        "k": compare_codes(kc[it].cpu().numpy(), qk, D, kb, True),
        "v": compare_codes(vc[it].cpu().numpy(), qv, D, vb, False),
        "km": compare_meta(km[it].cpu().numpy(), qk["meta"], D, True),
        "vm": compare_meta(vm[it].cpu().numpy(), qv["meta"], D, False),
    }


def test_prefill_quantize_full_size():
    k, v = synthetic.layered_kv_torch(2, 64, 8, 16384, 128, DEV)
    kt, vt = k.view(-1, 128, 128), v.view(-1, 128, 128)
    kc, vc, km, vm = kv.quantize_tiles(kt, vt, k_bits=4, v_bits=2, n_iters=5)
    torch.cuda.synchronize()
    assert torch.isfinite(km.float()).all() and torch.isfinite(vm.float()).all()
    assert _coverage(kc, 128, 4, True) == 0
    assert _coverage(vc, 128, 2, False) == 0
    idx = _sample(kt.shape[0], 192, 2)
    print(_check_quant_sample(kt, vt, kc, vc, km, vm, idx, 4, 2, 5))
    del k, v, kt, vt, kc, vc, km, vm
    _free()


def test_dequantize_full_size():
    k, v = synthetic.outlier_kv_torch(1, 256 * 8, 8192, 128, DEV)
    kt, vt = k.view(-1, 128, 128), v.view(-1, 128, 128)
    kc, vc, km, vm = kv.quantize_tiles(kt, vt, k_bits=4, v_bits=2, n_iters=5)
    idx = _sample(kt.shape[0], 128, 1)
    it = torch.from_numpy(idx).to(DEV)
    qk = oracle.quantize_tiles(kt[it].cpu().numpy(), 4, 5, True)
    qv = oracle.quantize_tiles(vt[it].cpu().numpy(), 2, 5, False)
    kc[it] = torch.from_numpy(qk["codes"]).to(DEV)
    vc[it] = torch.from_numpy(qv["codes"]).to(DEV)
    km[it] = torch.from_numpy(qk["meta"]).to(DEV)
    vm[it] = torch.from_numpy(qv["meta"]).to(DEV)
    ko, vo = kv.dequantize_tiles(kc, vc, km, vm, head_dim=128)
    torch.cuda.synchronize()
    rk, _ = oracle.dequantize_tiles(qk["codes"], qk["meta"], 128, 4, True)
    rv, _ = oracle.dequantize_tiles(qv["codes"], qv["meta"], 128, 2, False)
    print(compare_dequant(ko[it].cpu().numpy(), rk), compare_dequant(vo[it].cpu().numpy(), rv))
    # every tile: finite output.  Reconstruction: almost every tile within a
    # loose relative bound; the exceptions are the rare tiles with an outlier
    # in channel 0 whose centred-std normalisation runs away (the oracle gives
    # the same values there; see tests/golden/runaway_tiles.txt)
    for x, y in ((kt, ko), (vt, vo)):
        assert torch.isfinite(y.float()).all()
        num = (x.float() - y.float()).pow(2).sum(dim=(1, 2)).sqrt()
        den = x.float().pow(2).sum(dim=(1, 2)).sqrt()
        rel = num / den
        print("tiles with relative error > 0.5:", int((rel > 0.5).sum()), "of", rel.numel(),
              "median %.4f" % float(rel.median()))
        assert int((rel > 0.5).sum()) <= 1e-4 * rel.numel()
    del k, v, kt, vt, kc, vc, km, vm, ko, vo
    _free()


@pytest.mark.parametrize("d0", [64, 96, 256])
def test_head_dim_sweep_full_size(d0):
    k, v = synthetic.outlier_kv_host(4, 8, 32768, d0)
    kt, vt = synthetic.as_tiles(k), synthetic.as_tiles(v)
    D = oracle.padded_dim(d0)
    gk, gv = torch.from_numpy(kt).to(DEV), torch.from_numpy(vt).to(DEV)
    for n_iters in (3, 5):
        kc, vc, km, vm = kv.quantize_tiles(gk, gv, k_bits=4, v_bits=2, n_iters=n_iters)
        kc, vc, km, vm = (t.cpu().numpy() for t in (kc, vc, km, vm))
        worst = {}
        for s in range(0, kt.shape[0], 256):
            sl = slice(s, s + 256)
            qk = oracle.quantize_tiles(kt[sl], 4, n_iters, True, diag=True)
            qv = oracle.quantize_tiles(vt[sl], 2, n_iters, False, diag=True)
            st = [compare_codes(kc[sl], qk, D, 4, True), compare_codes(vc[sl], qv, D, 2, False)]
            compare_meta(km[sl], qk["meta"], D, True)
            compare_meta(vm[sl], qv["meta"], D, False)
            worst["mismatch"] = worst.get("mismatch", 0) + sum(x["mismatch"] for x in st)
            # dequantiser over the oracle's packed tiles
            ko, vo = kv.dequantize_tiles(*(torch.from_numpy(a).to(DEV) for a in
                                           (qk["codes"], qv["codes"], qk["meta"], qv["meta"])),
                                         head_dim=d0)
            rk, _ = oracle.dequantize_tiles(qk["codes"], qk["meta"], d0, 4, True)
            rv, _ = oracle.dequantize_tiles(qv["codes"], qv["meta"], d0, 2, False)
            compare_dequant(ko.cpu().numpy(), rk)
            compare_dequant(vo.cpu().numpy(), rv)
        print(d0, n_iters, worst)
    del gk, gv
    _free()


def test_decode_attention_full_size():
    B, n_kv, Hq, T, d0 = 64, 8, 32, 32768, 128
    tps = T // 128
    k, v = synthetic.outlier_kv_torch(5, B * n_kv, T, d0, DEV)
    kt, vt = k.view(-1, 128, d0), v.view(-1, 128, d0)
    kc, vc, km, vm = kv.quantize_tiles(kt, vt, k_bits=4, v_bits=2, n_iters=5)
    q = synthetic.query_torch(5, B, Hq, d0, DEV)
    pairs = [(0, 0), (17, 3), (40, 6), (63, 7)]
    oc = {}
    for b, g in pairs:
        sl = slice((b * n_kv + g) * tps, (b * n_kv + g + 1) * tps)
        qk = oracle.quantize_tiles(kt[sl].cpu().numpy(), 4, 5, True)
        qv = oracle.quantize_tiles(vt[sl].cpu().numpy(), 2, 5, False)
        kc[sl], vc[sl] = torch.from_numpy(qk["codes"]).to(DEV), torch.from_numpy(qv["codes"]).to(DEV)
        km[sl], vm[sl] = torch.from_numpy(qk["meta"]).to(DEV), torch.from_numpy(qv["meta"]).to(DEV)
        oc[(b, g)] = (qk, qv)
    out = kv.decode_attention(q, kc, vc, km, vm, n_kv_heads=n_kv, tiles_per_seq=tps)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    qh = q.cpu().numpy()
    G = Hq // n_kv
    for (b, g), (qk, qv) in oc.items():
        qsel = qh[b:b + 1, g * G:(g + 1) * G]
        ref = oracle.decode_attention(qsel, qk["codes"], qv["codes"], qk["meta"], qv["meta"],
                                      n_kv_heads=1, tiles_per_seq=tps)
        print((b, g), compare_attention(out[b:b + 1, g * G:(g + 1) * G].cpu().numpy(), ref))
    # context: error of the quantised-cache attention against fp16-cache attention
    errs = []
    for b in range(0, B, 16):
        Kb = k.view(B, n_kv, T, d0)[b].float()
        Vb = v.view(B, n_kv, T, d0)[b].float()
        qb = q[b].float().view(n_kv, G, d0)
        s = torch.bmm(qb, Kb.transpose(1, 2).contiguous()) * d0 ** -0.5
        o = torch.bmm(torch.softmax(s, dim=-1), Vb).reshape(Hq, d0)
        errs.append(float((out[b] - o).norm() / o.norm()))
    print("relative L2 vs fp16-cache attention:", max(errs))
    del k, v, kt, vt, kc, vc, km, vm
    _free()


def test_decode_attention_fp16_full_size():
    """The fp16-cache baseline at the decode-attention workload's size:
    64 seq x 8 KV heads x 32768 tokens, GQA 32/8, sampled sequences checked
    against the oracle's fp16-cache attention."""
    B, n_kv, Hq, T, d0 = 64, 8, 32, 32768, 128
    k, v = synthetic.outlier_kv_torch(5, B * n_kv, T, d0, DEV)
    k, v = k.view(B, n_kv, T, d0), v.view(B, n_kv, T, d0)
    q = synthetic.query_torch(5, B, Hq, d0, DEV)
    out = kv.decode_attention_fp16(q, k, v)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    qh = q.cpu().numpy()
    for b in (0, 29, 63):
        ref = oracle.decode_attention_fp16(qh[b:b + 1], k[b:b + 1].cpu().numpy(),
                                           v[b:b + 1].cpu().numpy())
        print(b, compare_attention(out[b:b + 1].cpu().numpy(), ref))
    del k, v
    _free()
