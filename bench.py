"""Benchmark of the KVarN hot path on one MI355X.

Workload: the prefill cache of a 64-layer, 8-KV-head, head_dim-128 model at
16384 tokens (fp16 K and V of [64*8][16384][128], about 4.3 GB), seeded
synthetic values with per-layer outlier channels and lognormal token
magnitudes.  One step runs the whole hot path over it:
  1. kvarn_quantize_tiles   (K4V2, 128-token tiles, 5 normalisation iterations)
  2. kvarn_dequantize_tiles (back to fp16)
  3. kvarn_decode_attention (one decode query per layer: 32 query heads over
     the 8 KV heads, all 16384 cached tokens, GQA)
Inputs are resident in HBM before timing starts.  `value` counts the
fp16-equivalent KV bytes the step moves through the path (the fp16 K/V fed to
the quantiser, produced by the dequantiser and represented by the cache the
attention reads) per second.  Per-stage times come from HIP events recorded on
the stream the kernels run on.

Prints one JSON line.  `--gpus` above 1 exits: this build runs on one GPU.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
LAYERS, KV_HEADS, TOKENS, HEAD_DIM, Q_HEADS = 64, 8, 16384, 128, 32
K_BITS, V_BITS, N_ITERS = 4, 2, 5


def per_tile_bytes(D):
    kc = 128 * D * K_BITS // 8
    vc = 128 * D * V_BITS // 8
    km = 2 * (2 * D + 128)
    vm = 2 * (256 + D)
    fp16 = 2 * 128 * D
    return {"fp16_pair": 2 * fp16, "packed_pair": kc + vc + km + vm}


def cpu_baseline(k, v, q, n_seq):
    """The oracle, untuned, on the first n_seq (layer, head) sequences."""
    import numpy as np
    import oracle

    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    tiles_per_seq = TOKENS // 128
    n_tiles = n_seq * tiles_per_seq
    kt = k.view(-1, 128, HEAD_DIM)[:n_tiles].cpu().numpy()
    vt = v.view(-1, 128, HEAD_DIM)[:n_tiles].cpu().numpy()
    n_layers = n_seq // KV_HEADS
    qh = q[:n_layers].cpu().numpy()
    t0 = time.perf_counter()
    qk = oracle.quantize_tiles(kt, K_BITS, N_ITERS, True)
    qv = oracle.quantize_tiles(vt, V_BITS, N_ITERS, False)
    oracle.dequantize_tiles(qk["codes"], qk["meta"], HEAD_DIM, K_BITS, True)
    oracle.dequantize_tiles(qv["codes"], qv["meta"], HEAD_DIM, V_BITS, False)
    oracle.decode_attention(qh, qk["codes"], qv["codes"], qk["meta"], qv["meta"],
                            n_kv_heads=KV_HEADS, tiles_per_seq=tiles_per_seq,
                            k_bits=K_BITS, v_bits=V_BITS)
    dt = time.perf_counter() - t0
    fp16_bytes = 3 * n_tiles * per_tile_bytes(HEAD_DIM)["fp16_pair"]
    return {"value": fp16_bytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": "%d of %d (layer, head) sequences (%d tile pairs): quantize + dequantize "
                      "+ decode attention of their %d query heads, fp64 oracle" % (
                          n_seq, LAYERS * KV_HEADS, n_tiles, n_layers * Q_HEADS)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seqs", type=int, default=128,
                    help="(layer, head) sequences in the CPU-oracle sample; 0 skips it")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs the KVarN path on one GPU only; "
              "--gpus %d is not supported (use --gpus 1)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_cache_bit_token_amd as kv
    from kv_cache_bit_token_amd import synthetic

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    k, v = synthetic.layered_kv_torch(2, LAYERS, KV_HEADS, TOKENS, HEAD_DIM, dev)
    kt = k.view(-1, 128, HEAD_DIM)
    vt = v.view(-1, 128, HEAD_DIM)
    n_tiles = kt.shape[0]
    tiles_per_seq = TOKENS // 128
    q = synthetic.query_torch(3, LAYERS, Q_HEADS, HEAD_DIM, dev)

    lay = kv.get_layout(HEAD_DIM, K_BITS, V_BITS, N_ITERS)
    kc = torch.empty((n_tiles, lay["k_code_bytes"]), dtype=torch.uint8, device=dev)
    vc = torch.empty((n_tiles, lay["v_code_bytes"]), dtype=torch.uint8, device=dev)
    km = torch.empty((n_tiles, lay["k_meta_bytes"] // 2), dtype=torch.float16, device=dev)
    vm = torch.empty((n_tiles, lay["v_meta_bytes"] // 2), dtype=torch.float16, device=dev)
    ko = torch.empty_like(kt)
    vo = torch.empty_like(vt)
    wsb = kv.decode_attention_workspace(batch=LAYERS, n_q_heads=Q_HEADS, n_kv_heads=KV_HEADS,
                                        tiles_per_seq=tiles_per_seq, head_dim=HEAD_DIM)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    out = torch.empty((LAYERS, Q_HEADS, HEAD_DIM), dtype=torch.float32, device=dev)

    def step(ev=None):
        if ev: ev[0].record()
        kv.quantize_tiles(kt, vt, k_bits=K_BITS, v_bits=V_BITS, n_iters=N_ITERS, out=(kc, vc, km, vm))
        if ev: ev[1].record()
        kv.dequantize_tiles(kc, vc, km, vm, head_dim=HEAD_DIM, k_bits=K_BITS, v_bits=V_BITS,
                            out=(ko, vo))
        if ev: ev[2].record()
        kv.decode_attention(q, kc, vc, km, vm, n_kv_heads=KV_HEADS, tiles_per_seq=tiles_per_seq,
                            k_bits=K_BITS, v_bits=V_BITS, workspace=ws, out=out)
        if ev: ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for s in range(args.steps):
        step(events[s])
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(end) / args.steps
    stage_ms = [sum(e[i].elapsed_time(e[i + 1]) for e in events) / args.steps for i in range(3)]

    b = per_tile_bytes(HEAD_DIM)
    fp16_total = n_tiles * b["fp16_pair"]              # 4.29 GB of fp16 K+V
    packed_total = n_tiles * b["packed_pair"]          # 0.91 GB packed
    q_bytes = LAYERS * Q_HEADS * HEAD_DIM * (2 + 4)
    hbm = {   # algorithmic HBM bytes of each stage
        "quantize": fp16_total + packed_total,
        "dequantize": packed_total + fp16_total,
        "decode_attention": packed_total + q_bytes,
    }
    stages = {}
    for name, ms in zip(("quantize", "dequantize", "decode_attention"), stage_ms):
        gbs = hbm[name] / (ms / 1e3)
        stages[name] = {"ms": round(ms, 4), "hbm_GBps": round(gbs / 1e9, 1),
                        "hbm_frac": round(gbs / HBM_PEAK, 4),
                        "fp16_equiv_GBps": round(fp16_total / (ms / 1e3) / 1e9, 1),
                        "tile_pairs_per_s": round(n_tiles / (ms / 1e3), 0)}
    dom = max(stages, key=lambda s: stages[s]["ms"])
    achieved = hbm[dom] / (stages[dom]["ms"] / 1e3)
    result = {
        "metric": "KV GB/s quantized/dequantized (fp16 in) and % of HBM peak, K4V2 g128",
        "value": round(3 * fp16_total / (ms_step / 1e3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "prefill-cache quantize + dequantize + decode attention, "
                               "64 layers x 8 KV heads x 16384 tokens x head_dim 128, K4V2 g128, "
                               "5 iterations, GQA 32/8",
                   "tiles": n_tiles, "kv_fp16_bytes": fp16_total, "packed_bytes": packed_total},
        "stages": stages,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved / 1e9, 1),
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK, 4), "traffic": None},
        "wall_s": round(t_wall, 3),
    }
    if args.cpu_seqs > 0:
        result["cpu_baseline"] = cpu_baseline(k, v, q, args.cpu_seqs)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
