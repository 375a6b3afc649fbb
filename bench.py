"""Benchmark of the KVarN hot path on one MI355X.

Workload (the step): the prefill cache of a 64-layer, 8-KV-head,
head_dim-128 model at 16384 tokens (fp16 K and V of [64*8][16384][128],
about 4.3 GB), seeded synthetic values with per-layer outlier channels and
lognormal token magnitudes.  One step runs the whole hot path over it:
  1. kvarn_quantize_tiles   (K4V2, 128-token tiles, 5 normalisation iterations)
  2. kvarn_dequantize_tiles (back to fp16)
  3. kvarn_decode_attention (one decode query per layer: 32 query heads over
     the 8 KV heads, all 16384 cached tokens, GQA)
Inputs are resident in HBM before timing starts.  `value` is the metric as
named: fp16 K/V bytes quantised plus fp16 K/V bytes dequantised, per second
of quantise + dequantise kernel time (the attention stage reads the packed
cache and is reported beside it, not folded into `value`).  Per-stage times
come from HIP events recorded on the stream the kernels run on.

`roofline` covers the dominant kernel, the quantiser.  Its bound is the
vector ALU, not HBM: at 5 iterations the method needs about 40 fp32
operations per element (quant_ops_per_elem below) against a 2-byte input
element, far above the HBM balance point.  `achieved` is those algorithmic
operations per second over the kernel's HIP-event time, `peak` the issue
rate of fp32 multiply-adds: 256 CUs x 4 SIMDs x 2.4 GHz x 32 lanes, because
each SIMD can issue two wave64 fp32 FMA/MUL/ADD instructions from different
waves in one four-cycle slot (157.3 TFLOP/s counting a multiply-add as two;
packed two-wide fp32 instructions are not used).  `rooflines` holds one
entry per kernel and workload: the HBM fraction of every kernel (algorithmic
bytes per launch over its time, against 8 TB/s) and the quantisers' ALU
fraction.  `traffic` is a kernel's measured HBM bytes per launch (rocprofv3
FETCH_SIZE + WRITE_SIZE, scaled by a plain device-to-device copy of known
size), recorded for the kernel sources whose SHA-256 prefix is stored beside
it; it reads null once a source differs or where no counters were taken.

By default the other workloads run too, kernel by kernel (dequantize
256 x 8 x 8192, the head_dim sweep, attention 64 x 8 x 32768 and its fp16
baseline), each with its own roofline entries.

Prints one JSON line.  `--gpus` above 1 exits: the benchmark runs on one GPU.
`--copy-calibration` instead runs a plain 1 GiB device copy (the reference
for scaling the FETCH_SIZE / WRITE_SIZE counters) and exits.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
VALU_PEAK = 256 * 4 * 32 * 2.4e9   # fp32 multiply-add lane operations/s (CUs x SIMDs x dual-issued lanes x clock)
LAYERS, KV_HEADS, TOKENS, HEAD_DIM, Q_HEADS = 64, 8, 16384, 128, 32
K_BITS, V_BITS, N_ITERS = 4, 2, 5


def quant_ops_per_elem(D, n_iters):
    """Algorithmic fp32 operations per element of the quantiser (K and V mean).

    rotation log2(D) butterflies; each standard-deviation pass scales the
    element by the cross-axis factor, adds it and accumulates its square (3);
    K runs 2*n_iters passes, V 2*n_iters - 1 (its last row factor cancels in
    its per-token groups); the quantiser scales the element into its group,
    takes min and max, and applies the affine map and the rounding (5).
    """
    lg = D.bit_length() - 1
    k = lg + 3 * 2 * n_iters + 5
    v = lg + 3 * (2 * n_iters - 1) + 5
    return (k + v) / 2


# HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
# (FETCH_SIZE scaled by the copy calibration), keyed by (kernel, workload),
# each with the SHA-256 prefix of the kernel's sources it was taken for.
# decode_attention is its partial kernel, which merges the splits in the
# workgroup on these workloads; fp16_decode_attention sums its partial and
# combine kernels.
TRAFFIC = {
    ("quantize", "prefill"): {"source_sha256": "7fe5374b5ba8147d", "fetch_bytes": 4295693461,
                              "write_bytes": 905969664},
    ("dequantize", "prefill"): {"source_sha256": "c2af6ee1b9d5d2aa", "fetch_bytes": 909857119,
                                "write_bytes": 4295037888},
    ("decode_attention", "prefill"): {"source_sha256": "23ec0f4f7f57c67e", "fetch_bytes": 906740413,
                                      "write_bytes": 1048576},
    ("dequantize", "dequantize_256x8x8192"): {"source_sha256": "c2af6ee1b9d5d2aa", "fetch_bytes": 1821906301,
                                              "write_bytes": 8590013440},
    ("quantize", "head_dim_64_iters_3"): {"source_sha256": "7fe5374b5ba8147d", "fetch_bytes": 67459352,
                                          "write_bytes": 14942208},
    ("dequantize", "head_dim_64_iters_3"): {"source_sha256": "c2af6ee1b9d5d2aa", "fetch_bytes": 15133818,
                                            "write_bytes": 67109056},
    ("quantize", "head_dim_64_iters_5"): {"source_sha256": "7fe5374b5ba8147d", "fetch_bytes": 67458840,
                                          "write_bytes": 14942208},
    ("dequantize", "head_dim_64_iters_5"): {"source_sha256": "c2af6ee1b9d5d2aa", "fetch_bytes": 15132794,
                                            "write_bytes": 67108864},
    ("quantize", "head_dim_96_iters_3"): {"source_sha256": "7fe5374b5ba8147d", "fetch_bytes": 101040425,
                                          "write_bytes": 28311552},
    ("dequantize", "head_dim_96_iters_3"): {"source_sha256": "c2af6ee1b9d5d2aa", "fetch_bytes": 28597542,
                                            "write_bytes": 100663296},
    ("quantize", "head_dim_96_iters_5"): {"source_sha256": "7fe5374b5ba8147d", "fetch_bytes": 101040297,
                                          "write_bytes": 28311552},
    ("dequantize", "head_dim_96_iters_5"): {"source_sha256": "c2af6ee1b9d5d2aa", "fetch_bytes": 28597414,
                                            "write_bytes": 100663296},
    ("quantize", "head_dim_256_iters_3"): {"source_sha256": "7fe5374b5ba8147d", "fetch_bytes": 268855806,
                                           "write_bytes": 55050240},
    ("dequantize", "head_dim_256_iters_3"): {"source_sha256": "c2af6ee1b9d5d2aa", "fetch_bytes": 55287429,
                                             "write_bytes": 268435584},
    ("quantize", "head_dim_256_iters_5"): {"source_sha256": "7fe5374b5ba8147d", "fetch_bytes": 268855038,
                                           "write_bytes": 55050240},
    ("dequantize", "head_dim_256_iters_5"): {"source_sha256": "c2af6ee1b9d5d2aa", "fetch_bytes": 55286661,
                                             "write_bytes": 268436608},
    ("decode_attention", "decode_attention_64x8x32768"): {"source_sha256": "23ec0f4f7f57c67e", "fetch_bytes": 1812656019,
                                                          "write_bytes": 1048576},
    ("fp16_decode_attention", "prefill"): {"source_sha256": "0fde22ebbf659794", "fetch_bytes": 4560699399,
                                           "write_bytes": 1048576},
    ("fp16_decode_attention", "decode_attention_64x8x32768"): {"source_sha256": "0fde22ebbf659794", "fetch_bytes": 9142235549,
                                                               "write_bytes": 1048576},
}
_CSRC = os.path.join(ROOT, "kv_cache_bit_token_amd", "csrc")
KERNEL_SOURCES = {
    "quantize": ("kvarn_quantize.hip", "kvarn_device.hpp", "kvarn_internal.hpp"),
    "dequantize": ("kvarn_dequantize.hip", "kvarn_device.hpp", "kvarn_internal.hpp"),
    "decode_attention": ("kvarn_attention.hip", "kvarn_device.hpp", "kvarn_rsrc.hpp", "kvarn_internal.hpp"),
    "fp16_decode_attention": ("kvarn_attention_fp16.hip", "kvarn_device.hpp", "kvarn_rsrc.hpp",
                              "kvarn_internal.hpp"),
}


def source_sha(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_sha(kernel):
    return source_sha([os.path.join(_CSRC, f) for f in KERNEL_SOURCES[kernel]])


def measured_traffic(kernel, workload):
    """Counter-measured HBM bytes per launch, or None when not taken for the
    current sources."""
    t = TRAFFIC.get((kernel, workload))
    if t is None or t["source_sha256"] != kernel_sha(kernel):
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def per_tile_bytes(D, k_bits=K_BITS, v_bits=V_BITS):
    """fp16 and packed bytes of one K+V tile pair, from the library's own
    layout query (host only)."""
    from kv_cache_bit_token_amd import api
    lay = api.get_layout(D, k_bits, v_bits, 0)
    packed = lay["k_code_bytes"] + lay["v_code_bytes"] + lay["k_meta_bytes"] + lay["v_meta_bytes"]
    return {"fp16_pair": 2 * 2 * 128 * D, "packed_pair": packed}


def hbm_roofline(kernel, workload, ms, algo_bytes, traffic=None):
    """HBM roofline entry of one kernel on one workload."""
    gbs = algo_bytes / (ms / 1e3)
    return {"kernel": kernel, "workload": workload, "bound": "hbm",
            "achieved": round(gbs / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK, 4), "traffic": traffic, "algorithmic_bytes": algo_bytes,
            "ms": round(ms, 4)}


def alu_roofline(workload, ms, D, n_iters, elems, traffic=None):
    """Vector-ALU roofline entry of the quantiser on one workload."""
    ops = quant_ops_per_elem(D, n_iters) * elems
    a = ops / (ms / 1e3)
    return {"kernel": "quantize", "workload": workload, "bound": "alu",
            "achieved": round(a / 1e12, 3), "peak": round(VALU_PEAK / 1e12, 3), "unit": "Top/s",
            "frac": round(a / VALU_PEAK, 4), "traffic": traffic,
            "ops_per_elem": quant_ops_per_elem(D, n_iters), "ms": round(ms, 4)}


def cpu_baseline(k, v, q, n_seq, chunk=32):
    """The oracle, untuned, on the first n_seq (layer, head) sequences, fed in
    chunks of `chunk` sequences (only the oracle calls are timed).  `value`
    is in the unit and sense of the bench's `value`: fp16 K+V bytes quantised
    plus dequantised per second of quantise + dequantise time; the oracle's
    decode attention over the same sequences is timed apart."""
    import oracle

    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    tiles_per_seq = TOKENS // 128
    kt_all = k.view(-1, 128, HEAD_DIM)
    vt_all = v.view(-1, 128, HEAD_DIM)
    dt = dt_att = 0.0
    for s0 in range(0, n_seq, chunk):
        s1 = min(n_seq, s0 + chunk)
        kt = kt_all[s0 * tiles_per_seq:s1 * tiles_per_seq].cpu().numpy()
        vt = vt_all[s0 * tiles_per_seq:s1 * tiles_per_seq].cpu().numpy()
        # the query heads of the (layer, head) sequences in this chunk
        layers = sorted({s // KV_HEADS for s in range(s0, s1)})
        t0 = time.perf_counter()
        qk = oracle.quantize_tiles(kt, K_BITS, N_ITERS, True)
        qv = oracle.quantize_tiles(vt, V_BITS, N_ITERS, False)
        oracle.dequantize_tiles(qk["codes"], qk["meta"], HEAD_DIM, K_BITS, True)
        oracle.dequantize_tiles(qv["codes"], qv["meta"], HEAD_DIM, V_BITS, False)
        dt += time.perf_counter() - t0
        for layer in layers:
            g0, g1 = max(s0, layer * KV_HEADS), min(s1, (layer + 1) * KV_HEADS)
            sl = slice((g0 - s0) * tiles_per_seq, (g1 - s0) * tiles_per_seq)
            g = (g0 % KV_HEADS, g1 - g0)
            qh = q[layer:layer + 1, g[0] * (Q_HEADS // KV_HEADS):(g[0] + g[1]) * (Q_HEADS // KV_HEADS)]
            qh = qh.cpu().numpy()
            t0 = time.perf_counter()
            oracle.decode_attention(qh, qk["codes"][sl], qv["codes"][sl], qk["meta"][sl], qv["meta"][sl],
                                    n_kv_heads=g[1], tiles_per_seq=tiles_per_seq,
                                    k_bits=K_BITS, v_bits=V_BITS)
            dt_att += time.perf_counter() - t0
        del qk, qv, kt, vt
    n_tiles = n_seq * tiles_per_seq
    fp16_bytes = 2 * n_tiles * per_tile_bytes(HEAD_DIM)["fp16_pair"]
    # one thread, on the first 512 tokens of the first (layer, head): quantise
    # and dequantise its 4 tile pairs
    oracle.set_threads(1)
    kt = kt_all[:4].cpu().numpy()
    vt = vt_all[:4].cpu().numpy()
    t0 = time.perf_counter()
    qk = oracle.quantize_tiles(kt, K_BITS, N_ITERS, True)
    qv = oracle.quantize_tiles(vt, V_BITS, N_ITERS, False)
    oracle.dequantize_tiles(qk["codes"], qk["meta"], HEAD_DIM, K_BITS, True)
    oracle.dequantize_tiles(qv["codes"], qv["meta"], HEAD_DIM, V_BITS, False)
    dt1 = time.perf_counter() - t0
    oracle.set_threads(threads)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(fp16_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 3), "cpu_model": model,
            "decode_attention_seconds": round(dt_att, 3),
            "single_thread": {"value": round(2 * 4 * per_tile_bytes(HEAD_DIM)["fp16_pair"] / dt1 / 1e9, 4),
                              "unit": "GB/s", "seconds": round(dt1, 4),
                              "sample": "first 512 tokens of the first (layer, head), 4 tile pairs"},
            "sample": "%d of %d (layer, head) sequences (%d tile pairs): quantize + dequantize, fp64 "
                      "oracle, same inputs and unit as value; decode attention of their query heads "
                      "timed apart" % (n_seq, LAYERS * KV_HEADS, n_tiles)}


def copy_calibration():
    """Plain device-to-device copy of exactly 1 GiB (read 1 GiB, write 1 GiB)."""
    import torch
    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def paged_attention_measure(kv, kc, vc, km, vm, q, reps=20):
    """Decode attention over the same packed cache laid out as a paged pool
    (shuffled physical blocks, one table row per layer) plus an fp16 tail of
    1-127 tokens per (layer, KV head); timed with HIP events, outside the
    step.  Bytes: the packed blocks, the tails' fp16 K and V, q and out."""
    import numpy as np
    import torch
    from kv_cache_bit_token_amd import synthetic
    from kv_cache_bit_token_amd.paged import paged_layout

    dev = q.device
    tps = TOKENS // 128
    table, nb, tl, pool = paged_layout(7, LAYERS, tps, pool_blocks=LAYERS * tps, full=True)
    # pool row p * KV_HEADS + g holds the tile (b * KV_HEADS + g) * tps + i of table[b][i] = p
    src = np.empty(pool * KV_HEADS, np.int64)
    for b in range(LAYERS):
        for i in range(tps):
            p = table[b, i]
            for g in range(KV_HEADS):
                src[p * KV_HEADS + g] = (b * KV_HEADS + g) * tps + i
    idx = torch.from_numpy(src).to(dev)
    pkc, pvc, pkm, pvm = (t.index_select(0, idx) for t in (kc, vc, km, vm))
    kt, vt = synthetic.outlier_kv_torch(8, LAYERS * KV_HEADS, 128, HEAD_DIM, dev)
    kt = kt.view(LAYERS, KV_HEADS, 128, HEAD_DIM)
    vt = vt.view(LAYERS, KV_HEADS, 128, HEAD_DIM)
    t_table = torch.from_numpy(table).to(dev)
    t_nb, t_tl = torch.from_numpy(nb).to(dev), torch.from_numpy(tl).to(dev)
    wsb = kv.decode_attention_paged_workspace(batch=LAYERS, n_q_heads=Q_HEADS, n_kv_heads=KV_HEADS,
                                              max_blocks=tps, head_dim=HEAD_DIM)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    out = torch.empty((LAYERS, Q_HEADS, HEAD_DIM), dtype=torch.float32, device=dev)

    def run():
        kv.decode_attention_paged(q, pkc, pvc, pkm, pvm, t_table, t_nb, t_tl, kt, vt,
                                  n_kv_heads=KV_HEADS, workspace=ws, out=out)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    b = per_tile_bytes(HEAD_DIM)
    packed = int(nb.sum()) * KV_HEADS * b["packed_pair"]
    tail = int(tl.sum()) * KV_HEADS * 2 * HEAD_DIM * 2
    nbytes = packed + tail + LAYERS * Q_HEADS * HEAD_DIM * (2 + 4)
    tokens = (int(nb.sum()) * 128 + int(tl.sum())) * KV_HEADS
    return {"ms": round(ms, 4), "hbm_GBps": round(nbytes / (ms / 1e3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms / 1e3) / HBM_PEAK, 4),
            "fp16_equiv_GBps": round(tokens * HEAD_DIM * 4 / (ms / 1e3) / 1e9, 1),
            "workload": "64 sequences x 8 KV heads x (128 shuffled pool blocks + 1-127 fp16 tail "
                        "tokens), GQA 32/8, K4V2; outside the timed step"}


def stream_reference(dev, units, reps=5):
    """Plain streaming kernels moving each stage's bytes per tile pair
    (libkvarn_streamref.so, built with the library): the rate this device
    delivers for that read/write mix, the reference for each stage's HBM
    fraction beside the nominal 8 TB/s.  Best over kernel layouts (a loop
    kernel; an unrolled one with plain or nontemporal stores; for the
    dequantize mix also phased kernels that read 4 or 8 units before writing
    them) and grid shapes: persistent grids of 4, 8 and 16 workgroups per CU,
    and grids with one workgroup per unit in address order, the unit a tile
    pair (64 KB of fp16) or 1/2, 1/4, 1/8, 1/16 or 1/32 of one.  `variants` keeps every layout's
    best rate and `grids` the grid shape it was reached with; `by_grid_GBps`
    the best rate of each grid shape over the layouts.  `fp16_write` is
    the dequantiser's output alone (write-only, the same 4.3 GB)."""
    import ctypes
    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "kv_cache_bit_token_amd", "libkvarn_streamref.so"))
    fn = lib.kvarn_stream_reference
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    b = per_tile_bytes(HEAD_DIM)
    big, small = b["fp16_pair"] // 16, b["packed_pair"] // 16
    src = torch.empty(units * big * 16, dtype=torch.uint8, device=dev)
    dst = torch.empty(units * big * 16, dtype=torch.uint8, device=dev)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    layouts = {0: "loop", 1: "unrolled", 2: "unrolled_nt", 3: "phased_4", 4: "phased_8"}
    mixes = {"quantize_mix": (big, small, (0, 1, 2)), "dequantize_mix": (small, big, (0, 1, 2, 3, 4)),
             "packed_read": (small, 0, (0, 1)), "fp16_read": (big, 0, (0, 1)),
             "fp16_write": (0, big, (1, 2))}
    out = {}
    for name, (rq, wq, kinds) in mixes.items():
        nbytes = units * (rq + wq) * 16
        # (label, units, rq, wq, workgroups)
        grids = [("%d_per_cu" % k, units, rq, wq, cus * k) for k in (4, 8, 16)]
        grids.append(("one_per_tile_pair", units, rq, wq, units))
        for div, label in ((2, "one_per_tile"), (4, "one_per_quarter_pair"), (8, "one_per_8th_pair"),
                           (16, "one_per_16th_pair"), (32, "one_per_32nd_pair")):
            grids.append((label, div * units, rq // div, wq // div, div * units))
        variants, shapes, by_grid = {}, {}, {}
        for unrolled in kinds:
            best = None
            for label, n, r, w, blocks in grids:
                if unrolled >= 3 and (r, w) != (rq, wq):
                    continue   # the phased kernels exist for the tile-pair unit only
                def run():
                    st = fn(src.data_ptr(), dst.data_ptr(), n, r, w, blocks, unrolled,
                            sink.data_ptr(), stream)
                    if st != 0:
                        raise RuntimeError("stream reference launch failed: %d" % st)
                for _ in range(2):
                    run()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    run()
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / reps
                rate = round(nbytes / (ms / 1e3) / 1e9, 1)
                by_grid[label] = max(by_grid.get(label, 0.0), rate)
                if best is None or ms < best[0]:
                    best = (ms, label)
            variants[layouts[unrolled]] = round(nbytes / (best[0] / 1e3) / 1e9, 1)
            shapes[layouts[unrolled]] = best[1]
        top = max(variants, key=variants.get)
        gbs = variants[top]
        out[name] = {"ms": round(nbytes / (gbs * 1e9) * 1e3, 4), "GBps": gbs,
                     "frac_of_peak": round(gbs * 1e9 / HBM_PEAK, 4), "best_layout": top,
                     "best_grid": shapes[top], "variants_GBps": variants, "grids": shapes,
                     "by_grid_GBps": by_grid}
    del src, dst
    torch.cuda.empty_cache()
    return out


def _alu_lib():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "kv_cache_bit_token_amd", "libkvarn_streamref.so"))
    lib.kvarn_valu_reference.restype = ctypes.c_int
    lib.kvarn_valu_reference.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_void_p]
    lib.kvarn_valu_class_reference.restype = ctypes.c_int
    lib.kvarn_valu_class_reference.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_void_p]
    lib.kvarn_valu_class_count.restype = ctypes.c_int
    lib.kvarn_valu_class_name.restype = ctypes.c_char_p
    lib.kvarn_valu_class_name.argtypes = [ctypes.c_int32]
    return lib


def _best_ms(launch, reps):
    import torch
    best = None
    for _ in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        st = launch()
        e1.record()
        torch.cuda.synchronize()
        if st != 0:
            raise RuntimeError("ALU reference launch failed: %d" % st)
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    return best


def alu_reference(dev, iters=4096, reps=3):
    """Plain fp32 multiply-add chains (libkvarn_streamref.so): the rate the
    device sustains for the cheapest VALU instructions at 4 waves per SIMD
    (the quantiser's occupancy) and at 8, in lane operations per second, and
    the engine clock it ran at (shader-clock over 100 MHz wall-clock ticks)."""
    import ctypes
    import torch

    lib = _alu_lib()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    out = {}
    for waves in (4, 8):
        blocks = cus * waves          # 256-thread workgroups: one wave per SIMD each
        buf = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
        ticks = torch.zeros(blocks * 4 * 2, dtype=torch.int64, device=dev)
        best = _best_ms(lambda: lib.kvarn_valu_reference(buf.data_ptr(), ticks.data_ptr(), blocks,
                                                         iters, stream), reps)
        ops = blocks * 256 * iters * 16
        out["fma_%d_waves_per_simd_Tops" % waves] = round(ops / (best / 1e3) / 1e12, 2)
        t = ticks.view(-1, 2).double()
        out["clock_MHz_%d_waves" % waves] = round(float((t[:, 0] / t[:, 1]).mean()) * 100.0, 0)
        del buf, ticks
    return out


def alu_classes(dev, iters=2048, reps=2):
    """Issue rate of single VALU instruction classes (16 per loop trip, eight
    independent registers) at 4 and 8 waves per SIMD: lane operations per
    second and cycles per wave instruction per SIMD at the measured clock."""
    import ctypes
    import torch

    lib = _alu_lib()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    clk = alu_reference(dev)
    out = {"clock": clk}
    for cls in range(lib.kvarn_valu_class_count()):
        name = lib.kvarn_valu_class_name(cls).decode()
        row = {}
        for waves in (4, 8):
            blocks = cus * waves
            buf = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
            best = _best_ms(lambda: lib.kvarn_valu_class_reference(cls, buf.data_ptr(), blocks,
                                                                   iters, stream), reps)
            instr = blocks * 4 * iters * 16             # wave instructions
            mhz = clk["clock_MHz_%d_waves" % waves]
            row["%d_waves_Tops" % waves] = round(instr * 64 / (best / 1e3) / 1e12, 2)
            row["%d_waves_cycles_per_instr" % waves] = round(
                best / 1e3 * mhz * 1e6 / (instr / (cus * 4)), 2)
            del buf
        out[name] = row
    return out


def fp16_attention_measure(kv, k, v, q, packed_out, packed_ms, reps=20):
    """Decode attention over the uncompressed fp16 cache of the same workload
    (the baseline of the pages' throughput comparison), timed with HIP events
    outside the step.  Bytes: the fp16 K and V, q and out.  Also reports the
    packed path's speed-up over it and the relative L2 distance between the
    two attention outputs."""
    import torch

    kk = k.view(LAYERS, KV_HEADS, TOKENS, HEAD_DIM)
    vv = v.view(LAYERS, KV_HEADS, TOKENS, HEAD_DIM)
    wsb = kv.decode_attention_fp16_workspace(batch=LAYERS, n_q_heads=Q_HEADS, n_kv_heads=KV_HEADS,
                                             seq_len=TOKENS, head_dim=HEAD_DIM)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=q.device)
    out = torch.empty((LAYERS, Q_HEADS, HEAD_DIM), dtype=torch.float32, device=q.device)

    def run():
        kv.decode_attention_fp16(q, kk, vv, workspace=ws, out=out)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = 2 * k.numel() * 2 + LAYERS * Q_HEADS * HEAD_DIM * (2 + 4)
    rel = float((packed_out - out).norm() / out.norm())
    return {"ms": round(ms, 4), "hbm_GBps": round(nbytes / (ms / 1e3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms / 1e3) / HBM_PEAK, 4), "bytes": nbytes,
            "packed_speedup": round(ms / packed_ms, 3),
            "packed_rel_l2": round(rel, 6),
            "workload": "same 64 x 8 x 16384 x 128 cache and queries, uncompressed fp16; "
                        "outside the timed step"}


def config_sweep(kv, synthetic, dev, rooflines, reps=10):
    """The other workloads, timed kernel by kernel with HIP events (inputs
    resident; small working sets rotated across copies totalling > 512 MB so
    the 256 MB last-level cache cannot hold them):
      dequantize         256 seq x 8 KV heads x 8192 tokens x 128 (packed by the quantiser)
      head_dim sweep     8 KV heads x 32768 tokens, head_dim 64 / 96 / 256, 3 and 5 iterations
      decode attention   64 seq x 8 KV heads x 32768 tokens, GQA 32/8, and its fp16 baseline
    Appends one roofline entry per kernel and workload to `rooflines`."""
    import torch

    def timed(fns):
        for f in fns[:2]:
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fns[i % len(fns)]()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def rates(ms, fp16_bytes, hbm_bytes, pairs):
        return {"ms": round(ms, 4), "fp16_equiv_GBps": round(fp16_bytes / (ms / 1e3) / 1e9, 1),
                "hbm_GBps": round(hbm_bytes / (ms / 1e3) / 1e9, 1),
                "hbm_frac": round(hbm_bytes / (ms / 1e3) / HBM_PEAK, 4),
                "tile_pairs_per_s": round(pairs / (ms / 1e3), 0)}

    out = {}
    # dequantize, 256 x 8 x 8192
    wl = "dequantize_256x8x8192"
    k, v = synthetic.outlier_kv_torch(1, 256 * 8, 8192, 128, dev)
    kt, vt = k.view(-1, 128, 128), v.view(-1, 128, 128)
    packed = kv.quantize_tiles(kt, vt)
    n = kt.shape[0]
    b = per_tile_bytes(128)
    ms = timed([lambda: kv.dequantize_tiles(*packed, head_dim=128, out=(kt, vt))])
    hbm = n * (b["fp16_pair"] + b["packed_pair"])
    out[wl] = rates(ms, n * b["fp16_pair"], hbm, n)
    rooflines.append(hbm_roofline("dequantize", wl, ms, hbm, measured_traffic("dequantize", wl)))
    del k, v, kt, vt, packed
    torch.cuda.empty_cache()
    # head_dim sweep
    for d0 in (64, 96, 256):
        D = 64 if d0 <= 64 else (128 if d0 <= 128 else 256)
        k, v = synthetic.outlier_kv_torch(4, 8, 32768, d0, dev)
        kt, vt = k.view(-1, 128, d0), v.view(-1, 128, d0)
        n = kt.shape[0]
        fp16 = 2 * n * 128 * d0 * 2
        copies = max(2, -(-(512 << 20) // fp16) + 1)
        ins = [(kt.clone(), vt.clone()) for _ in range(copies)]
        lay = kv.get_layout(d0, 4, 2, 5)
        packed_b = n * (lay["k_code_bytes"] + lay["v_code_bytes"] + lay["k_meta_bytes"] + lay["v_meta_bytes"])
        for it in (3, 5):
            outs = [kv.quantize_tiles(a, c, n_iters=it) for a, c in ins]
            ms_q = timed([lambda a=a, c=c, o=o: kv.quantize_tiles(a, c, n_iters=it, out=o)
                          for (a, c), o in zip(ins, outs)])
            ms_d = timed([lambda a=a, c=c, o=o: kv.dequantize_tiles(*o, head_dim=d0, out=(a, c))
                          for (a, c), o in zip(ins, outs)])
            key = "head_dim_%d_iters_%d" % (d0, it)
            out[key] = {"padded": D, "quantize": rates(ms_q, fp16, fp16 + packed_b, n),
                        "dequantize": rates(ms_d, fp16, fp16 + packed_b, n)}
            rooflines.append(hbm_roofline("quantize", key, ms_q, fp16 + packed_b,
                                          measured_traffic("quantize", key)))
            rooflines.append(alu_roofline(key, ms_q, D, it, 2 * n * 128 * D,
                                          measured_traffic("quantize", key)))
            rooflines.append(hbm_roofline("dequantize", key, ms_d, fp16 + packed_b,
                                          measured_traffic("dequantize", key)))
            del outs
        del k, v, kt, vt, ins
        torch.cuda.empty_cache()
    # decode attention, 64 x 8 x 32768, and the fp16 baseline
    wl = "decode_attention_64x8x32768"
    k, v = synthetic.outlier_kv_torch(5, 64 * 8, 32768, 128, dev)
    kt, vt = k.view(-1, 128, 128), v.view(-1, 128, 128)
    kc, vc, km, vm = kv.quantize_tiles(kt, vt)
    q = synthetic.query_torch(5, 64, 32, 128, dev)
    n = kt.shape[0]
    wsb = kv.decode_attention_workspace(batch=64, n_q_heads=32, n_kv_heads=8, tiles_per_seq=256,
                                        head_dim=128)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    o = torch.empty((64, 32, 128), dtype=torch.float32, device=dev)
    ms = timed([lambda: kv.decode_attention(q, kc, vc, km, vm, n_kv_heads=8, tiles_per_seq=256,
                                            workspace=ws, out=o)])
    qb = 64 * 32 * 128 * (2 + 4)
    out[wl] = rates(ms, n * b["fp16_pair"], n * b["packed_pair"] + qb, n)
    rooflines.append(hbm_roofline("decode_attention", wl, ms, n * b["packed_pair"] + qb,
                                  measured_traffic("decode_attention", wl)))
    k4, v4 = k.view(64, 8, 32768, 128), v.view(64, 8, 32768, 128)
    wsf = torch.empty(max(kv.decode_attention_fp16_workspace(batch=64, n_q_heads=32, n_kv_heads=8,
                                                             seq_len=32768, head_dim=128), 16),
                      dtype=torch.uint8, device=dev)
    ms_f = timed([lambda: kv.decode_attention_fp16(q, k4, v4, workspace=wsf, out=o)])
    out["fp16_" + wl] = rates(ms_f, n * b["fp16_pair"], n * b["fp16_pair"] + qb, n)
    out["fp16_" + wl]["packed_speedup"] = round(ms_f / ms, 3)
    rooflines.append(hbm_roofline("fp16_decode_attention", wl, ms_f, n * b["fp16_pair"] + qb,
                                  measured_traffic("fp16_decode_attention", wl)))
    del k, v, kt, vt, kc, vc, km, vm, k4, v4
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seqs", type=int, default=LAYERS * KV_HEADS,
                    help="(layer, head) sequences in the CPU-oracle sample; 0 skips it")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the paged-cache decode-attention measurement")
    ap.add_argument("--no-fp16", action="store_true",
                    help="skip the fp16-cache decode-attention baseline")
    ap.add_argument("--no-stream-ref", action="store_true",
                    help="skip the streaming reference kernels")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (dequantize 256x8x8192, head_dim sweep, "
                         "attention 64x8x32768), timed kernel by kernel after the step")
    ap.add_argument("--cold-stages", action="store_true",
                    help="fill the last-level cache with clean, unrelated lines before each stage of the "
                         "step (outside the stage timers, inside ms_per_step), so that no stage reads "
                         "what the previous one left cached")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--alu-classes", action="store_true",
                    help="run only the per-class VALU issue-rate kernels, print their JSON and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.alu_classes:
        import torch
        print(json.dumps(alu_classes(torch.device("cuda:0"))), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the KVarN path is benchmarked on one GPU only; "
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

    if args.cold_stages:
        # 1 GiB written (evicting and writing back whatever the 256 MB
        # last-level cache holds), then another 1 GiB read, so that each stage
        # starts with that cache full of clean lines of unrelated data
        junk = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
        clean = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        acc = torch.zeros(1, dtype=torch.float32, device=dev)

    def between_stages():
        if args.cold_stages:
            junk.add_(1.0)
            torch.sum(clean, dim=0, keepdim=True, out=acc)

    def step(ev=None):
        # ev: start and end of each stage (quantise, dequantise, attention)
        between_stages()
        if ev: ev[0].record()
        kv.quantize_tiles(kt, vt, k_bits=K_BITS, v_bits=V_BITS, n_iters=N_ITERS, out=(kc, vc, km, vm))
        if ev: ev[1].record()
        between_stages()
        if ev: ev[2].record()
        kv.dequantize_tiles(kc, vc, km, vm, head_dim=HEAD_DIM, k_bits=K_BITS, v_bits=V_BITS,
                            out=(ko, vo))
        if ev: ev[3].record()
        between_stages()
        if ev: ev[4].record()
        kv.decode_attention(q, kc, vc, km, vm, n_kv_heads=KV_HEADS, tiles_per_seq=tiles_per_seq,
                            k_bits=K_BITS, v_bits=V_BITS, workspace=ws, out=out)
        if ev: ev[5].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
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
    stage_ms = [sum(e[2 * i].elapsed_time(e[2 * i + 1]) for e in events) / args.steps for i in range(3)]

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
    for name in ("quantize", "dequantize"):
        stages[name]["meets_70pct_hbm_target"] = stages[name]["hbm_frac"] >= 0.70
    qd_ms = stage_ms[0] + stage_ms[1]
    wl = "prefill"
    elems = n_tiles * 2 * 128 * HEAD_DIM
    # the dominant kernel, the quantiser: vector-ALU bound
    roofline = alu_roofline(wl, stage_ms[0], HEAD_DIM, N_ITERS, elems,
                            measured_traffic("quantize", wl))
    roofline["hbm_frac"] = stages["quantize"]["hbm_frac"]
    roofline["algorithmic_hbm_bytes"] = hbm["quantize"]
    rooflines = [
        roofline,
        hbm_roofline("quantize", wl, stage_ms[0], hbm["quantize"], measured_traffic("quantize", wl)),
        hbm_roofline("dequantize", wl, stage_ms[1], hbm["dequantize"],
                     measured_traffic("dequantize", wl)),
        hbm_roofline("decode_attention", wl, stage_ms[2], hbm["decode_attention"],
                     measured_traffic("decode_attention", wl)),
    ]
    result = {
        "metric": "KV GB/s quantized/dequantized (fp16 in) and % of HBM peak, K4V2 g128",
        "value": round(2 * fp16_total / (qd_ms / 1e3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "prefill-cache quantize + dequantize + decode attention, "
                               "64 layers x 8 KV heads x 16384 tokens x head_dim 128, K4V2 g128, "
                               "5 iterations, GQA 32/8",
                   "value_counts": "fp16 K+V bytes quantised + dequantised per second of "
                                   "quantise + dequantise kernel time (attention reported apart)",
                   "hbm_frac_quantize_dequantize": round((hbm["quantize"] + hbm["dequantize"])
                                                         / (qd_ms / 1e3) / HBM_PEAK, 4),
                   "tiles": n_tiles, "kv_fp16_bytes": fp16_total, "packed_bytes": packed_total,
                   "cold_stages": bool(args.cold_stages)},
        "stages": stages,
        "roofline": roofline,
        "wall_s": round(t_wall, 3),
    }
    if not args.no_stream_ref:
        ref = stream_reference(dev, n_tiles)
        result["stream_reference"] = ref
        alu = alu_reference(dev)
        roofline["alu_reference"] = alu
        roofline["frac_of_alu_reference"] = round(
            roofline["achieved"] / alu["fma_4_waves_per_simd_Tops"], 4)
        for stage, mix in (("quantize", "quantize_mix"), ("dequantize", "dequantize_mix"),
                           ("decode_attention", "packed_read")):
            stages[stage]["achievable_frac"] = round(stages[stage]["hbm_GBps"] / ref[mix]["GBps"], 4)
    if not args.no_fp16:
        f = fp16_attention_measure(kv, k, v, q, out, stages["decode_attention"]["ms"])
        result["fp16_decode_attention"] = f
        rooflines.append(hbm_roofline("fp16_decode_attention", wl, f["ms"], f["bytes"],
                                      measured_traffic("fp16_decode_attention", wl)))
        if "stream_reference" in result:
            f["achievable_frac"] = round(f["hbm_GBps"] / result["stream_reference"]["fp16_read"]["GBps"], 4)
    if not args.no_paged:
        result["paged_decode_attention"] = paged_attention_measure(kv, kc, vc, km, vm, q)
    if not args.no_configs:
        del ko, vo
        torch.cuda.empty_cache()
        result["other_workloads"] = config_sweep(kv, synthetic, dev, rooflines)
    result["rooflines"] = rooflines
    if args.cpu_seqs > 0:
        result["cpu_baseline"] = cpu_baseline(k, v, q, args.cpu_seqs)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
