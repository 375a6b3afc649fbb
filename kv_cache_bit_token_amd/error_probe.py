"""Synthetic error-accumulation probe of the quantised cache.

Pages: digest page (ai-feeds.com), "方法" and the error-accumulation framing
of the title (quantisation error grows over long autoregressive decodes; the
attention output against full precision is the reconstruction proxy);
deep-dive page (vatt-ghern.pages.dev), the section on why naive 2-bit
quantisation loses accuracy over long decodes and its error-accumulation
widget.  No model or dataset is involved: the tokens come from
synthetic.FeedbackSource, whose next token depends on the previous attention
output, so an output error propagates into every later token.

Three caches are driven side by side on the GPU, one decode step at a time:
  fp16   the uncompressed cache (kvarn_decode_attention_fp16), the reference;
  kvarn  the paged KVarN cache: each full 128-token page quantised into a pool
         slot (kvarn_quantize_tiles_to), the unfilled page kept in fp16 and
         read as the tail (kvarn_decode_attention_paged);
  naive  per-token asymmetric round-to-nearest of the raw rows (no rotation,
         no normalisation), K and V at the same bit widths, stored
         dequantised and read like the fp16 cache.  This comparator runs as
         plain torch operations; it is not part of the KVarN path.
Each quantised cache runs twice: teacher-forced (fed the reference
trajectory's tokens: the per-step attention-output error) and free-running
(driven by its own outputs: the accumulated divergence).  Errors are relative
L2 distances to the reference output of the same step.

    python -m kv_cache_bit_token_amd.error_probe --steps 2048
"""
import argparse
import json

import numpy as np
import torch

from . import api
from .synthetic import FeedbackSource

TILE = 128


class Fp16Cache:
    """One sequence, one KV head, rows appended one token at a time."""

    def __init__(self, max_tokens, d0, device):
        self.k = torch.zeros((1, 1, max_tokens, d0), dtype=torch.float16, device=device)
        self.v = torch.zeros_like(self.k)
        self.n = 0

    def append(self, k_row, v_row):
        self.k[0, 0, self.n] = k_row
        self.v[0, 0, self.n] = v_row
        self.n += 1

    def attend(self, q):
        return api.decode_attention_fp16(q, self.k[:, :, :self.n], self.v[:, :, :self.n])


def naive_rtn(x, bits):
    """Per-row asymmetric RTN of the raw values, dequantised (comparator)."""
    xf = x.float()
    mn, mx = xf.min(), xf.max()
    s = (mx - mn) / float((1 << bits) - 1)
    if float(s) == 0.0:
        return x
    return (torch.round((xf - mn) / s) * s + mn).to(torch.float16)


class NaiveRtnCache(Fp16Cache):
    def __init__(self, max_tokens, d0, device, k_bits, v_bits):
        super().__init__(max_tokens, d0, device)
        self.kb, self.vb = k_bits, v_bits

    def append(self, k_row, v_row):
        super().append(naive_rtn(k_row, self.kb), naive_rtn(v_row, self.vb))


class KvarnCache:
    """One sequence, one KV head: whole pages in a packed pool, the unfilled
    page in an fp16 tail, quantised into the next pool slot when it fills."""

    def __init__(self, max_tokens, d0, device, k_bits, v_bits, n_iters):
        blocks = max_tokens // TILE + 1
        lay = api.get_layout(d0, k_bits, v_bits, n_iters)
        self.kc = torch.zeros((blocks, lay["k_code_bytes"]), dtype=torch.uint8, device=device)
        self.vc = torch.zeros((blocks, lay["v_code_bytes"]), dtype=torch.uint8, device=device)
        self.km = torch.zeros((blocks, lay["k_meta_bytes"] // 2), dtype=torch.float16, device=device)
        self.vm = torch.zeros((blocks, lay["v_meta_bytes"] // 2), dtype=torch.float16, device=device)
        self.table = torch.arange(blocks, dtype=torch.int32, device=device).view(1, blocks)
        self.tk = torch.zeros((1, 1, TILE, d0), dtype=torch.float16, device=device)
        self.tv = torch.zeros_like(self.tk)
        self.nb_t = torch.zeros(1, dtype=torch.int32, device=device)
        self.tl_t = torch.zeros(1, dtype=torch.int32, device=device)
        self.slot = torch.zeros(1, dtype=torch.int64, device=device)
        self.nb, self.tl = 0, 0
        self.d0, self.bits = d0, (k_bits, v_bits, n_iters)

    def append(self, k_row, v_row):
        self.tk[0, 0, self.tl] = k_row
        self.tv[0, 0, self.tl] = v_row
        self.tl += 1
        if self.tl == TILE:
            self.slot.fill_(self.nb)
            kb, vb, it = self.bits
            api.quantize_tiles_to(self.tk.view(1, TILE, self.d0), self.tv.view(1, TILE, self.d0),
                                  self.slot, self.kc, self.vc, self.km, self.vm,
                                  k_bits=kb, v_bits=vb, n_iters=it)
            self.nb, self.tl = self.nb + 1, 0

    def attend(self, q):
        self.nb_t.fill_(self.nb)
        self.tl_t.fill_(self.tl)
        kb, vb, _ = self.bits
        return api.decode_attention_paged(q, self.kc, self.vc, self.km, self.vm, self.table,
                                          self.nb_t, self.tl_t, self.tk, self.tv, n_kv_heads=1,
                                          k_bits=kb, v_bits=vb)


def run_probe(steps=2048, head_dim=128, n_q_heads=4, seed=0, beta=0.5, k_bits=4, v_bits=2,
              n_iters=5, device="cuda", trace=None):
    """-> dict of per-step relative errors (numpy) for the four quantised runs.

    trace: an optional list that receives, per step, the reference
    trajectory's tokens (q, k, v as numpy float16), the fp16 reference output
    and the teacher-forced KVarN output (numpy float32), so that another
    implementation can replay the same teacher-forced stream."""
    dev = torch.device(device)
    src = FeedbackSource(seed, head_dim, n_q_heads, beta=beta)
    ref = Fp16Cache(steps, head_dim, dev)
    runs = {
        "kvarn_forced": KvarnCache(steps, head_dim, dev, k_bits, v_bits, n_iters),
        "naive_forced": NaiveRtnCache(steps, head_dim, dev, k_bits, v_bits),
        "kvarn_free": KvarnCache(steps, head_dim, dev, k_bits, v_bits, n_iters),
        "naive_free": NaiveRtnCache(steps, head_dim, dev, k_bits, v_bits),
    }
    err = {name: np.zeros(steps) for name in runs}
    o_prev = {"ref": None, "kvarn_free": None, "naive_free": None}
    up = lambda a: torch.from_numpy(a).to(dev)   # noqa: E731
    for t in range(steps):
        q, k, v = (up(a) for a in src.token(t, o_prev["ref"]))
        ref.append(k, v)
        o_ref = ref.attend(q[None])[0]
        outs = {}
        for name in ("kvarn_forced", "naive_forced"):
            runs[name].append(k, v)
            outs[name] = runs[name].attend(q[None])[0]
        for name in ("kvarn_free", "naive_free"):
            qf, kf, vf = (up(a) for a in src.token(t, o_prev[name]))
            runs[name].append(kf, vf)
            outs[name] = runs[name].attend(qf[None])[0]
            o_prev[name] = outs[name].cpu().numpy()
        if trace is not None:
            trace.append({"q": q.cpu().numpy(), "k": k.cpu().numpy(), "v": v.cpu().numpy(),
                          "ref": o_ref.cpu().numpy(), "kvarn": outs["kvarn_forced"].cpu().numpy()})
        nr = o_ref.norm()
        rel = torch.stack([(outs[n] - o_ref).norm() / nr for n in runs]).cpu().numpy()
        for i, n in enumerate(runs):
            err[n][t] = rel[i]
        o_prev["ref"] = o_ref.cpu().numpy()
    return err


def summarise(err, window=256):
    out = {}
    for name, e in err.items():
        w = min(window, len(e))
        out[name] = {"first": round(float(e[:w].mean()), 4), "last": round(float(e[-w:].mean()), 4),
                     "mean": round(float(e.mean()), 4), "max": round(float(e.max()), 4)}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--steps", type=int, default=2048)
    ap.add_argument("--head-dim", type=int, default=128)
    ap.add_argument("--q-heads", type=int, default=4)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--beta", type=float, default=0.5)
    ap.add_argument("--window", type=int, default=256)
    args = ap.parse_args()
    err = run_probe(steps=args.steps, head_dim=args.head_dim, n_q_heads=args.q_heads,
                    seed=args.seed, beta=args.beta)
    print(json.dumps({"steps": args.steps, "head_dim": args.head_dim, "q_heads": args.q_heads,
                      "seed": args.seed, "beta": args.beta, "window": args.window,
                      "relative_l2_vs_fp16": summarise(err, args.window)}), flush=True)


if __name__ == "__main__":
    main()
