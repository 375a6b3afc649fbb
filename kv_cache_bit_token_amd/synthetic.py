"""Seeded synthetic K/V inputs shaped like the pages' workloads.

This module only draws random numbers and shapes them (outlier channels,
outlier tokens, per-token magnitude); it holds none of the quantiser's
arithmetic.  Both the GPU path's tests and the oracle's tests take their
inputs from here.

Workload shapes follow the KV-cache arithmetic of the deep-dive page
("KV cache 為什麼能壓到 4-bit／2-bit ...", section on where the memory of a
16K-context request goes): 64 layers, 8 KV heads after GQA, head_dim 128,
fp16, 16384 tokens.  The pages' own measurements used a real model and
dataset (Qwen3-32B, AIME25) that are not available here; these seeded draws
stand in for real activations, with the structure the pages describe:
a few channels much larger than the rest, and tokens of very different
magnitude.

Recipes (K is drawn before V in every recipe):
  outlier_kv_host   numpy PCG64 (default_rng(seed)), float32 N(0,1); per head
                    and tensor, `n_ch` channels x`ch_mult`, then
                    round(tok_frac * tokens) tokens x`tok_mult`; clip to
                    +-30000; cast to fp16 (round to nearest even).
  outlier_kv_torch  the same recipe drawn with torch's generator on any
                    device (used for the multi-GB shapes).
  layered_kv_torch  per layer and tensor: n = round(U(0.01, 0.03) * D0)
                    outlier channels with multipliers U(20, 60), shared by the
                    layer's heads and all tokens; then every (layer, head,
                    token) row scaled by lognormal(0, 1); clip; fp16.
"""
import numpy as np

CLIP = 30000.0


def outlier_kv_host(seed, n_heads, n_tokens, d0, n_ch=4, ch_mult=50.0,
                    tok_frac=0.02, tok_mult=10.0):
    """Returns (K, V), each numpy float16 [n_heads][n_tokens][d0]."""
    rng = np.random.default_rng(seed)
    n_tok = int(round(tok_frac * n_tokens))
    outs = []
    for _tensor in range(2):
        x = rng.standard_normal((n_heads, n_tokens, d0), dtype=np.float32)
        for h in range(n_heads):
            ch = rng.choice(d0, n_ch, replace=False)
            x[h][:, ch] *= np.float32(ch_mult)
            tk = rng.choice(n_tokens, n_tok, replace=False)
            x[h][tk, :] *= np.float32(tok_mult)
        np.clip(x, -CLIP, CLIP, out=x)
        outs.append(x.astype(np.float16))
    return outs[0], outs[1]


def _torch():
    import torch
    return torch


def outlier_kv_torch(seed, n_heads, n_tokens, d0, device, n_ch=4, ch_mult=50.0,
                     tok_frac=0.02, tok_mult=10.0, chunk_heads=256):
    """Same recipe as outlier_kv_host, drawn with torch on `device`.

    Returns (K, V) torch.float16 [n_heads][n_tokens][d0].  Heads are drawn in
    chunks so the float32 staging stays small.
    """
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    n_tok = int(round(tok_frac * n_tokens))
    outs = []
    for _tensor in range(2):
        out = torch.empty((n_heads, n_tokens, d0), dtype=torch.float16, device=device)
        for h0 in range(0, n_heads, chunk_heads):
            h1 = min(n_heads, h0 + chunk_heads)
            nh = h1 - h0
            x = torch.randn((nh, n_tokens, d0), generator=g, device=device, dtype=torch.float32)
            ch = torch.rand((nh, d0), generator=g, device=device).argsort(dim=1)[:, :n_ch]
            cm = torch.ones((nh, d0), device=device)
            cm.scatter_(1, ch, ch_mult)
            tk = torch.rand((nh, n_tokens), generator=g, device=device).argsort(dim=1)[:, :n_tok]
            tm = torch.ones((nh, n_tokens), device=device)
            tm.scatter_(1, tk, tok_mult)
            x.mul_(cm[:, None, :]).mul_(tm[:, :, None]).clamp_(-CLIP, CLIP)
            out[h0:h1] = x.to(torch.float16)
            del x
        outs.append(out)
    return outs[0], outs[1]


def layered_kv_torch(seed, n_layers, n_kv_heads, n_tokens, d0, device, chunk_layers=4):
    """Prefill-cache recipe: returns (K, V) torch.float16
    [n_layers * n_kv_heads][n_tokens][d0] (layer-major, then head)."""
    torch = _torch()
    rng = np.random.default_rng(seed)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    outs = []
    for _tensor in range(2):
        # per-layer outlier channels and multipliers (host, small)
        cm = np.ones((n_layers, d0), np.float32)
        for layer in range(n_layers):
            n = int(round(rng.uniform(0.01, 0.03) * d0))
            ch = rng.choice(d0, n, replace=False)
            cm[layer, ch] = rng.uniform(20.0, 60.0, size=n).astype(np.float32)
        cm_t = torch.from_numpy(cm).to(device)
        out = torch.empty((n_layers * n_kv_heads, n_tokens, d0), dtype=torch.float16, device=device)
        for l0 in range(0, n_layers, chunk_layers):
            l1 = min(n_layers, l0 + chunk_layers)
            nl = l1 - l0
            x = torch.randn((nl, n_kv_heads, n_tokens, d0), generator=g, device=device,
                            dtype=torch.float32)
            mag = torch.empty((nl, n_kv_heads, n_tokens), device=device).log_normal_(
                0.0, 1.0, generator=g)
            x.mul_(cm_t[l0:l1, None, None, :]).mul_(mag[..., None]).clamp_(-CLIP, CLIP)
            out[l0 * n_kv_heads:l1 * n_kv_heads] = x.reshape(nl * n_kv_heads, n_tokens, d0).to(
                torch.float16)
            del x, mag
        outs.append(out)
    return outs[0], outs[1]


def query_torch(seed, batch, n_q_heads, d0, device):
    """Decode queries ~N(0, 1), torch.float16 [batch][n_q_heads][d0]."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn((batch, n_q_heads, d0), generator=g, device=device).to(torch.float16)


def query_host(seed, batch, n_q_heads, d0):
    """Decode queries ~N(0, 1), numpy float16 [batch][n_q_heads][d0]."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((batch, n_q_heads, d0), dtype=np.float32).astype(np.float16)


def as_tiles(x):
    """[heads][tokens][d0] -> [heads * tokens/128][128][d0] (a view)."""
    h, t, d0 = x.shape
    assert t % 128 == 0, "whole 128-token tiles only"
    return x.reshape(h * (t // 128), 128, d0)


class FeedbackSource:
    """Synthetic autoregressive token source for the error-accumulation probe.

    Token t's query, key and value rows are fixed random projections of a
    hidden vector x_t = unit-RMS(z_t + beta * unit-RMS(W_o . o_{t-1})), where z_t is
    fresh N(0, 1) noise drawn from a per-step stream (numpy PCG64 seeded with
    (seed, t), so every cache sees the same noise at step t) and o_{t-1} is
    the previous step's attention output of the cache being driven.  The
    feedback enters at a fixed share of the noise's energy (beta), so the
    stream stays a mix of fresh and carried-over content.  An error in one
    output therefore changes every later token, as in autoregressive
    decoding.  Keys and values carry the outlier-channel
    structure: K has n_ch channels with a large fixed offset of either sign
    (|offset| ~ U(20, 50), the same for every token, so it shifts every score
    of a query alike), V has n_ch channels scaled by U(20, 50); both rows
    carry a per-token magnitude exp(tok_sigma * N(0, 1)).  Holds none of the
    method's arithmetic.
    """

    def __init__(self, seed, d0, n_q_heads, beta=0.5, n_ch=4, ch_mult=(20.0, 50.0),
                 tok_sigma=0.5):
        rng = np.random.default_rng(seed)
        self.seed, self.d0, self.hq = int(seed), int(d0), int(n_q_heads)
        self.beta, self.tok_sigma = float(beta), float(tok_sigma)
        self.wo = rng.standard_normal((d0, n_q_heads * d0)) / np.sqrt(n_q_heads * d0)
        self.wk = rng.standard_normal((d0, d0)) / np.sqrt(d0)
        self.wv = rng.standard_normal((d0, d0)) / np.sqrt(d0)
        self.wq = rng.standard_normal((n_q_heads * d0, d0)) / np.sqrt(d0)
        self.bk = np.zeros(d0)
        self.bk[rng.choice(d0, n_ch, replace=False)] = (rng.uniform(*ch_mult, n_ch)
                                                       * rng.choice([-1.0, 1.0], n_ch))
        self.cv = np.ones(d0)
        self.cv[rng.choice(d0, n_ch, replace=False)] = rng.uniform(*ch_mult, n_ch)

    def token(self, t, o_prev=None):
        """-> (q [n_q_heads][d0], k [d0], v [d0]) numpy float16 for step t;
        o_prev: the previous attention output [n_q_heads][d0] (None at t = 0)."""
        rng = np.random.default_rng([self.seed, int(t)])
        x = rng.standard_normal(self.d0)
        mag = np.exp(self.tok_sigma * rng.standard_normal())
        if o_prev is not None:
            fb = self.wo @ np.asarray(o_prev, np.float64).reshape(-1)
            rms = np.sqrt(np.mean(fb * fb))
            if rms > 0:
                x = x + self.beta * fb / rms
        x = x / np.sqrt(np.mean(x * x))
        k = (self.wk @ x) * mag + self.bk
        v = (self.wv @ x) * self.cv * mag
        q = (self.wq @ x).reshape(self.hq, self.d0)
        return q.astype(np.float16), k.astype(np.float16), v.astype(np.float16)
