"""The error-accumulation probe's caches on the oracle (test helpers).

The same caches as kv_cache_bit_token_amd.error_probe, built from the
oracle's quantiser and attention: an fp16 cache, a naive per-token RTN cache
and the paged KVarN cache (whole pages quantised, the unfilled page read as
its fp16 tail).  One sequence, one KV head.
"""
import numpy as np

import oracle

D0, HQ = 128, 4


def _naive(x, bits):
    x = x.astype(np.float64)
    mn, mx = x.min(), x.max()
    s = (mx - mn) / ((1 << bits) - 1)
    return x.astype(np.float16) if s == 0 else (np.rint((x - mn) / s) * s + mn).astype(np.float16)


class _Fp16:
    def __init__(self, steps, bits=None):
        self.k = np.zeros((1, 1, steps, D0), np.float16)
        self.v = self.k.copy()
        self.n, self.bits = 0, bits

    def append(self, k, v):
        if self.bits:
            k, v = _naive(k, self.bits[0]), _naive(v, self.bits[1])
        self.k[0, 0, self.n], self.v[0, 0, self.n] = k, v
        self.n += 1

    def attend(self, q):
        return oracle.decode_attention_fp16(q[None], self.k[:, :, :self.n], self.v[:, :, :self.n])[0]


class _Kvarn:
    def __init__(self):
        self.tk = np.zeros((1, 1, 128, D0), np.float16)
        self.tv = self.tk.copy()
        self.tl = 0
        self.pages = []

    def append(self, k, v):
        self.tk[0, 0, self.tl], self.tv[0, 0, self.tl] = k, v
        self.tl += 1
        if self.tl == 128:
            qk = oracle.quantize_tiles(self.tk[0].copy(), 4, 5, True)
            qv = oracle.quantize_tiles(self.tv[0].copy(), 2, 5, False)
            self.pages.append((qk["codes"][0], qv["codes"][0], qk["meta"][0], qv["meta"][0]))
            self.tl = 0

    def attend(self, q):
        nb = len(self.pages)
        if nb:
            kc, vc, km, vm = (np.stack(x) for x in zip(*self.pages))
        else:
            kc = vc = np.zeros((1, 1), np.uint8)
            km = vm = np.zeros((1, 1), np.float16)
        table = np.arange(max(nb, 1), dtype=np.int32)[None]
        return oracle.decode_attention_paged(q[None], kc, vc, km, vm, table,
                                             np.array([nb], np.int32), np.array([self.tl], np.int32),
                                             self.tk, self.tv, n_kv_heads=1)[0]
