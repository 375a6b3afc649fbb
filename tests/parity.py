"""Parity rules between the HIP path and the oracle (shared by the GPU tests).

Codes: bit-exact, except codes off by exactly one where the oracle's own
value sits at a rounding boundary.  A mismatch is excused when the oracle's
fp64 u = (Y - z)/s lies within W = 1e-6 * max(1, |u|, (|Y| + |z|)/s) of a
half integer: the distance by which a relative perturbation of 1e-6 in the
quantities u is computed from (Y, z, s) can move u, i.e. 1e-6 times u's
relative condition number.  At most 1e-4 of the codes of a workload may be
excused.  Every comparison also reports the ratio under the narrower window
1e-6 * max(1, |u|) and how many codes fall outside it.

Scales (SK, RK, SV, CV): |a - b| <= 1e-3 |b|.  Zero points (ZK, ZV):
|a - b| <= 1e-3 max(|b|, the group's stored scale).
Dequantised values: |a - b| <= 1e-3 (|b| + rms of b's token row).
Attention outputs, per query head: max |a - b| <= 2e-3 + A, where A = 0
unless the head's error exceeds 2e-3; then A = 16 * 2^-24 * kappa with
kappa = sum_t p_t * sm_scale * |q| |k_t| * max_j |v_tj - o_j| (p, o the
oracle's probabilities and output; K, V the oracle's dequantised cache).
kappa bounds the first-order change of o when every score's dot product
carries an absolute error of one fp32 unit of its terms' magnitude
(sm_scale |q| |k_t| by Cauchy-Schwarz, in any orthonormal basis, so for
the rotated-domain kernel too); 16 units cover the score's roundings (the
fixed-point rounding of the query-side operand to 27 bits per head and
tile, the join of the exact integer limb sums, the scale products).  Where two tokens of very different value nearly tie for the
largest score, fp32 scores alone move o by more than 2e-3
(tests/test_oracle_dequant_attention.py shows it on the decode-attention
workload), so an fp32 kernel cannot meet a bare 2e-3 there.  The number of
heads that use the allowance is reported.

Every comparison appends its statistics to REPORT, which tests/conftest.py
prints in the terminal summary, so the figures survive a quiet (-q) run.
"""
import numpy as np

import oracle

CODE_WINDOW = 1e-6
CODE_MAX_FRACTION = 1e-4

REPORT = []


def record(label, stats):
    REPORT.append((label, stats))
    return stats


def unpack_all(codes, D, bits, is_key):
    return np.stack([oracle.unpack(c, D, bits, is_key) for c in codes])


def _excuse(g, o, q, bits, is_key):
    """Window statistics of the code mismatches of some tiles (q: the oracle's
    diagnostics of those tiles).  Returns (mismatch, unexcused, worst ratio,
    outside the narrow window, worst narrow ratio)."""
    bad = g != o
    if not bad.any():
        return 0, 0, 0.0, 0, 0.0
    diff = np.abs(g.astype(np.int64) - o.astype(np.int64))[bad]
    assert diff.max() == 1, "code off by %d" % diff.max()
    y, u = q["y"], q["u"]
    if is_key:
        z = np.broadcast_to(q["z"][:, None, :], y.shape)
        sc = np.broadcast_to(q["s"][:, None, :], y.shape)
    else:
        z = np.broadcast_to(q["z"][:, :, None], y.shape)
        sc = np.broadcast_to(q["s"][:, :, None], y.shape)
    ub, yb, zb, sb = u[bad], y[bad], z[bad], sc[bad]
    cond = np.where(sb > 0, (np.abs(yb) + np.abs(zb)) / np.where(sb > 0, sb, 1.0), 0.0)
    dist = np.abs(ub - np.floor(ub) - 0.5)
    narrow = dist / (CODE_WINDOW * np.maximum(1.0, np.abs(ub)))
    ratio = dist / (CODE_WINDOW * np.maximum(np.maximum(1.0, np.abs(ub)), cond))
    return (int(bad.sum()), int((ratio > 1.0).sum()), float(ratio.max()),
            int((narrow > 1.0).sum()), float(narrow.max()))


def compare_codes(gpu_codes, q, D, bits, is_key):
    """gpu_codes: [n][code_bytes] uint8; q: oracle.quantize_tiles(..., diag=True).

    Returns a dict of statistics; raises AssertionError on a violation."""
    g = unpack_all(gpu_codes, D, bits, is_key)
    o = unpack_all(q["codes"], D, bits, is_key)
    mis, unex, worst, out_n, worst_n = _excuse(g, o, q, bits, is_key)
    stats = {"codes": int(g.size), "mismatch": mis, "unexcused": unex, "worst_window_ratio": worst,
             "outside_narrow_window": out_n, "worst_narrow_ratio": worst_n}
    assert unex == 0, stats
    assert mis <= CODE_MAX_FRACTION * g.size, stats
    return stats


class CodeTally:
    """Code parity of a whole workload, tile chunk by tile chunk.

    Packed bytes are compared first; only tiles whose bytes differ are
    unpacked and run through the oracle again with diagnostics (u), so a
    multi-GB workload is checked on every code without holding the oracle's
    fp64 diagnostics of every tile."""

    def __init__(self, label):
        self.label = label
        self.codes = 0
        self.mismatch = 0
        self.unexcused = 0
        self.worst = 0.0
        self.outside_narrow = 0
        self.worst_narrow = 0.0
        self.tiles_differing = 0

    def add(self, gpu_codes, oracle_codes, x16, bits, n_iters, is_key):
        """gpu_codes, oracle_codes: [n][code_bytes] uint8 of the same tiles;
        x16: those tiles' fp16 input [n][128][d0] (host)."""
        gpu_codes = np.asarray(gpu_codes)
        oracle_codes = np.asarray(oracle_codes)
        D = oracle.padded_dim(x16.shape[-1])
        self.codes += gpu_codes.shape[0] * 128 * D
        diff = np.nonzero((gpu_codes != oracle_codes).any(axis=1))[0]
        if diff.size == 0:
            return
        self.tiles_differing += int(diff.size)
        q = oracle.quantize_tiles(np.ascontiguousarray(x16[diff]), bits, n_iters, is_key, diag=True)
        assert np.array_equal(q["codes"], oracle_codes[diff]), "oracle is not deterministic"
        g = unpack_all(gpu_codes[diff], D, bits, is_key)
        o = unpack_all(oracle_codes[diff], D, bits, is_key)
        mis, unex, worst, out_n, worst_n = _excuse(g, o, q, bits, is_key)
        self.mismatch += mis
        self.unexcused += unex
        self.worst = max(self.worst, worst)
        self.outside_narrow += out_n
        self.worst_narrow = max(self.worst_narrow, worst_n)

    def finish(self):
        stats = {"codes": self.codes, "mismatch": self.mismatch,
                 "mismatch_fraction": self.mismatch / max(self.codes, 1),
                 "unexcused": self.unexcused, "worst_window_ratio": self.worst,
                 "outside_narrow_window": self.outside_narrow,
                 "worst_narrow_ratio": self.worst_narrow,
                 "tiles_differing": self.tiles_differing}
        record(self.label, stats)
        assert self.unexcused == 0, stats
        assert self.mismatch <= CODE_MAX_FRACTION * self.codes, stats
        return stats


def compare_meta(gpu_meta, oracle_meta, D, is_key):
    g = np.asarray(gpu_meta, dtype=np.float16).astype(np.float64)
    o = np.asarray(oracle_meta, dtype=np.float16).astype(np.float64)
    if is_key:
        gs, gz, gr = g[:, :D], g[:, D:2 * D], g[:, 2 * D:]
        os_, oz, or_ = o[:, :D], o[:, D:2 * D], o[:, 2 * D:]
    else:
        gs, gz, gr = g[:, :128], g[:, 128:256], g[:, 256:]
        os_, oz, or_ = o[:, :128], o[:, 128:256], o[:, 256:]
    scale_err = max(_rel(gs, os_), _rel(gr, or_))
    zerr = np.abs(gz - oz) / np.maximum(np.maximum(np.abs(oz), np.abs(os_)), 1e-300)
    zero_err = float(np.where((gz == oz), 0.0, zerr).max())
    assert scale_err <= 1e-3, ("scale", scale_err)
    assert zero_err <= 1e-3, ("zero", zero_err)
    return {"scale_rel": scale_err, "zero_rel": zero_err}


def _rel(a, b):
    d = np.abs(a - b)
    r = np.where(d == 0, 0.0, d / np.maximum(np.abs(b), 1e-300))
    return float(r.max())


def compare_dequant(gpu, ref):
    """gpu: fp16 [n][128][d0]; ref: oracle float64 (or fp16) [n][128][d0]."""
    a = np.asarray(gpu, dtype=np.float64)
    b = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt((b ** 2).mean(axis=-1, keepdims=True))
    err = np.abs(a - b) / (np.abs(b) + rms + 1e-300)
    worst = float(err.max())
    assert worst <= 1e-3, worst
    return {"dequant_rel": worst}


ATTN_TOL = 2e-3
ATTN_CONDITION_ULPS = 16


def attention_allowance(q, K, V, sm_scale=None):
    """Conditioning allowance of the attention rule for the query heads q
    [G][d0] over one sequence's cache K, V [T][d0] (fp64, the oracle's
    dequantised values or the fp16 cache): 16 * 2^-24 * kappa per head."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(q.shape[-1])
    s = sm_scale * (q @ K.T)                                   # [G][T]
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    o = p @ V                                                   # [G][d0]
    term = sm_scale * np.linalg.norm(q, axis=1)[:, None] * np.linalg.norm(K, axis=1)[None, :]
    kappa = np.empty(q.shape[0])
    for h in range(q.shape[0]):
        dv = np.abs(V - o[h]).max(axis=1)                      # [T]
        kappa[h] = float((p[h] * term[h] * dv).sum())
    return ATTN_CONDITION_ULPS * 2.0 ** -24 * kappa


def compare_attention(gpu, ref, cache=None, tol=ATTN_TOL):
    """gpu, ref: [batch][n_q_heads][d0].  cache(b, h) -> (q [1][d0], K, V) in
    fp64 for query head h of sequence b, used only for heads whose error
    exceeds `tol` (without it, `tol` alone is the bar)."""
    err = np.abs(np.asarray(gpu, np.float64) - ref).max(axis=-1)     # [batch][heads]
    stats = {"attn_abs": float(err.max()), "heads": int(err.size),
             "heads_over_2e-3": int((err > tol).sum())}
    over = np.argwhere(err > tol)
    if over.size:
        assert cache is not None, stats
        worst = 0.0
        for b, h in over:
            qh, K, V = cache(int(b), int(h))
            allow = attention_allowance(qh, K, V)[0]
            ratio = err[b, h] / (tol + allow)
            worst = max(worst, float(ratio))
            assert ratio <= 1.0, dict(stats, head=(int(b), int(h)), err=float(err[b, h]),
                                      allowance=float(allow))
        stats["worst_ratio_to_conditioned_bar"] = worst
    return stats


def packed_cache(q, k_codes, v_codes, k_meta, v_meta, n_kv_heads, tiles_per_seq, k_bits=4,
                 v_bits=2):
    """cache(b, h) for compare_attention over a packed cache laid out as
    kvarn_decode_attention reads it: the oracle dequantises the (b, g) tiles."""
    q = np.asarray(q)
    d0 = q.shape[-1]
    G = q.shape[1] // n_kv_heads

    def cache(b, h):
        g = h // G
        sl = slice((b * n_kv_heads + g) * tiles_per_seq, (b * n_kv_heads + g + 1) * tiles_per_seq)
        K, _ = oracle.dequantize_tiles(k_codes[sl], k_meta[sl], d0, k_bits, True)
        V, _ = oracle.dequantize_tiles(v_codes[sl], v_meta[sl], d0, v_bits, False)
        return q[b, h][None].astype(np.float64), K.reshape(-1, d0), V.reshape(-1, d0)
    return cache


def fp16_cache(q, k, v):
    """cache(b, h) for compare_attention over an fp16 cache [B][Hkv][T][d0]."""
    q = np.asarray(q)
    G = q.shape[1] // k.shape[1]

    def cache(b, h):
        g = h // G
        return (q[b, h][None].astype(np.float64), np.asarray(k[b, g], np.float64),
                np.asarray(v[b, g], np.float64))
    return cache
