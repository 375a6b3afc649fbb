"""Parity rules between the HIP path and the oracle (shared by the GPU tests).

Codes: bit-exact, except codes off by exactly one where the oracle's own
value sits at a rounding boundary.  A mismatch is excused when the oracle's
u = (Y - z)/s lies within W = 1e-6 * max(1, (|Y| + |z|)/s) of a half
integer: the distance a relative perturbation of 1e-6 in the operands Y and z
can move u.  At most 1e-4 of the codes may be excused.

Scales (SK, RK, SV, CV): |a - b| <= 1e-3 |b|.  Zero points (ZK, ZV):
|a - b| <= 1e-3 max(|b|, the group's stored scale).
Dequantised values: |a - b| <= 1e-3 (|b| + rms of b's token row).
Attention outputs: max |a - b| <= 2e-3.
"""
import numpy as np

import oracle

CODE_WINDOW = 1e-6
CODE_MAX_FRACTION = 1e-4


def unpack_all(codes, D, bits, is_key):
    return np.stack([oracle.unpack(c, D, bits, is_key) for c in codes])


def compare_codes(gpu_codes, q, D, bits, is_key):
    """gpu_codes: [n][code_bytes] uint8; q: oracle.quantize_tiles(..., diag=True).

    Returns a dict of statistics; raises AssertionError on a violation."""
    g = unpack_all(gpu_codes, D, bits, is_key).astype(np.int64)
    o = unpack_all(q["codes"], D, bits, is_key).astype(np.int64)
    bad = g != o
    n = g.size
    stats = {"codes": n, "mismatch": int(bad.sum()), "worst_window_ratio": 0.0}
    if not bad.any():
        return stats
    diff = np.abs(g - o)[bad]
    assert diff.max() == 1, "code off by %d" % diff.max()
    y, u = q["y"], q["u"]
    if is_key:
        z = np.broadcast_to(q["z"][:, None, :], y.shape)
        s = np.broadcast_to(q["s"][:, None, :], y.shape)
    else:
        z = np.broadcast_to(q["z"][:, :, None], y.shape)
        s = np.broadcast_to(q["s"][:, :, None], y.shape)
    yb, zb, sb, ub = y[bad], z[bad], s[bad], u[bad]
    mag = np.where(sb > 0, (np.abs(yb) + np.abs(zb)) / np.where(sb > 0, sb, 1.0), 1.0)
    W = CODE_WINDOW * np.maximum(1.0, mag)
    dist = np.abs(ub - np.floor(ub) - 0.5)
    ratio = dist / W
    stats["worst_window_ratio"] = float(ratio.max())
    stats["unexcused"] = int((ratio > 1.0).sum())
    assert stats["unexcused"] == 0, stats
    assert stats["mismatch"] <= CODE_MAX_FRACTION * n, stats
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


def compare_attention(gpu, ref, tol=2e-3):
    worst = float(np.abs(np.asarray(gpu, np.float64) - ref).max())
    assert worst <= tol, worst
    return {"attn_abs": worst}
