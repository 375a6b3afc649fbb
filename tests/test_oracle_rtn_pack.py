"""Pins of the oracle's asymmetric RTN, fold and bit packing.

Pages: deep-dive page (vatt-ghern.pages.dev), section "為什麼樸素的 2-bit
量化會在長 decode 裡掉準" (the worked 2-bit example: range [min, max], 2^b
levels, scale = range / (2^b - 1), code = round((v - min)/scale)) and the
KEY/VALUE table in "四個步驟" (keys scaled per channel, values per token);
hotdry page (blog.hotdry.top), "非对称量化与尺度折叠" (K 4-bit, V 2-bit,
per-channel K scales and per-token V scales folded back on read) and the
deep-dive page's capacity widget text (K4V2 g128 stores below a quarter of
fp16).
"""
import os

import numpy as np
import pytest

import oracle
from kv_cache_bit_token_amd import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_2bit.txt")


def _read_golden(path):
    out = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.split()
    return out


def test_worked_example_from_page():
    g = _read_golden(GOLDEN)
    bits = int(g["bits"][0])
    vals16 = np.array([float(x) for x in g["values"]], np.float16)
    v = vals16.astype(np.float64)
    z, s, codes, u = oracle.rtn_group(v, bits)
    assert z == pytest.approx(float(g["min"][0]), abs=1e-3)
    assert v.max() == float(g["max"][0])
    sd = int(g["scale_decimals"][0])
    assert round(s, sd) == pytest.approx(float(g["scale"][0]), abs=10 ** -sd / 2)
    ud = int(g["u_decimals"][0])
    for val, up, cp in zip(g["u_checked_values"], g["u_printed"], g["codes_checked"]):
        i = int(np.nonzero(vals16 == np.float16(float(val)))[0][0])
        assert round(u[i], ud) == pytest.approx(float(up), abs=10 ** -ud / 2), (val, u[i])
        assert codes[i] == int(cp)
    # every value other than the outlier lands in code 0 and comes back as ~min
    assert list(codes) == [0, 0, 0, 0, 0, 0, 3]
    assert 0 * s + z == pytest.approx(float(g["dequant_of_code0"][0]), abs=1e-3)


@pytest.mark.parametrize("bits", [2, 4])
def test_rtn_is_nearest_level_brute_force(bits):
    rng = np.random.default_rng(bits)
    L = (1 << bits) - 1
    for _ in range(200):
        n = int(rng.integers(2, 40))
        v = rng.standard_normal(n) * rng.uniform(0.01, 100) + rng.uniform(-5, 5)
        z, s, codes, u = oracle.rtn_group(v, bits)
        levels = v.min() + np.arange(L + 1) * (v.max() - v.min()) / L
        ref = np.abs(v[:, None] - levels[None, :]).argmin(1)
        assert np.array_equal(codes, ref)
        assert np.all(np.abs(v - (codes * s + z)) <= s / 2 * (1 + 1e-12))
        assert codes[v.argmin()] == 0 and codes[v.argmax()] == L


def test_rtn_flat_group():
    z, s, codes, u = oracle.rtn_group(np.full(9, -2.25), 4)
    assert z == -2.25 and s == 0.0 and not codes.any()


def _cfg1():
    k, v = synthetic.outlier_kv_host(0, 1, 512, 128)
    return synthetic.as_tiles(k), synthetic.as_tiles(v)


@pytest.mark.parametrize("is_key,bits", [(True, 4), (False, 2), (True, 2), (False, 4)])
def test_group_axis_and_error_bound(is_key, bits):
    kt, vt = _cfg1()
    x = kt if is_key else vt
    q = oracle.quantize_tiles(x, bits, 5, is_key, diag=True)
    L = (1 << bits) - 1
    for i in range(x.shape[0]):
        c = oracle.unpack(q["codes"][i], 128, bits, is_key).astype(np.float64)
        y, z, s = q["y"][i], q["z"][i], q["s"][i]
        ax = 0 if is_key else 1            # K groups run over tokens (axis 0) per channel
        assert np.all(c.min(axis=ax) == 0) and np.all(c.max(axis=ax) == L)
        zz = z[None, :] if is_key else z[:, None]
        ss = s[None, :] if is_key else s[:, None]
        assert np.all(np.abs(y - (c * ss + zz)) <= ss / 2 * (1 + 1e-12) + 1e-300)
        lo = np.take_along_axis(c, np.expand_dims(np.argmin(y, axis=ax), ax), ax)
        hi = np.take_along_axis(c, np.expand_dims(np.argmax(y, axis=ax), ax), ax)
        assert np.all(lo == 0) and np.all(hi == L)


@pytest.mark.parametrize("is_key,bits", [(True, 4), (False, 2)])
def test_stored_fields_error_bound(is_key, bits):
    """|Xt - dequant_rotated| obeys the bound built from the fp16 rounding of
    each stored field (rotated domain, before the inverse rotation)."""
    kt, vt = _cfg1()
    x = (kt if is_key else vt)[:2]
    q = oracle.quantize_tiles(x, bits, 5, is_key, diag=True)
    D = 128
    for i in range(x.shape[0]):
        xt = oracle.rotate_tile(x[i])
        c = oracle.unpack(q["codes"][i], D, bits, is_key).astype(np.float64)
        m = q["meta"][i].astype(np.float64)
        lr, lc, z, s = q["lr"][i], q["lc"][i], q["z"][i], q["s"][i]
        if is_key:
            S, Z, R = m[:D][None, :], m[D:2 * D][None, :], m[2 * D:][:, None]
            S0 = (np.exp(lc) * s)[None, :]
            Z0 = (np.exp(lc) * z)[None, :]
            R0 = np.exp(lr)[:, None]
        else:
            S, Z, R = m[:128][:, None], m[128:256][:, None], m[256:][None, :]
            S0 = (np.exp(lr) * s)[:, None]
            Z0 = (np.exp(lr) * z)[:, None]
            R0 = np.exp(lc)[None, :]
        deq = R * (c * S + Z)
        bound = (R0 * S0 / 2 + R0 * (c * np.abs(S - S0) + np.abs(Z - Z0))
                 + np.abs(R - R0) * np.abs(c * S + Z))
        assert np.all(np.abs(xt - deq) <= bound * (1 + 1e-9) + 1e-12)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("is_key", [True, False])
def test_pack_roundtrip(D, bits, is_key):
    rng = np.random.default_rng(D + bits)
    c = rng.integers(0, 1 << bits, size=(128, D)).astype(np.uint8)
    p = oracle.pack(c, bits, is_key)
    assert p.size == 128 * D * bits // 8
    assert np.array_equal(oracle.unpack(p, D, bits, is_key), c)


def test_pack_bit_layout_by_hand():
    D = 128
    c = np.zeros((128, D), np.uint8)
    c[0, 0], c[0, 1], c[0, 2], c[1, 0] = 0x3, 0xA, 0x5, 0xF
    p = oracle.pack(c, 4, True)          # K: element t*D + j, 4 bits, LSB first
    assert p[0] == 0xA3 and p[1] == 0x05 and p[D // 2] == 0x0F
    c = np.zeros((128, D), np.uint8)
    c[0, 0], c[1, 0], c[2, 0], c[3, 0], c[0, 1] = 1, 2, 3, 1, 2
    p = oracle.pack(c, 2, False)         # V: element j*128 + t, 2 bits, LSB first
    assert p[0] == (1 | 2 << 2 | 3 << 4 | 1 << 6) and p[128 * 2 // 8] == 2


def test_sizes_match_capacity_claim():
    # K4V2, 128-token tiles, head_dim 128: codes + fp16 meta per tile pair
    D = 128
    pair = (oracle.code_bytes(D, 4) + oracle.code_bytes(D, 2)
            + 2 * oracle.meta_halves(D, True) + 2 * oracle.meta_halves(D, False))
    assert pair == 13824
    fp16 = 2 * 128 * D * 2
    assert pair / fp16 < 0.25          # under a quarter of the fp16 bytes
    assert 4.0 < fp16 / pair < 5.0
