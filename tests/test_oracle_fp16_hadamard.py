"""Pins of the oracle's binary16 conversion and Hadamard rotation.

binary16 is checked against numpy's own conversion (an independent library);
the rotation against scipy.linalg.hadamard (library Sylvester construction),
the closed form H H^T = n I, and the energy / involution properties of an
orthonormal rotation.  Page: "KVarN Hadamard 旋转与方差归一化" (blog.hotdry.top),
section "Hadamard 旋转"; deep-dive page (vatt-ghern.pages.dev), stage card
"Hadamard rotation" and the worked example's closing remark on the 28.0 outlier.
"""
import numpy as np
import pytest
import scipy.linalg

import oracle


def test_half_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _all_finite_halves():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = b.view(np.float16).astype(np.float64)
    return np.unique(v[np.isfinite(v)])


def test_half_encode_ties_and_random():
    vals = _all_finite_halves()
    mids = (vals[:-1] + vals[1:]) / 2.0               # exact ties between neighbours
    rng = np.random.default_rng(123)
    rnd = rng.uniform(vals[:-1], vals[1:])             # one point in every gap
    extra = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 70000.0, -65520.0,
                      2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26, 1e-300,
                      6.1e-5, 6.103515625e-05, -6.0975e-05])
    xs = np.concatenate([vals, mids, rnd, extra])
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([oracle.double_to_half(float(x)) for x in xs], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(xs[i], hex(got[i]), hex(ref[i])) for i in bad[:5]]


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_is_sylvester_and_orthogonal(n):
    H = np.array([[oracle.hadamard_entry(i, j) for j in range(n)] for i in range(n)])
    assert np.array_equal(H, scipy.linalg.hadamard(n))
    assert np.array_equal(H @ H.T, n * np.eye(n, dtype=H.dtype))


@pytest.mark.parametrize("n", [2, 8, 64, 128, 256])
def test_fwht_equals_dense_product(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal(n)
    ref = x @ scipy.linalg.hadamard(n)
    got = oracle.fwht(x)
    assert np.allclose(got, ref, rtol=0, atol=1e-12 * np.abs(x).sum())


@pytest.mark.parametrize("d0", [64, 96, 128, 256])
def test_rotate_tile_is_padded_orthonormal_hadamard(d0):
    rng = np.random.default_rng(d0)
    x16 = rng.standard_normal((128, d0)).astype(np.float16)
    D = oracle.padded_dim(d0)
    assert D == {64: 64, 96: 128, 128: 128, 256: 256}[d0]
    xp = np.zeros((128, D))
    xp[:, :d0] = x16.astype(np.float64)
    ref = xp @ scipy.linalg.hadamard(D) / np.sqrt(D)
    xt = oracle.rotate_tile(x16)
    assert np.allclose(xt, ref, rtol=0, atol=1e-12)
    # energy of every token row is preserved (orthonormal rotation)
    assert np.allclose((xt ** 2).sum(1), (xp ** 2).sum(1), rtol=1e-12)
    # the scaled transform is its own inverse
    back = np.stack([oracle.fwht(r) for r in xt]) / np.sqrt(D)
    assert np.allclose(back, xp, rtol=0, atol=1e-12)


def test_one_hot_spreads_evenly():
    D = 128
    for k in (0, 5, 77, 127):
        x = np.zeros((128, D), np.float16)
        x[:, k] = 1.0
        xt = oracle.rotate_tile(x)
        assert np.allclose(np.abs(xt), 1.0 / np.sqrt(D), rtol=0, atol=1e-15)


def test_outlier_drops_to_single_digits():
    # A 28.0 outlier among small values (the worked example's group) lands in
    # single digits after rotation.
    rng = np.random.default_rng(7)
    row = rng.uniform(-0.6, 0.6, 128)
    row[37] = 28.0
    x = np.tile(row, (128, 1)).astype(np.float16)
    xt = oracle.rotate_tile(x)
    assert np.abs(x.astype(np.float64)).max() == 28.0
    assert np.abs(xt).max() < 10.0
