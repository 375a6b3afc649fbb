"""ctypes binding of the CPU oracle (kvarn_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  The product package never imports it.

All arrays are numpy.  binary16 data travels as numpy.float16 (viewed as
uint16 at the C boundary); double results come back as float64.
"""
import ctypes
import os

import numpy as np

TILE = 128
_HERE = os.path.dirname(os.path.abspath(__file__))
# KVARN_ORACLE_LIB lets a mutation check load a deliberately broken build of
# this same source; normal runs use the in-tree library.
_LIB_PATH = os.environ.get("KVARN_ORACLE_LIB", os.path.join(_HERE, "libkvarn_oracle.so"))
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i64 = ctypes.c_int64
_int = ctypes.c_int
_i32p = ctypes.POINTER(ctypes.c_int32)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    src = os.path.join(_HERE, "kvarn_oracle.c")
    if "KVARN_ORACLE_LIB" not in os.environ and (
            not os.path.exists(_LIB_PATH) or os.path.getmtime(src) > os.path.getmtime(_LIB_PATH)):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "oracle_half_to_double": (ctypes.c_double, [ctypes.c_uint16]),
        "oracle_double_to_half": (ctypes.c_uint16, [ctypes.c_double]),
        "oracle_padded_dim": (_int, [_int]),
        "oracle_hadamard_entry": (_int, [_int, _int]),
        "oracle_fwht": (None, [_dp, _int]),
        "oracle_rotate_tile": (None, [_u16p, _int, _dp]),
        "oracle_normalise": (None, [_dp, _int, _int, _dp, _dp]),
        "oracle_recentre": (None, [_dp, _dp, _int]),
        "oracle_rtn_group": (None, [_dp, _int, _int, _int, _dp, _dp, _u8p, _int, _dp]),
        "oracle_code_bytes": (_i64, [_int, _int]),
        "oracle_meta_halves": (_i64, [_int, _int]),
        "oracle_pack": (None, [_u8p, _int, _int, _int, _u8p]),
        "oracle_unpack": (None, [_u8p, _int, _int, _int, _u8p]),
        "oracle_quantize_tiles": (None, [_i64, _int, _int, _int, _int, _u16p, _u8p, _u16p,
                                         _dp, _dp, _dp, _dp, _dp, _dp]),
        "oracle_dequantize_tiles": (None, [_i64, _int, _int, _int, _u8p, _u16p, _dp, _u16p]),
        "oracle_decode_attention": (None, [_int, _int, _int, _int, _int, _int, _int, _u16p,
                                           _u8p, _u8p, _u16p, _u16p, ctypes.c_double, _dp]),
        "oracle_decode_attention_paged": (None, [_int, _int, _int, _int, _int, _int, _int, _i32p,
                                                 _i32p, _i32p, _u16p, _u8p, _u8p, _u16p, _u16p,
                                                 _u16p, _u16p, ctypes.c_double, _dp]),
        "oracle_decode_attention_fp16": (None, [_int, _int, _int, _i64, _int, _u16p, _u16p, _u16p,
                                                ctypes.c_double, _dp]),
        "oracle_set_threads": (None, [_int]),
        "oracle_max_threads": (_int, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a, typ):
    if a is None:
        return ctypes.cast(None, typ)
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(typ)


def _h(a):
    """float16 array -> contiguous uint16 view."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    assert a.dtype == np.uint16
    return a


# ---------------------------------------------------------------- scalars

def half_to_double(bits: int) -> float:
    return _load().oracle_half_to_double(int(bits))


def double_to_half(x: float) -> int:
    return _load().oracle_double_to_half(float(x))


def padded_dim(d0: int) -> int:
    return _load().oracle_padded_dim(int(d0))


def hadamard_entry(i: int, j: int) -> int:
    return _load().oracle_hadamard_entry(int(i), int(j))


def code_bytes(D: int, bits: int) -> int:
    return _load().oracle_code_bytes(int(D), int(bits))


def meta_halves(D: int, is_key: bool) -> int:
    return _load().oracle_meta_halves(int(D), int(bool(is_key)))


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return _load().oracle_max_threads()


# ---------------------------------------------------------------- steps

def fwht(x):
    """Unnormalised Walsh-Hadamard transform of a 1-D vector (x H_n)."""
    y = np.array(x, dtype=np.float64, copy=True)
    _load().oracle_fwht(_ptr(y, _dp), y.shape[0])
    return y


def rotate_tile(x16):
    """[128][d0] float16 tile -> [128][D] rotated (padded, scaled) tile."""
    x = _h(x16)
    d0 = x.shape[1]
    out = np.empty((TILE, padded_dim(d0)), np.float64)
    _load().oracle_rotate_tile(_ptr(x, _u16p), d0, _ptr(out, _dp))
    return out


def normalise(xt, n_iters: int):
    """Rotated tile [128][D] -> (lr[128], lc[D]) log-factors."""
    xt = np.ascontiguousarray(xt, dtype=np.float64)
    D = xt.shape[1]
    lr = np.empty(TILE, np.float64)
    lc = np.empty(D, np.float64)
    _load().oracle_normalise(_ptr(xt, _dp), D, int(n_iters), _ptr(lr, _dp), _ptr(lc, _dp))
    return lr, lc


def recentre(lr, lc):
    """Gauge step: move mean(lc) from the column to the row log-factors."""
    lr = np.array(lr, dtype=np.float64, copy=True)
    lc = np.array(lc, dtype=np.float64, copy=True)
    _load().oracle_recentre(_ptr(lr, _dp), _ptr(lc, _dp), lc.shape[0])
    return lr, lc


def rtn_group(v, bits: int):
    """One asymmetric RTN group -> (z, s, codes, u)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    n = v.shape[0]
    z = ctypes.c_double()
    s = ctypes.c_double()
    codes = np.empty(n, np.uint8)
    u = np.empty(n, np.float64)
    _load().oracle_rtn_group(_ptr(v, _dp), n, 1, int(bits), ctypes.byref(z), ctypes.byref(s),
                             _ptr(codes, _u8p), 1, _ptr(u, _dp))
    return z.value, s.value, codes, u


def pack(codes, bits: int, is_key: bool):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    D = codes.shape[1]
    out = np.empty(code_bytes(D, bits), np.uint8)
    _load().oracle_pack(_ptr(codes, _u8p), D, int(bits), int(bool(is_key)), _ptr(out, _u8p))
    return out


def unpack(packed, D: int, bits: int, is_key: bool):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.empty((TILE, D), np.uint8)
    _load().oracle_unpack(_ptr(packed, _u8p), int(D), int(bits), int(bool(is_key)), _ptr(out, _u8p))
    return out


# ---------------------------------------------------------------- batched

def quantize_tiles(x16, bits: int, n_iters: int, is_key: bool, diag: bool = False):
    """Quantise [n_tiles][128][d0] float16 tiles of one tensor.

    Returns dict with 'codes' [n][code_bytes] uint8 and 'meta' [n][meta_halves]
    float16; with diag=True also 'y', 'u' [n][128][D], 'z', 's' [n][G],
    'lr' [n][128], 'lc' [n][D] (float64).
    """
    x = _h(x16)
    n, t, d0 = x.shape
    assert t == TILE
    D = padded_dim(d0)
    G = D if is_key else TILE
    codes = np.empty((n, code_bytes(D, bits)), np.uint8)
    meta = np.empty((n, meta_halves(D, is_key)), np.uint16)
    out = {"codes": codes}
    arrs = {}
    if diag:
        arrs = {
            "y": np.empty((n, TILE, D)), "u": np.empty((n, TILE, D)),
            "z": np.empty((n, G)), "s": np.empty((n, G)),
            "lr": np.empty((n, TILE)), "lc": np.empty((n, D)),
        }
    g = lambda k: _ptr(arrs.get(k), _dp)  # noqa: E731
    _load().oracle_quantize_tiles(n, d0, int(bits), int(n_iters), int(bool(is_key)),
                                  _ptr(x, _u16p), _ptr(codes, _u8p), _ptr(meta, _u16p),
                                  g("y"), g("u"), g("z"), g("s"), g("lr"), g("lc"))
    out["meta"] = meta.view(np.float16)
    out.update(arrs)
    return out


def dequantize_tiles(codes, meta16, d0: int, bits: int, is_key: bool):
    """Packed tiles -> (float64 [n][128][d0], float16 [n][128][d0])."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    meta = _h(meta16)
    n = codes.shape[0]
    o64 = np.empty((n, TILE, d0), np.float64)
    o16 = np.empty((n, TILE, d0), np.uint16)
    _load().oracle_dequantize_tiles(n, int(d0), int(bits), int(bool(is_key)),
                                    _ptr(codes, _u8p), _ptr(meta, _u16p),
                                    _ptr(o64, _dp), _ptr(o16, _u16p))
    return o64, o16.view(np.float16)


def decode_attention(q16, k_codes, v_codes, k_meta16, v_meta16, *, n_kv_heads: int,
                     tiles_per_seq: int, k_bits: int = 4, v_bits: int = 2,
                     sm_scale: float = None):
    """q [batch][n_q_heads][d0] float16 -> out [batch][n_q_heads][d0] float64."""
    q = _h(q16)
    batch, hq, d0 = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d0)
    kc = np.ascontiguousarray(k_codes, dtype=np.uint8)
    vc = np.ascontiguousarray(v_codes, dtype=np.uint8)
    km, vm = _h(k_meta16), _h(v_meta16)
    out = np.empty((batch, hq, d0), np.float64)
    _load().oracle_decode_attention(batch, hq, int(n_kv_heads), int(tiles_per_seq), d0,
                                    int(k_bits), int(v_bits), _ptr(q, _u16p),
                                    _ptr(kc, _u8p), _ptr(vc, _u8p), _ptr(km, _u16p),
                                    _ptr(vm, _u16p), float(sm_scale), _ptr(out, _dp))
    return out


def decode_attention_paged(q16, k_codes, v_codes, k_meta16, v_meta16, block_table, n_blocks,
                           tail_len, k_tail16, v_tail16, *, n_kv_heads: int, k_bits: int = 4,
                           v_bits: int = 2, sm_scale: float = None):
    """Paged cache plus fp16 tail.  block_table [batch][max_blocks] int32 (physical
    block p holds tiles p * n_kv_heads + g), n_blocks / tail_len [batch] int32,
    k_tail / v_tail [batch][n_kv_heads][128][d0] float16.  -> [batch][hq][d0] f64."""
    q = _h(q16)
    batch, hq, d0 = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d0)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    nb = np.ascontiguousarray(n_blocks, dtype=np.int32)
    tl = np.ascontiguousarray(tail_len, dtype=np.int32)
    assert bt.ndim == 2 and bt.shape[0] == batch and nb.shape == (batch,) and tl.shape == (batch,)
    kc = np.ascontiguousarray(k_codes, dtype=np.uint8)
    vc = np.ascontiguousarray(v_codes, dtype=np.uint8)
    km, vm = _h(k_meta16), _h(v_meta16)
    kt, vt = _h(k_tail16), _h(v_tail16)
    assert kt.shape == (batch, n_kv_heads, 128, d0) and vt.shape == kt.shape
    out = np.empty((batch, hq, d0), np.float64)
    _load().oracle_decode_attention_paged(
        batch, hq, int(n_kv_heads), bt.shape[1], d0, int(k_bits), int(v_bits),
        bt.ctypes.data_as(_i32p), nb.ctypes.data_as(_i32p), tl.ctypes.data_as(_i32p),
        _ptr(q, _u16p), _ptr(kc, _u8p), _ptr(vc, _u8p), _ptr(km, _u16p), _ptr(vm, _u16p),
        _ptr(kt, _u16p), _ptr(vt, _u16p), float(sm_scale), _ptr(out, _dp))
    return out


def decode_attention_fp16(q16, k16, v16, *, sm_scale: float = None):
    """Attention over an uncompressed fp16 cache.  q [batch][n_q_heads][d0],
    k / v [batch][n_kv_heads][seq_len][d0] float16 -> [batch][n_q_heads][d0] f64."""
    q = _h(q16)
    batch, hq, d0 = q.shape
    k, v = _h(k16), _h(v16)
    assert k.ndim == 4 and k.shape[0] == batch and k.shape[3] == d0 and v.shape == k.shape
    hkv, seq = k.shape[1], k.shape[2]
    assert hq % hkv == 0
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d0)
    out = np.empty((batch, hq, d0), np.float64)
    _load().oracle_decode_attention_fp16(batch, hq, hkv, seq, d0, _ptr(q, _u16p), _ptr(k, _u16p),
                                         _ptr(v, _u16p), float(sm_scale), _ptr(out, _dp))
    return out
