"""Host-side checks of the C ABI (no GPU needed).

libkvarn.so must load and export every function include/kvarn.h declares,
and every argument error must come back as its status code from host-side
validation, before anything touches a GPU.  Calls with valid arguments are
limited to ones that launch nothing (n_tiles == 0, both tensors skipped).
"""
import ctypes
import os
import re

import pytest

from kv_cache_bit_token_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvarn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvarn_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared():
        assert hasattr(lib, name), name


def P(head_dim=128, tile=128, kb=4, vb=2, it=5):
    return _lib.Params(head_dim, tile, kb, vb, it)


def test_layout_and_errors():
    lib = _lib.load()
    lay = _lib.TileLayout()
    assert lib.kvarn_get_layout(ctypes.byref(P()), ctypes.byref(lay)) == 0
    assert (lay.padded_dim, lay.k_code_bytes, lay.v_code_bytes, lay.k_meta_bytes,
            lay.v_meta_bytes) == (128, 8192, 4096, 768, 768)
    assert lib.kvarn_get_layout(ctypes.byref(P(96)), ctypes.byref(lay)) == 0 and lay.padded_dim == 128
    assert lib.kvarn_get_layout(ctypes.byref(P(40)), ctypes.byref(lay)) == 0 and lay.padded_dim == 64
    assert lib.kvarn_get_layout(ctypes.byref(P(256, kb=2, vb=4)), ctypes.byref(lay)) == 0
    assert (lay.padded_dim, lay.k_code_bytes, lay.v_code_bytes) == (256, 8192, 16384)
    cases = [
        (None, 1), (P(head_dim=32), 2), (P(head_dim=264), 2), (P(head_dim=100), 2),
        (P(tile=64), 3), (P(kb=3), 4), (P(vb=8), 4), (P(it=-1), 5), (P(it=17), 5),
    ]
    for p, want in cases:
        arg = None if p is None else ctypes.byref(p)
        assert lib.kvarn_get_layout(arg, ctypes.byref(lay)) == want, (p and (p.head_dim, p.tile_tokens))
    assert lib.kvarn_get_layout(ctypes.byref(P()), None) == 1


def test_preset_parser():
    lib = _lib.load()
    p = _lib.Params()
    assert lib.kvarn_params_from_preset(b"kvarn_k4v2_g128", 128, 5, ctypes.byref(p)) == 0
    assert (p.head_dim, p.tile_tokens, p.k_bits, p.v_bits, p.n_iters) == (128, 128, 4, 2, 5)
    assert lib.kvarn_params_from_preset(b"kvarn_k2v2_g128", 96, 3, ctypes.byref(p)) == 0
    assert (p.k_bits, p.v_bits, p.head_dim) == (2, 2, 96)
    assert lib.kvarn_params_from_preset(b"kvarn_k4v2_g64", 128, 5, ctypes.byref(p)) == 3
    assert lib.kvarn_params_from_preset(b"kvarn_k8v2_g128", 128, 5, ctypes.byref(p)) == 4
    assert lib.kvarn_params_from_preset(b"fp8", 128, 5, ctypes.byref(p)) == 4
    assert lib.kvarn_params_from_preset(b"kvarn_k4v2_g", 128, 5, ctypes.byref(p)) == 3
    assert lib.kvarn_params_from_preset(None, 128, 5, ctypes.byref(p)) == 1
    assert lib.kvarn_params_from_preset(b"kvarn_k4v2_g128", 128, 99, ctypes.byref(p)) == 5


A = ctypes.c_void_p(0x10000)        # aligned, never dereferenced by these calls
MIS = ctypes.c_void_p(0x10008)      # 8-byte aligned only


def test_quantize_validation_without_launch():
    lib = _lib.load()
    q = lib.kvarn_quantize_tiles
    ok = ctypes.byref(P())
    # valid but launches nothing
    assert q(ok, 0, A, A, A, A, A, A, None) == 0
    assert q(ok, 5, None, None, None, None, None, None, None) == 0
    # errors
    assert q(None, 1, A, A, A, A, A, A, None) == 1
    assert q(ctypes.byref(P(head_dim=30)), 1, A, A, A, A, A, A, None) == 2
    assert q(ctypes.byref(P(tile=256)), 1, A, A, A, A, A, A, None) == 3
    assert q(ctypes.byref(P(kb=1)), 1, A, A, A, A, A, A, None) == 4
    assert q(ctypes.byref(P(it=40)), 1, A, A, A, A, A, A, None) == 5
    assert q(ok, 1, A, A, None, A, A, A, None) == 1          # K set partly NULL
    assert q(ok, 1, A, A, A, A, A, None, None) == 1          # V set partly NULL
    assert q(ok, -1, A, A, A, A, A, A, None) == 6
    assert q(ok, 1 << 40, A, A, A, A, A, A, None) == 6
    assert q(ok, 1, MIS, A, A, A, A, A, None) == 7
    assert q(ok, 1, A, A, A, A, A, MIS, None) == 7


def test_dequantize_validation_without_launch():
    lib = _lib.load()
    d = lib.kvarn_dequantize_tiles
    ok = ctypes.byref(P())
    assert d(ok, 0, A, A, A, A, A, A, None) == 0
    assert d(ok, 3, None, None, None, None, None, None, None) == 0
    assert d(None, 1, A, A, A, A, A, A, None) == 1
    assert d(ctypes.byref(P(vb=3)), 1, A, A, A, A, A, A, None) == 4
    assert d(ok, 1, A, A, None, A, A, A, None) == 1
    assert d(ok, -2, A, A, A, A, A, A, None) == 6
    assert d(ok, 1, A, A, A, A, MIS, A, None) == 7


def test_attention_validation_without_launch():
    lib = _lib.load()
    ws = lib.kvarn_decode_attention_workspace
    nb = ctypes.c_size_t()
    ok = ctypes.byref(P())
    assert ws(ok, 64, 32, 8, 256, ctypes.byref(nb)) == 0 and nb.value > 0
    need = nb.value
    assert ws(ok, 64, 30, 8, 256, ctypes.byref(nb)) == 6      # 30 % 8 != 0
    assert ws(ok, -1, 32, 8, 256, ctypes.byref(nb)) == 6
    assert ws(ok, 1, 64, 2, 1, ctypes.byref(nb)) == 6         # group of 32 heads > 16
    assert ws(ok, 64, 32, 8, 256, None) == 1
    at = lib.kvarn_decode_attention
    assert at(ok, 0, 32, 8, 256, A, A, A, A, A, 0.1, A, A, need, None) == 0   # empty batch
    assert at(ok, 64, 32, 8, 256, None, A, A, A, A, 0.1, A, A, need, None) == 1
    assert at(ok, 64, 32, 8, 256, A, A, A, A, A, 0.1, A, None, need, None) == 1
    assert at(ok, 64, 32, 8, 256, A, A, A, A, A, 0.1, A, A, need - 4, None) == 8
    assert at(ok, 64, 32, 8, 256, A, A, A, A, MIS, 0.1, A, A, need, None) == 7
    assert at(ctypes.byref(P(head_dim=7)), 64, 32, 8, 256, A, A, A, A, A, 0.1, A, A, need, None) == 2


def test_noalloc_attention_validation_without_launch():
    """The allocation-free entry point refuses, before touching any GPU, a
    shape whose workspace exceeds the static scratch, and validates like
    kvarn_decode_attention otherwise."""
    lib = _lib.load()
    na = lib.kvarn_decode_attention_noalloc
    ok = ctypes.byref(P())
    assert na(ok, 0, 32, 8, 256, A, A, A, A, A, 0.1, A, None) == 0        # empty batch
    assert na(ok, 64, 32, 8, 256, None, A, A, A, A, 0.1, A, None) == 1
    assert na(ok, 64, 32, 8, 256, A, A, A, None, A, 0.1, A, None) == 1
    assert na(ok, 64, 32, 8, 256, A, A, A, A, MIS, 0.1, A, None) == 7
    assert na(ok, 64, 30, 8, 256, A, A, A, A, A, 0.1, A, None) == 6
    # G = 16, head_dim 256, 8192 pairs of one tile: 8192 * 16 * 258 * 4 B of partials
    big = ctypes.byref(P(head_dim=256))
    nb = ctypes.c_size_t()
    assert lib.kvarn_decode_attention_workspace(big, 8192, 16, 1, 1, ctypes.byref(nb)) == 0
    assert nb.value > (64 << 20)
    assert na(big, 8192, 16, 1, 1, A, A, A, A, A, 0.1, A, None) == 8


def test_quantize_to_validation_without_launch():
    lib = _lib.load()
    q = lib.kvarn_quantize_tiles_to
    ok = ctypes.byref(P())
    assert q(ok, 0, A, A, A, 4, A, A, A, A, None) == 0          # nothing to do
    assert q(ok, 3, A, A, A, 0, A, A, A, A, None) == 0          # empty pool: every tile skipped
    assert q(ok, 3, None, None, None, 4, None, None, None, None, None) == 0
    assert q(ok, 3, A, A, None, 4, A, A, A, A, None) == 1       # no destination table
    assert q(ok, 3, A, A, A, -1, A, A, A, A, None) == 6
    assert q(ok, -3, A, A, A, 4, A, A, A, A, None) == 6
    assert q(ok, 3, A, A, MIS, 4, A, A, A, A, None) == 7
    assert q(ok, 3, A, None, A, 4, A, A, A, A, None) == 1       # V set partly NULL
    assert q(ctypes.byref(P(it=-1)), 3, A, A, A, 4, A, A, A, A, None) == 5


def test_paged_attention_validation_without_launch():
    lib = _lib.load()
    ws = lib.kvarn_decode_attention_paged_workspace
    nb = ctypes.c_size_t()
    ok = ctypes.byref(P())
    assert ws(ok, 16, 32, 8, 256, ctypes.byref(nb)) == 0 and nb.value > 0
    need = nb.value
    assert ws(ok, 16, 32, 8, 0, ctypes.byref(nb)) == 0 and 0 < nb.value < need   # tail slot only
    assert ws(ok, 16, 32, 8, -1, ctypes.byref(nb)) == 6
    assert ws(ok, 16, 31, 8, 4, ctypes.byref(nb)) == 6
    assert ws(ok, 16, 32, 8, 4, None) == 1
    at = lib.kvarn_decode_attention_paged
    args = lambda **kw: [kw.get("p", ok), kw.get("batch", 16), 32, 8, 256, kw.get("pool", 100),
                         kw.get("table", A), A, kw.get("tail", A), A, A, A, A, A,
                         kw.get("kt", A), A, 0.1, A, kw.get("ws", A), kw.get("wsb", need), None]
    assert at(*args(batch=0)) == 0                                 # empty batch: no launch
    assert at(*args(tail=None)) == 1
    assert at(*args(kt=None)) == 1
    assert at(*args(table=None)) == 1                              # pool present, table missing
    assert at(*args(ws=None)) == 1
    assert at(*args(wsb=need - 8)) == 8
    assert at(*args(pool=-5)) == 6
    assert at(*args(table=MIS)) == 7
    assert at(*args(p=ctypes.byref(P(head_dim=300)))) == 2


def test_fp16_attention_validation_without_launch():
    lib = _lib.load()
    ws = lib.kvarn_decode_attention_fp16_workspace
    nb = ctypes.c_size_t()
    assert ws(128, 64, 32, 8, 32768, ctypes.byref(nb)) == 0 and nb.value > 0
    need = nb.value
    assert ws(128, 64, 32, 8, 0, ctypes.byref(nb)) == 0 and nb.value == 0
    assert ws(130, 64, 32, 8, 100, ctypes.byref(nb)) == 2          # not a multiple of 8
    assert ws(128, 64, 32, 8, -1, ctypes.byref(nb)) == 6
    assert ws(128, 64, 32, 6, 100, ctypes.byref(nb)) == 6          # 32 % 6 != 0
    assert ws(128, 1, 32, 1, 100, ctypes.byref(nb)) == 6           # group of 32 heads
    assert ws(256, 1, 4, 1, 1 << 22, ctypes.byref(nb)) == 6        # 2 GiB of K per head
    assert ws(128, 64, 32, 8, 100, None) == 1
    at = lib.kvarn_decode_attention_fp16
    args = lambda **kw: [kw.get("hd", 128), kw.get("batch", 64), 32, 8, kw.get("T", 32768),
                         kw.get("q", A), kw.get("k", A), A, 0.1, kw.get("out", A),
                         kw.get("ws", A), kw.get("wsb", need), None]
    assert at(*args(batch=0)) == 0                                  # empty batch: no launch
    assert at(*args(q=None)) == 1
    assert at(*args(out=None)) == 1
    assert at(*args(k=None)) == 1
    assert at(*args(ws=None)) == 1
    assert at(*args(wsb=need - 4)) == 8
    assert at(*args(k=MIS)) == 7
    assert at(*args(hd=300)) == 2


def test_status_strings():
    lib = _lib.load()
    for code in range(10):
        assert lib.kvarn_status_str(code)
    assert lib.kvarn_status_str(42) == b"unknown status"


@pytest.mark.parametrize("name", ["quantize_tiles", "dequantize_tiles", "decode_attention",
                                  "quantize_tiles_to", "decode_attention_paged",
                                  "decode_attention_fp16"])
def test_python_api_refuses_cpu_tensors(name):
    import torch
    import kv_cache_bit_token_amd as kv
    x = torch.zeros(1, 128, 128, dtype=torch.float16)
    kc = torch.zeros(1, 8192, dtype=torch.uint8)
    vc = torch.zeros(1, 4096, dtype=torch.uint8)
    m = torch.zeros(1, 384, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU tensor"):
        if name == "quantize_tiles":
            kv.quantize_tiles(x, x)
        elif name == "dequantize_tiles":
            kv.dequantize_tiles(kc, vc, m, m, head_dim=128)
        elif name == "decode_attention":
            kv.decode_attention(torch.zeros(1, 4, 128, dtype=torch.float16), kc, vc, m, m,
                                n_kv_heads=1, tiles_per_seq=1)
        elif name == "quantize_tiles_to":
            kv.quantize_tiles_to(x, x, torch.zeros(1, dtype=torch.int64), kc.repeat(2, 1),
                                 vc.repeat(2, 1), m.repeat(2, 1), m.repeat(2, 1))
        elif name == "decode_attention_fp16":
            t = torch.zeros(1, 1, 128, 128, dtype=torch.float16)
            kv.decode_attention_fp16(torch.zeros(1, 4, 128, dtype=torch.float16), t, t)
        else:
            i = torch.zeros(1, 1, dtype=torch.int32)
            t = torch.zeros(1, 1, 128, 128, dtype=torch.float16)
            kv.decode_attention_paged(torch.zeros(1, 4, 128, dtype=torch.float16), kc, vc, m, m, i,
                                      i[0], i[0], t, t, n_kv_heads=1)


def test_grid_bounds_refused_on_the_host():
    """Counts that would not fit one launch grid come back as KVARN_E_SHAPE."""
    lib = _lib.load()
    ok = ctypes.byref(P())
    q = lib.kvarn_quantize_tiles
    assert q(ok, 1 << 30, A, A, A, A, A, A, None) == 6            # 2^30 tiles of K and of V
    assert q(ok, (1 << 30) - 1, None, None, None, None, None, None, None) == 0   # skipped: no launch
    nb = ctypes.c_size_t()
    ws = lib.kvarn_decode_attention_workspace
    assert ws(ok, 1 << 27, 32, 8, 0, ctypes.byref(nb)) == 6         # 2^32 (b, head) pairs
    assert ws(ok, 1 << 20, 32, 8, 1 << 10, ctypes.byref(nb)) == 6   # 2^33 tiles
    fws = lib.kvarn_decode_attention_fp16_workspace
    assert fws(128, 1 << 27, 32, 8, 128, ctypes.byref(nb)) == 6


def _api_cases():
    """(call, expected message) pairs: each passes one buffer whose size does
    not fit the packed layout or the shape the other arguments imply.  CPU
    tensors suffice: the binding checks sizes before anything touches a GPU."""
    import torch
    import kv_cache_bit_token_amd as kv
    f16, u8, i32 = torch.float16, torch.uint8, torch.int32
    x = torch.zeros(2, 128, 128, dtype=f16)
    c = lambda n, w=8192: torch.zeros(n, w, dtype=u8)
    vc = lambda n, w=4096: torch.zeros(n, w, dtype=u8)
    m = lambda n, w=384: torch.zeros(n, w, dtype=f16)
    q = torch.zeros(2, 8, 128, dtype=f16)
    t = torch.zeros(2, 2, 128, 128, dtype=f16)
    i = torch.zeros(2, 3, dtype=i32)
    n = torch.zeros(2, dtype=i32)
    return [
        (lambda: kv.quantize_tiles(x, x, out=(c(1), vc(2), m(2), m(2))), "k_codes must have 2 rows"),
        (lambda: kv.quantize_tiles(x, x, out=(c(2), vc(2, 8192), m(2), m(2))), "v_codes rows"),
        (lambda: kv.quantize_tiles(x, x, out=(c(2), vc(2), m(2, 320), m(2))), "k_meta rows"),
        (lambda: kv.quantize_tiles(x, None, out=(c(2), vc(2), m(2), None)), "v_codes must be given"),
        (lambda: kv.dequantize_tiles(c(2), vc(2), m(2), m(2), head_dim=64), "k_codes rows"),
        (lambda: kv.dequantize_tiles(c(2), vc(3), m(2), m(2), head_dim=128), "v_codes must have 2"),
        (lambda: kv.dequantize_tiles(c(2), vc(2), m(2), m(2), head_dim=128, k_bits=2), "k_codes rows"),
        (lambda: kv.dequantize_tiles(c(2), vc(2), m(2), None, head_dim=128), "v_codes and v_meta"),
        (lambda: kv.dequantize_tiles(c(2), vc(2), m(2), m(2), head_dim=128,
                                     out=(x[:, :, :96], x)), "k out must be"),
        (lambda: kv.decode_attention(q, c(5), vc(6), m(6), m(6), n_kv_heads=2, tiles_per_seq=3),
         "k_codes must have at least 12 rows"),
        (lambda: kv.decode_attention(q, c(12), vc(12), m(12), m(12, 300), n_kv_heads=2,
                                     tiles_per_seq=3), "v_meta rows"),
        (lambda: kv.decode_attention(q, c(12), vc(12), m(12), m(12), n_kv_heads=2, tiles_per_seq=3,
                                     out=torch.zeros(2, 8, 64)), "out must be"),
        (lambda: kv.quantize_tiles_to(x, x, torch.zeros(2, dtype=torch.int64), c(4), vc(3), m(4),
                                      m(4)), "v_codes must have 4 rows"),
        (lambda: kv.quantize_tiles_to(x, x, torch.zeros(2, dtype=torch.int64), c(4), vc(4), m(4),
                                      m(4, 100)), "v_meta rows"),
        (lambda: kv.decode_attention_paged(q, c(6), vc(6), m(5), m(6), i, n, n, t, t, n_kv_heads=2),
         "k_meta must have 6 rows"),
        (lambda: kv.decode_attention_paged(q, c(5), vc(5), m(5), m(5), i, n, n, t, t, n_kv_heads=2),
         "pool rows"),
        (lambda: kv.decode_attention_fp16(q, t, t, out=torch.zeros(2, 4, 128)), "out must be"),
    ]


def test_python_api_checks_buffer_sizes_on_the_host():
    for call, msg in _api_cases():
        with pytest.raises(ValueError, match=msg):
            call()
