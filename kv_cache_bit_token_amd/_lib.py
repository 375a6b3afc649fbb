"""ctypes declarations of include/kvarn.h (libkvarn.so)."""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvarn.so")

# Every symbol include/kvarn.h declares, with (restype, argtypes).
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class Params(ctypes.Structure):
    _fields_ = [("head_dim", _i32), ("tile_tokens", _i32), ("k_bits", _i32),
                ("v_bits", _i32), ("n_iters", _i32)]


class TileLayout(ctypes.Structure):
    _fields_ = [("padded_dim", _i32), ("k_code_bytes", _i64), ("v_code_bytes", _i64),
                ("k_meta_bytes", _i64), ("v_meta_bytes", _i64)]


_P = ctypes.POINTER(Params)
SIGNATURES = {
    "kvarn_get_layout": (ctypes.c_int, [_P, ctypes.POINTER(TileLayout)]),
    "kvarn_params_from_preset": (ctypes.c_int, [ctypes.c_char_p, _i32, _i32, _P]),
    "kvarn_quantize_tiles": (ctypes.c_int, [_P, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "kvarn_dequantize_tiles": (ctypes.c_int, [_P, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "kvarn_decode_attention_workspace": (ctypes.c_int, [_P, _i32, _i32, _i32, _i32,
                                                        ctypes.POINTER(ctypes.c_size_t)]),
    "kvarn_decode_attention": (ctypes.c_int, [_P, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                              _vp, ctypes.c_float, _vp, _vp, ctypes.c_size_t,
                                              _vp]),
    "kvarn_decode_attention_noalloc": (ctypes.c_int, [_P, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                                      _vp, _vp, ctypes.c_float, _vp, _vp]),
    "kvarn_quantize_tiles_to": (ctypes.c_int, [_P, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp,
                                               _vp]),
    "kvarn_decode_attention_paged_workspace": (ctypes.c_int, [_P, _i32, _i32, _i32, _i32,
                                                              ctypes.POINTER(ctypes.c_size_t)]),
    "kvarn_decode_attention_paged": (ctypes.c_int, [_P, _i32, _i32, _i32, _i32, _i64, _vp, _vp,
                                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                    ctypes.c_float, _vp, _vp, ctypes.c_size_t,
                                                    _vp]),
    "kvarn_decode_attention_fp16_workspace": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i64,
                                                             ctypes.POINTER(ctypes.c_size_t)]),
    "kvarn_decode_attention_fp16": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp,
                                                   ctypes.c_float, _vp, _vp, ctypes.c_size_t, _vp]),
    "kvarn_status_str": (ctypes.c_char_p, [ctypes.c_int]),
}

STATUS = {0: "KVARN_OK", 1: "KVARN_E_NULL", 2: "KVARN_E_HEAD_DIM", 3: "KVARN_E_TILE",
          4: "KVARN_E_BITS", 5: "KVARN_E_ITERS", 6: "KVARN_E_SHAPE", 7: "KVARN_E_ALIGN",
          8: "KVARN_E_WORKSPACE", 9: "KVARN_E_HIP"}

_lib = None


def load():
    """Load libkvarn.so; raise loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libkvarn.so is not built (run __graft_entry__.build() or "
                           "python -m kv_cache_bit_token_amd.build); there is no fallback")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
