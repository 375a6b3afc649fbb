"""KVarN KV-cache quantiser hot path for MI355X (gfx950).

The compute lives in the C-ABI library libkvarn.so (hand-written HIP
kernels); this package is its thin Python binding.  Importing the package is
cheap; the shared library is loaded on first use of the API, and every API
call fails loudly if the library (or a GPU) is missing -- there is no CPU
fallback.
"""

__all__ = [
    "quantize_tiles", "dequantize_tiles", "decode_attention",
    "decode_attention_workspace", "get_layout", "params_from_preset", "KvarnError",
    "quantize_tiles_to", "decode_attention_paged", "decode_attention_paged_workspace",
    "decode_attention_fp16", "decode_attention_fp16_workspace", "decode_attention_noalloc",
]


def __getattr__(name):
    if name in __all__:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
