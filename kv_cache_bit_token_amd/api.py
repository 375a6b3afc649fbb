"""Python binding of libkvarn.so, same names as the C ABI.

Argument marshalling only: every step of the path runs in the HIP kernels
behind include/kvarn.h.  torch supplies device memory (outputs are allocated
with torch on the inputs' device) and the stream (the current stream).  All
tensors must be CUDA (ROCm) tensors; there is no CPU fallback.
"""
import ctypes

import torch

from . import _lib

TILE = 128


class KvarnError(RuntimeError):
    def __init__(self, fn, status):
        lib = _lib.load()
        msg = lib.kvarn_status_str(status).decode()
        super().__init__("%s failed: %s (%s)" % (fn, _lib.STATUS.get(status, status), msg))
        self.status = status


def _check(fn, st):
    if st != 0:
        raise KvarnError(fn, st)


def _params(head_dim, k_bits, v_bits, n_iters, tile_tokens=TILE):
    return _lib.Params(int(head_dim), int(tile_tokens), int(k_bits), int(v_bits), int(n_iters))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_gpu(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (the KVarN path has no CPU fallback)" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))


def _same_device(ref, *ts):
    for t, name in ts:
        if t is not None and t.device != ref.device:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, ref.device))


def _rows(t, name, rows, width, exact=True):
    """t must be [rows, ...] with `width` elements per row (at least `rows`
    rows when exact is False).  The C ABI sees only pointers, so this is the
    one place where a buffer too small for the layout is caught."""
    if t is None or (rows == 0 and not exact):   # nothing will be read
        return
    if t.dim() < 1 or (t.shape[0] != rows if exact else t.shape[0] < rows):
        raise ValueError("%s must have %s%d rows (got shape %s)"
                         % (name, "" if exact else "at least ", rows, tuple(t.shape)))
    if t.numel() != t.shape[0] * width:
        raise ValueError("%s rows must hold %d elements of the packed layout (got shape %s)"
                         % (name, width, tuple(t.shape)))


def _shape(t, name, shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must be %s (got %s)" % (name, tuple(shape), tuple(t.shape)))


def _cache_rows(k_codes, v_codes, k_meta, v_meta, lay, rows, exact):
    _rows(k_codes, "k_codes", rows, lay["k_code_bytes"], exact)
    _rows(v_codes, "v_codes", rows, lay["v_code_bytes"], exact)
    _rows(k_meta, "k_meta", rows, lay["k_meta_bytes"] // 2, exact)
    _rows(v_meta, "v_meta", rows, lay["v_meta_bytes"] // 2, exact)


def get_layout(head_dim, k_bits=4, v_bits=2, n_iters=5):
    """Per-tile sizes of the packed format (host only)."""
    lib = _lib.load()
    p = _params(head_dim, k_bits, v_bits, n_iters)
    lay = _lib.TileLayout()
    _check("kvarn_get_layout", lib.kvarn_get_layout(ctypes.byref(p), ctypes.byref(lay)))
    return {"padded_dim": lay.padded_dim, "k_code_bytes": lay.k_code_bytes,
            "v_code_bytes": lay.v_code_bytes, "k_meta_bytes": lay.k_meta_bytes,
            "v_meta_bytes": lay.v_meta_bytes}


def params_from_preset(preset, head_dim, n_iters=5):
    """Parse e.g. 'kvarn_k4v2_g128' -> dict(head_dim, tile_tokens, k_bits, v_bits, n_iters)."""
    lib = _lib.load()
    p = _lib.Params()
    _check("kvarn_params_from_preset",
           lib.kvarn_params_from_preset(preset.encode(), int(head_dim), int(n_iters), ctypes.byref(p)))
    return {"head_dim": p.head_dim, "tile_tokens": p.tile_tokens, "k_bits": p.k_bits,
            "v_bits": p.v_bits, "n_iters": p.n_iters}


def quantize_tiles(k, v, *, k_bits=4, v_bits=2, n_iters=5, out=None):
    """Quantise fp16 K and V tiles.

    k, v: torch.float16 GPU tensors whose trailing dims are [128, head_dim]
    (all leading dims are tiles); either may be None to skip that tensor.
    Returns (k_codes, v_codes, k_meta, v_meta): uint8 [n_tiles, code_bytes]
    and float16 [n_tiles, meta_halves] (None for a skipped tensor).  `out`
    may pass preallocated outputs in the same order.
    """
    ref = k if k is not None else v
    if ref is None:
        raise ValueError("nothing to quantise")
    head_dim = ref.shape[-1]
    n_tiles = ref.numel() // (TILE * head_dim)
    for t, name in ((k, "k"), (v, "v")):
        if t is not None and (t.dim() < 2 or t.shape[-2] != TILE
                              or t.numel() != n_tiles * TILE * head_dim):
            raise ValueError("%s must be [..., 128, head_dim] with the same tile count" % name)
    lay = get_layout(head_dim, k_bits, v_bits, n_iters)
    if out is not None:
        kc, vc, km, vm = out
        for t, name, x in ((kc, "k_codes", k), (km, "k_meta", k), (vc, "v_codes", v),
                           (vm, "v_meta", v)):
            if (t is None) != (x is None):
                raise ValueError("out: %s must be given exactly when its input is" % name)
        _cache_rows(kc, vc, km, vm, lay, n_tiles, True)
    for t, name in ((k, "k"), (v, "v")):
        _need_gpu(t, name, torch.float16)
    dev = ref.device
    if out is None:
        kc = torch.empty((n_tiles, lay["k_code_bytes"]), dtype=torch.uint8, device=dev) if k is not None else None
        vc = torch.empty((n_tiles, lay["v_code_bytes"]), dtype=torch.uint8, device=dev) if v is not None else None
        km = torch.empty((n_tiles, lay["k_meta_bytes"] // 2), dtype=torch.float16, device=dev) if k is not None else None
        vm = torch.empty((n_tiles, lay["v_meta_bytes"] // 2), dtype=torch.float16, device=dev) if v is not None else None
    else:
        for t, name in ((kc, "k_codes"), (vc, "v_codes")):
            _need_gpu(t, name, torch.uint8)
        for t, name in ((km, "k_meta"), (vm, "v_meta")):
            _need_gpu(t, name, torch.float16)
    _same_device(ref, (k, "k"), (v, "v"), (kc, "k_codes"), (vc, "v_codes"), (km, "k_meta"),
                 (vm, "v_meta"))
    lib = _lib.load()
    p = _params(head_dim, k_bits, v_bits, n_iters)
    st = lib.kvarn_quantize_tiles(ctypes.byref(p), n_tiles, _ptr(k), _ptr(v), _ptr(kc), _ptr(vc),
                                  _ptr(km), _ptr(vm), _stream(dev))
    _check("kvarn_quantize_tiles", st)
    return kc, vc, km, vm


def dequantize_tiles(k_codes, v_codes, k_meta, v_meta, *, head_dim, k_bits=4, v_bits=2,
                     out=None):
    """Inverse of quantize_tiles -> (k, v) torch.float16 [n_tiles, 128, head_dim]."""
    ref = k_codes if k_codes is not None else v_codes
    if ref is None:
        raise ValueError("nothing to dequantise")
    n_tiles = ref.shape[0]
    for c, m, name in ((k_codes, k_meta, "k"), (v_codes, v_meta, "v")):
        if (c is None) != (m is None):
            raise ValueError("%s_codes and %s_meta must both be given or both be None" % (name, name))
    lay = get_layout(head_dim, k_bits, v_bits, 0)
    _cache_rows(k_codes, v_codes, k_meta, v_meta, lay, n_tiles, True)
    if out is not None:
        ko, vo = out
        for t, name, x in ((ko, "k out", k_codes), (vo, "v out", v_codes)):
            if (t is None) != (x is None):
                raise ValueError("out: %s must be given exactly when its codes are" % name)
            _shape(t, name, (n_tiles, TILE, head_dim))
    for t, name in ((k_codes, "k_codes"), (v_codes, "v_codes")):
        _need_gpu(t, name, torch.uint8)
    for t, name in ((k_meta, "k_meta"), (v_meta, "v_meta")):
        _need_gpu(t, name, torch.float16)
    dev = ref.device
    if out is None:
        ko = torch.empty((n_tiles, TILE, head_dim), dtype=torch.float16, device=dev) if k_codes is not None else None
        vo = torch.empty((n_tiles, TILE, head_dim), dtype=torch.float16, device=dev) if v_codes is not None else None
    else:
        _need_gpu(ko, "k out", torch.float16)
        _need_gpu(vo, "v out", torch.float16)
    _same_device(ref, (k_codes, "k_codes"), (v_codes, "v_codes"), (k_meta, "k_meta"),
                 (v_meta, "v_meta"), (ko, "k out"), (vo, "v out"))
    lib = _lib.load()
    p = _params(head_dim, k_bits, v_bits, 0)
    st = lib.kvarn_dequantize_tiles(ctypes.byref(p), n_tiles, _ptr(k_codes), _ptr(v_codes),
                                    _ptr(k_meta), _ptr(v_meta), _ptr(ko), _ptr(vo), _stream(dev))
    _check("kvarn_dequantize_tiles", st)
    return ko, vo


def decode_attention_workspace(*, batch, n_q_heads, n_kv_heads, tiles_per_seq, head_dim,
                               k_bits=4, v_bits=2):
    lib = _lib.load()
    p = _params(head_dim, k_bits, v_bits, 0)
    nb = ctypes.c_size_t()
    _check("kvarn_decode_attention_workspace",
           lib.kvarn_decode_attention_workspace(ctypes.byref(p), int(batch), int(n_q_heads),
                                                int(n_kv_heads), int(tiles_per_seq),
                                                ctypes.byref(nb)))
    return nb.value


def decode_attention(q, k_codes, v_codes, k_meta, v_meta, *, n_kv_heads, tiles_per_seq,
                     k_bits=4, v_bits=2, sm_scale=None, workspace=None, out=None):
    """One decode step over the packed cache.

    q: torch.float16 [batch, n_q_heads, head_dim]; cache tile i of (b, g) at
    row (b * n_kv_heads + g) * tiles_per_seq + i of the code/meta tensors
    (each with at least batch * n_kv_heads * tiles_per_seq rows).
    Returns float32 [batch, n_q_heads, head_dim].
    """
    if q.dim() != 3:
        raise ValueError("q must be [batch, n_q_heads, head_dim]")
    batch, hq, head_dim = q.shape
    lay = get_layout(head_dim, k_bits, v_bits, 0)
    _cache_rows(k_codes, v_codes, k_meta, v_meta, lay,
                int(batch) * int(n_kv_heads) * int(tiles_per_seq), False)
    _shape(out, "out", (batch, hq, head_dim))
    _need_gpu(q, "q", torch.float16)
    for t, name in ((k_codes, "k_codes"), (v_codes, "v_codes")):
        _need_gpu(t, name, torch.uint8)
    for t, name in ((k_meta, "k_meta"), (v_meta, "v_meta")):
        _need_gpu(t, name, torch.float16)
    _need_gpu(out, "out", torch.float32)
    _need_gpu(workspace, "workspace")
    _same_device(q, (k_codes, "k_codes"), (v_codes, "v_codes"), (k_meta, "k_meta"),
                 (v_meta, "v_meta"), (out, "out"), (workspace, "workspace"))
    if sm_scale is None:
        sm_scale = head_dim ** -0.5
    nbytes = decode_attention_workspace(batch=batch, n_q_heads=hq, n_kv_heads=n_kv_heads,
                                        tiles_per_seq=tiles_per_seq, head_dim=head_dim,
                                        k_bits=k_bits, v_bits=v_bits)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((batch, hq, head_dim), dtype=torch.float32, device=q.device)
    lib = _lib.load()
    p = _params(head_dim, k_bits, v_bits, 0)
    st = lib.kvarn_decode_attention(ctypes.byref(p), batch, hq, int(n_kv_heads), int(tiles_per_seq),
                                    _ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_meta),
                                    _ptr(v_meta), float(sm_scale), _ptr(out), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(q.device))
    _check("kvarn_decode_attention", st)
    return out


def decode_attention_noalloc(q, k_codes, v_codes, k_meta, v_meta, out, *, n_kv_heads,
                             tiles_per_seq, k_bits=4, v_bits=2, sm_scale=None):
    """decode_attention with its scratch in the library's static device buffer:
    allocates nothing (no workspace; `out`, float32 [batch, n_q_heads,
    head_dim], is required).  Shapes whose workspace exceeds the static
    buffer (64 MiB) are refused; calls that overlap on one GPU race."""
    if q.dim() != 3:
        raise ValueError("q must be [batch, n_q_heads, head_dim]")
    batch, hq, head_dim = q.shape
    lay = get_layout(head_dim, k_bits, v_bits, 0)
    _cache_rows(k_codes, v_codes, k_meta, v_meta, lay,
                int(batch) * int(n_kv_heads) * int(tiles_per_seq), False)
    if out is None:
        raise ValueError("out is required (this entry point allocates nothing)")
    _shape(out, "out", (batch, hq, head_dim))
    _need_gpu(q, "q", torch.float16)
    for t, name in ((k_codes, "k_codes"), (v_codes, "v_codes")):
        _need_gpu(t, name, torch.uint8)
    for t, name in ((k_meta, "k_meta"), (v_meta, "v_meta")):
        _need_gpu(t, name, torch.float16)
    _need_gpu(out, "out", torch.float32)
    _same_device(q, (k_codes, "k_codes"), (v_codes, "v_codes"), (k_meta, "k_meta"),
                 (v_meta, "v_meta"), (out, "out"))
    if sm_scale is None:
        sm_scale = head_dim ** -0.5
    lib = _lib.load()
    p = _params(head_dim, k_bits, v_bits, 0)
    st = lib.kvarn_decode_attention_noalloc(ctypes.byref(p), batch, hq, int(n_kv_heads),
                                            int(tiles_per_seq), _ptr(q), _ptr(k_codes),
                                            _ptr(v_codes), _ptr(k_meta), _ptr(v_meta),
                                            float(sm_scale), _ptr(out), _stream(q.device))
    _check("kvarn_decode_attention_noalloc", st)
    return out


def quantize_tiles_to(k, v, dst_tile, k_codes, v_codes, k_meta, v_meta, *, k_bits=4, v_bits=2,
                      n_iters=5):
    """Quantise fp16 K and V tiles into chosen slots of a tile pool.

    k, v: torch.float16 GPU tensors [..., 128, head_dim] (either may be None);
    dst_tile: torch.int64 GPU tensor [n_tiles], the pool slot of each input
    tile (slots outside the pool skip their tile); k_codes .. v_meta: the pool
    tensors, [pool_tiles, ...] as returned by quantize_tiles, written in place
    (those of a skipped tensor are ignored).
    """
    ref = k if k is not None else v
    if ref is None:
        raise ValueError("nothing to quantise")
    head_dim = ref.shape[-1]
    n_tiles = ref.numel() // (TILE * head_dim)
    for t, name in ((k, "k"), (v, "v")):
        if t is not None and (t.dim() < 2 or t.shape[-2] != TILE
                              or t.numel() != n_tiles * TILE * head_dim):
            raise ValueError("%s must be [..., 128, head_dim] with the same tile count" % name)
    if dst_tile.numel() != n_tiles:
        raise ValueError("dst_tile needs one entry per input tile")
    kc, km = (k_codes, k_meta) if k is not None else (None, None)
    vc, vm = (v_codes, v_meta) if v is not None else (None, None)
    for t, name in ((kc, "k_codes"), (km, "k_meta"), (vc, "v_codes"), (vm, "v_meta")):
        if t is None and (k if name[0] == "k" else v) is not None:
            raise ValueError("%s pool is needed for the given %s tiles" % (name, name[0]))
    pool = (kc if kc is not None else vc).shape[0]
    lay = get_layout(head_dim, k_bits, v_bits, n_iters)
    _cache_rows(kc, vc, km, vm, lay, pool, True)
    for t, name in ((k, "k"), (v, "v")):
        _need_gpu(t, name, torch.float16)
    _need_gpu(dst_tile, "dst_tile", torch.int64)
    for t, name in ((kc, "k_codes"), (vc, "v_codes")):
        _need_gpu(t, name, torch.uint8)
    for t, name in ((km, "k_meta"), (vm, "v_meta")):
        _need_gpu(t, name, torch.float16)
    _same_device(ref, (k, "k"), (v, "v"), (dst_tile, "dst_tile"), (kc, "k_codes"),
                 (vc, "v_codes"), (km, "k_meta"), (vm, "v_meta"))
    lib = _lib.load()
    p = _params(head_dim, k_bits, v_bits, n_iters)
    st = lib.kvarn_quantize_tiles_to(ctypes.byref(p), n_tiles, _ptr(k), _ptr(v), _ptr(dst_tile),
                                     int(pool), _ptr(kc), _ptr(vc), _ptr(km), _ptr(vm),
                                     _stream(ref.device))
    _check("kvarn_quantize_tiles_to", st)


def decode_attention_paged_workspace(*, batch, n_q_heads, n_kv_heads, max_blocks, head_dim,
                                     k_bits=4, v_bits=2):
    lib = _lib.load()
    p = _params(head_dim, k_bits, v_bits, 0)
    nb = ctypes.c_size_t()
    _check("kvarn_decode_attention_paged_workspace",
           lib.kvarn_decode_attention_paged_workspace(ctypes.byref(p), int(batch), int(n_q_heads),
                                                      int(n_kv_heads), int(max_blocks),
                                                      ctypes.byref(nb)))
    return nb.value


def decode_attention_paged(q, k_codes, v_codes, k_meta, v_meta, block_table, n_blocks, tail_len,
                           k_tail, v_tail, *, n_kv_heads, k_bits=4, v_bits=2, sm_scale=None,
                           workspace=None, out=None):
    """One decode step over a paged packed cache plus an fp16 tail.

    q: float16 [batch, n_q_heads, head_dim]; block_table: int32
    [batch, max_blocks] (physical block p holds pool tiles p * n_kv_heads + g);
    n_blocks, tail_len: int32 [batch]; k_tail, v_tail: float16
    [batch, n_kv_heads, 128, head_dim]; pool tensors as from quantize_tiles
    with pool_blocks * n_kv_heads rows.  Returns float32 [batch, n_q_heads, head_dim].
    """
    if q.dim() != 3:
        raise ValueError("q must be [batch, n_q_heads, head_dim]")
    batch, hq, head_dim = q.shape
    if block_table.dim() != 2:
        raise ValueError("block_table must be [batch, max_blocks]")
    max_blocks = block_table.shape[1]
    if block_table.shape[0] != batch or n_blocks.numel() != batch or tail_len.numel() != batch:
        raise ValueError("block_table, n_blocks and tail_len need one row per sequence")
    if tuple(k_tail.shape) != (batch, n_kv_heads, TILE, head_dim) or k_tail.shape != v_tail.shape:
        raise ValueError("k_tail, v_tail must be [batch, n_kv_heads, 128, head_dim]")
    if k_codes.shape[0] % int(n_kv_heads) != 0:
        raise ValueError("pool rows must be pool_blocks * n_kv_heads")
    pool_blocks = k_codes.shape[0] // n_kv_heads
    lay = get_layout(head_dim, k_bits, v_bits, 0)
    _cache_rows(k_codes, v_codes, k_meta, v_meta, lay, pool_blocks * int(n_kv_heads), True)
    _shape(out, "out", (batch, hq, head_dim))
    _need_gpu(q, "q", torch.float16)
    for t, name in ((k_codes, "k_codes"), (v_codes, "v_codes")):
        _need_gpu(t, name, torch.uint8)
    for t, name in ((k_meta, "k_meta"), (v_meta, "v_meta"), (k_tail, "k_tail"), (v_tail, "v_tail")):
        _need_gpu(t, name, torch.float16)
    for t, name in ((block_table, "block_table"), (n_blocks, "n_blocks"), (tail_len, "tail_len")):
        _need_gpu(t, name, torch.int32)
    _need_gpu(out, "out", torch.float32)
    _need_gpu(workspace, "workspace")
    _same_device(q, (k_codes, "k_codes"), (v_codes, "v_codes"), (k_meta, "k_meta"),
                 (v_meta, "v_meta"), (block_table, "block_table"), (n_blocks, "n_blocks"),
                 (tail_len, "tail_len"), (k_tail, "k_tail"), (v_tail, "v_tail"), (out, "out"),
                 (workspace, "workspace"))
    if sm_scale is None:
        sm_scale = head_dim ** -0.5
    nbytes = decode_attention_paged_workspace(batch=batch, n_q_heads=hq, n_kv_heads=n_kv_heads,
                                              max_blocks=max_blocks, head_dim=head_dim,
                                              k_bits=k_bits, v_bits=v_bits)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((batch, hq, head_dim), dtype=torch.float32, device=q.device)
    lib = _lib.load()
    p = _params(head_dim, k_bits, v_bits, 0)
    st = lib.kvarn_decode_attention_paged(
        ctypes.byref(p), batch, hq, int(n_kv_heads), int(max_blocks), int(pool_blocks),
        _ptr(block_table), _ptr(n_blocks), _ptr(tail_len), _ptr(q), _ptr(k_codes), _ptr(v_codes),
        _ptr(k_meta), _ptr(v_meta), _ptr(k_tail), _ptr(v_tail), float(sm_scale), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q.device))
    _check("kvarn_decode_attention_paged", st)
    return out


def decode_attention_fp16_workspace(*, batch, n_q_heads, n_kv_heads, seq_len, head_dim):
    lib = _lib.load()
    nb = ctypes.c_size_t()
    _check("kvarn_decode_attention_fp16_workspace",
           lib.kvarn_decode_attention_fp16_workspace(int(head_dim), int(batch), int(n_q_heads),
                                                     int(n_kv_heads), int(seq_len), ctypes.byref(nb)))
    return nb.value


def decode_attention_fp16(q, k, v, *, sm_scale=None, workspace=None, out=None):
    """One decode step over an uncompressed fp16 cache (the baseline).

    q: float16 [batch, n_q_heads, head_dim]; k, v: float16
    [batch, n_kv_heads, seq_len, head_dim].  Returns float32 [batch, n_q_heads, head_dim].
    """
    if q.dim() != 3:
        raise ValueError("q must be [batch, n_q_heads, head_dim]")
    if k.dim() != 4 or k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[2]:
        raise ValueError("k, v must be [batch, n_kv_heads, seq_len, head_dim] matching q")
    batch, hq, head_dim = q.shape
    _shape(out, "out", (batch, hq, head_dim))
    _need_gpu(q, "q", torch.float16)
    _need_gpu(k, "k", torch.float16)
    _need_gpu(v, "v", torch.float16)
    _need_gpu(out, "out", torch.float32)
    _need_gpu(workspace, "workspace")
    _same_device(q, (k, "k"), (v, "v"), (out, "out"), (workspace, "workspace"))
    n_kv, seq_len = k.shape[1], k.shape[2]
    if sm_scale is None:
        sm_scale = head_dim ** -0.5
    nbytes = decode_attention_fp16_workspace(batch=batch, n_q_heads=hq, n_kv_heads=n_kv,
                                             seq_len=seq_len, head_dim=head_dim)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((batch, hq, head_dim), dtype=torch.float32, device=q.device)
    lib = _lib.load()
    st = lib.kvarn_decode_attention_fp16(
        int(head_dim), batch, hq, int(n_kv), int(seq_len), _ptr(q), _ptr(k), _ptr(v),
        float(sm_scale), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(q.device))
    _check("kvarn_decode_attention_fp16", st)
    return out
