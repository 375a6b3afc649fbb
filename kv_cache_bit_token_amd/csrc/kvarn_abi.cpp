// kvarn_abi.cpp -- the C ABI of include/kvarn.h: argument validation (host,
// before any HIP call), layout arithmetic, and the launches.
#include "kvarn.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "kvarn_internal.hpp"

namespace {

constexpr int TILE = 128;

kvarn_status check_params(const kvarn_params* p, int* D) {
    if (!p) return KVARN_E_NULL;
    if (p->tile_tokens != TILE) return KVARN_E_TILE;
    if (p->head_dim < 33 || p->head_dim > 256 || (p->head_dim % 8) != 0) return KVARN_E_HEAD_DIM;
    if ((p->k_bits != 2 && p->k_bits != 4) || (p->v_bits != 2 && p->v_bits != 4)) return KVARN_E_BITS;
    if (p->n_iters < 0 || p->n_iters > 16) return KVARN_E_ITERS;
    int d = 64;
    while (d < p->head_dim) d *= 2;
    *D = d;
    return KVARN_OK;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// A pointer set is all NULL (skip: returns 0), all set (returns 1) or mixed (-1).
int pointer_set(const void* a, const void* b, const void* c) {
    const int n = (a != nullptr) + (b != nullptr) + (c != nullptr);
    return n == 0 ? 0 : (n == 3 ? 1 : -1);
}

int64_t code_bytes(int D, int bits) { return (int64_t)TILE * D * bits / 8; }

// Largest tile count one launch grid can hold (K and V share the grid, whose
// x dimension holds at most 2^31 - 1 workgroups).
constexpr int64_t kMaxTiles = ((int64_t)1 << 30) - 1;

}  // namespace

extern "C" {

const char* kvarn_status_str(kvarn_status s) {
    switch (s) {
        case KVARN_OK: return "ok";
        case KVARN_E_NULL: return "null pointer or partly null pointer set";
        case KVARN_E_HEAD_DIM: return "head_dim must be 33..256 and a multiple of 8";
        case KVARN_E_TILE: return "tile_tokens must be 128";
        case KVARN_E_BITS: return "k_bits and v_bits must be 2 or 4";
        case KVARN_E_ITERS: return "n_iters must be 0..16";
        case KVARN_E_SHAPE: return "invalid count or head grouping";
        case KVARN_E_ALIGN: return "device pointers must be 16-byte aligned";
        case KVARN_E_WORKSPACE: return "attention workspace (or the static scratch) too small for this shape";
        case KVARN_E_HIP: return "HIP runtime error at launch";
    }
    return "unknown status";
}

kvarn_status kvarn_get_layout(const kvarn_params* params, kvarn_tile_layout* layout) {
    if (!layout) return KVARN_E_NULL;
    int D = 0;
    kvarn_status st = check_params(params, &D);
    if (st != KVARN_OK) return st;
    layout->padded_dim = D;
    layout->k_code_bytes = code_bytes(D, params->k_bits);
    layout->v_code_bytes = code_bytes(D, params->v_bits);
    layout->k_meta_bytes = 2 * (2 * D + TILE);
    layout->v_meta_bytes = 2 * (2 * TILE + D);
    return KVARN_OK;
}

kvarn_status kvarn_params_from_preset(const char* preset, int32_t head_dim, int32_t n_iters,
                                      kvarn_params* params) {
    if (!preset || !params) return KVARN_E_NULL;
    // exact form: "kvarn_k<digit>v<digit>_g<digits>"
    const char* pre = "kvarn_k";
    if (strncmp(preset, pre, strlen(pre)) != 0) return KVARN_E_BITS;
    const char* s = preset + strlen(pre);
    if (s[0] < '0' || s[0] > '9' || s[1] != 'v' || s[2] < '0' || s[2] > '9' || s[3] != '_' ||
        s[4] != 'g')
        return KVARN_E_BITS;
    const int kb = s[0] - '0', vb = s[2] - '0';
    long g = 0;
    const char* q = s + 5;
    if (*q == '\0') return KVARN_E_TILE;
    for (; *q; ++q) {
        if (*q < '0' || *q > '9' || g > 100000) return KVARN_E_TILE;
        g = g * 10 + (*q - '0');
    }
    kvarn_params p;
    p.head_dim = head_dim;
    p.tile_tokens = (int32_t)g;
    p.k_bits = kb;
    p.v_bits = vb;
    p.n_iters = n_iters;
    int D = 0;
    kvarn_status st = check_params(&p, &D);
    if (st != KVARN_OK) return st;
    *params = p;
    return KVARN_OK;
}

kvarn_status kvarn_quantize_tiles(const kvarn_params* params, int64_t n_tiles, const void* k_fp16,
                                  const void* v_fp16, void* k_codes, void* v_codes, void* k_meta,
                                  void* v_meta, void* stream) {
    int D = 0;
    kvarn_status st = check_params(params, &D);
    if (st != KVARN_OK) return st;
    const int ks = pointer_set(k_fp16, k_codes, k_meta);
    const int vs = pointer_set(v_fp16, v_codes, v_meta);
    if (ks < 0 || vs < 0) return KVARN_E_NULL;
    if (n_tiles < 0 || n_tiles > kMaxTiles) return KVARN_E_SHAPE;
    if (misaligned(k_fp16) || misaligned(v_fp16) || misaligned(k_codes) || misaligned(v_codes) ||
        misaligned(k_meta) || misaligned(v_meta))
        return KVARN_E_ALIGN;
    if (n_tiles == 0 || (ks == 0 && vs == 0)) return KVARN_OK;

    kvarn::QuantArgs a;
    a.k = static_cast<const uint16_t*>(k_fp16);
    a.v = static_cast<const uint16_t*>(v_fp16);
    a.kc = static_cast<uint8_t*>(k_codes);
    a.vc = static_cast<uint8_t*>(v_codes);
    a.km = static_cast<uint16_t*>(k_meta);
    a.vm = static_cast<uint16_t*>(v_meta);
    a.n_k = ks ? n_tiles : 0;
    a.n_v = vs ? n_tiles : 0;
    a.d0 = params->head_dim;
    a.n_iters = params->n_iters;
    hipError_t e = kvarn::launch_quantize(a, D, params->k_bits, params->v_bits,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVARN_OK : KVARN_E_HIP;
}

kvarn_status kvarn_dequantize_tiles(const kvarn_params* params, int64_t n_tiles,
                                    const void* k_codes, const void* v_codes, const void* k_meta,
                                    const void* v_meta, void* k_out, void* v_out, void* stream) {
    int D = 0;
    kvarn_status st = check_params(params, &D);
    if (st != KVARN_OK) return st;
    const int ks = pointer_set(k_codes, k_meta, k_out);
    const int vs = pointer_set(v_codes, v_meta, v_out);
    if (ks < 0 || vs < 0) return KVARN_E_NULL;
    if (n_tiles < 0 || n_tiles > kMaxTiles) return KVARN_E_SHAPE;
    if (misaligned(k_codes) || misaligned(v_codes) || misaligned(k_meta) || misaligned(v_meta) ||
        misaligned(k_out) || misaligned(v_out))
        return KVARN_E_ALIGN;
    if (n_tiles == 0 || (ks == 0 && vs == 0)) return KVARN_OK;

    kvarn::DequantArgs a;
    a.kc = static_cast<const uint8_t*>(k_codes);
    a.vc = static_cast<const uint8_t*>(v_codes);
    a.km = static_cast<const uint16_t*>(k_meta);
    a.vm = static_cast<const uint16_t*>(v_meta);
    a.ko = static_cast<uint16_t*>(k_out);
    a.vo = static_cast<uint16_t*>(v_out);
    a.n_k = ks ? n_tiles : 0;
    a.n_v = vs ? n_tiles : 0;
    a.d0 = params->head_dim;
    hipError_t e = kvarn::launch_dequantize(a, D, params->k_bits, params->v_bits,
                                            static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVARN_OK : KVARN_E_HIP;
}

static kvarn_status check_attention_shape(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                          int32_t tiles_per_seq) {
    if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || tiles_per_seq < 0)
        return KVARN_E_SHAPE;
    if (n_q_heads % n_kv_heads != 0) return KVARN_E_SHAPE;
    if (n_q_heads / n_kv_heads > 16) return KVARN_E_SHAPE;   // GQA group of at most 16 heads
    if ((int64_t)batch * n_q_heads > INT32_MAX) return KVARN_E_SHAPE;   // one workgroup per (b, head)
    if ((int64_t)batch * n_kv_heads * tiles_per_seq > kMaxTiles) return KVARN_E_SHAPE;
    return KVARN_OK;
}

kvarn_status kvarn_decode_attention_workspace(const kvarn_params* params, int32_t batch,
                                              int32_t n_q_heads, int32_t n_kv_heads,
                                              int32_t tiles_per_seq, size_t* bytes) {
    if (!bytes) return KVARN_E_NULL;
    int D = 0;
    kvarn_status st = check_params(params, &D);
    if (st != KVARN_OK) return st;
    st = check_attention_shape(batch, n_q_heads, n_kv_heads, tiles_per_seq);
    if (st != KVARN_OK) return st;
    const int ns = kvarn::attention_splits(batch, n_kv_heads, tiles_per_seq);
    *bytes = kvarn::attention_workspace_bytes(batch, n_q_heads, D, ns);
    return KVARN_OK;
}

}  // extern "C"

namespace {

// Shared by kvarn_decode_attention (caller's workspace) and
// kvarn_decode_attention_noalloc (the library's static scratch: workspace ==
// nullptr and use_static set).
kvarn_status decode_attention_impl(const kvarn_params* params, int32_t batch, int32_t n_q_heads,
                                   int32_t n_kv_heads, int32_t tiles_per_seq, const void* q_fp16,
                                   const void* k_codes, const void* v_codes, const void* k_meta,
                                   const void* v_meta, float sm_scale, float* out, void* workspace,
                                   size_t workspace_bytes, bool use_static, void* stream) {
    int D = 0;
    kvarn_status st = check_params(params, &D);
    if (st != KVARN_OK) return st;
    st = check_attention_shape(batch, n_q_heads, n_kv_heads, tiles_per_seq);
    if (st != KVARN_OK) return st;
    if (!q_fp16 || !out) return KVARN_E_NULL;
    if (tiles_per_seq > 0 && (!k_codes || !v_codes || !k_meta || !v_meta || (!workspace && !use_static)))
        return KVARN_E_NULL;
    if (misaligned(q_fp16) || misaligned(out) || misaligned(k_codes) || misaligned(v_codes) ||
        misaligned(k_meta) || misaligned(v_meta) || misaligned(workspace))
        return KVARN_E_ALIGN;
    const int ns = kvarn::attention_splits(batch, n_kv_heads, tiles_per_seq);
    const size_t need = kvarn::attention_workspace_bytes(batch, n_q_heads, D, ns);
    if (use_static) workspace_bytes = kvarn::kStaticScratchBytes;
    if (tiles_per_seq > 0 && workspace_bytes < need) return KVARN_E_WORKSPACE;
    if (batch == 0) return KVARN_OK;
    if (use_static && tiles_per_seq > 0) {
        // the device address of this GPU's copy of the static array
        if (kvarn::static_scratch(&workspace) != hipSuccess) return KVARN_E_HIP;
    }

    kvarn::AttnArgs a;
    a.q = static_cast<const uint16_t*>(q_fp16);
    a.kc = static_cast<const uint8_t*>(k_codes);
    a.vc = static_cast<const uint8_t*>(v_codes);
    a.km = static_cast<const uint16_t*>(k_meta);
    a.vm = static_cast<const uint16_t*>(v_meta);
    a.out = out;
    a.ws = static_cast<float*>(workspace);
    a.batch = batch;
    a.n_q_heads = n_q_heads;
    a.n_kv_heads = n_kv_heads;
    a.tiles_per_seq = tiles_per_seq;
    a.n_splits = ns;
    a.n_parts = ns;
    a.d0 = params->head_dim;
    a.sm_scale = sm_scale;
    hipError_t e = kvarn::launch_attention(a, D, params->k_bits, params->v_bits,
                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVARN_OK : KVARN_E_HIP;
}

}  // namespace

extern "C" {

kvarn_status kvarn_decode_attention(const kvarn_params* params, int32_t batch, int32_t n_q_heads,
                                    int32_t n_kv_heads, int32_t tiles_per_seq, const void* q_fp16,
                                    const void* k_codes, const void* v_codes, const void* k_meta,
                                    const void* v_meta, float sm_scale, float* out,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    return decode_attention_impl(params, batch, n_q_heads, n_kv_heads, tiles_per_seq, q_fp16,
                                 k_codes, v_codes, k_meta, v_meta, sm_scale, out, workspace,
                                 workspace_bytes, false, stream);
}

kvarn_status kvarn_decode_attention_noalloc(const kvarn_params* params, int32_t batch,
                                            int32_t n_q_heads, int32_t n_kv_heads,
                                            int32_t tiles_per_seq, const void* q_fp16,
                                            const void* k_codes, const void* v_codes,
                                            const void* k_meta, const void* v_meta,
                                            float sm_scale, float* out, void* stream) {
    return decode_attention_impl(params, batch, n_q_heads, n_kv_heads, tiles_per_seq, q_fp16,
                                 k_codes, v_codes, k_meta, v_meta, sm_scale, out, nullptr, 0, true,
                                 stream);
}

kvarn_status kvarn_quantize_tiles_to(const kvarn_params* params, int64_t n_tiles,
                                     const void* k_fp16, const void* v_fp16,
                                     const int64_t* dst_tile, int64_t pool_tiles, void* k_codes,
                                     void* v_codes, void* k_meta, void* v_meta, void* stream) {
    int D = 0;
    kvarn_status st = check_params(params, &D);
    if (st != KVARN_OK) return st;
    const int ks = pointer_set(k_fp16, k_codes, k_meta);
    const int vs = pointer_set(v_fp16, v_codes, v_meta);
    if (ks < 0 || vs < 0) return KVARN_E_NULL;
    if (n_tiles < 0 || n_tiles > kMaxTiles || pool_tiles < 0 || pool_tiles > kMaxTiles)
        return KVARN_E_SHAPE;
    if (n_tiles > 0 && (ks || vs) && !dst_tile) return KVARN_E_NULL;
    if (misaligned(k_fp16) || misaligned(v_fp16) || misaligned(k_codes) || misaligned(v_codes) ||
        misaligned(k_meta) || misaligned(v_meta) || misaligned(dst_tile))
        return KVARN_E_ALIGN;
    if (n_tiles == 0 || pool_tiles == 0 || (ks == 0 && vs == 0)) return KVARN_OK;

    kvarn::QuantArgs a;
    a.k = static_cast<const uint16_t*>(k_fp16);
    a.v = static_cast<const uint16_t*>(v_fp16);
    a.kc = static_cast<uint8_t*>(k_codes);
    a.vc = static_cast<uint8_t*>(v_codes);
    a.km = static_cast<uint16_t*>(k_meta);
    a.vm = static_cast<uint16_t*>(v_meta);
    a.n_k = ks ? n_tiles : 0;
    a.n_v = vs ? n_tiles : 0;
    a.d0 = params->head_dim;
    a.n_iters = params->n_iters;
    a.dst = dst_tile;
    a.pool = pool_tiles;
    hipError_t e = kvarn::launch_quantize(a, D, params->k_bits, params->v_bits,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVARN_OK : KVARN_E_HIP;
}

kvarn_status kvarn_decode_attention_paged_workspace(const kvarn_params* params, int32_t batch,
                                                    int32_t n_q_heads, int32_t n_kv_heads,
                                                    int32_t max_blocks, size_t* bytes) {
    if (!bytes) return KVARN_E_NULL;
    int D = 0;
    kvarn_status st = check_params(params, &D);
    if (st != KVARN_OK) return st;
    st = check_attention_shape(batch, n_q_heads, n_kv_heads, max_blocks);
    if (st != KVARN_OK) return st;
    int ns = kvarn::attention_splits(batch, n_kv_heads, max_blocks);
    if (max_blocks == 0) ns = 0;
    *bytes = kvarn::attention_workspace_bytes(batch, n_q_heads, D, ns + 1);
    return KVARN_OK;
}

kvarn_status kvarn_decode_attention_paged(const kvarn_params* params, int32_t batch,
                                          int32_t n_q_heads, int32_t n_kv_heads,
                                          int32_t max_blocks, int64_t pool_blocks,
                                          const int32_t* block_table, const int32_t* n_blocks,
                                          const int32_t* tail_len, const void* q_fp16,
                                          const void* k_codes, const void* v_codes,
                                          const void* k_meta, const void* v_meta,
                                          const void* k_tail, const void* v_tail,
                                          float sm_scale, float* out, void* workspace,
                                          size_t workspace_bytes, void* stream) {
    int D = 0;
    kvarn_status st = check_params(params, &D);
    if (st != KVARN_OK) return st;
    st = check_attention_shape(batch, n_q_heads, n_kv_heads, max_blocks);
    if (st != KVARN_OK) return st;
    if (pool_blocks < 0 || pool_blocks * (int64_t)n_kv_heads > kMaxTiles) return KVARN_E_SHAPE;
    if (!q_fp16 || !out || !workspace || !n_blocks || !tail_len || !k_tail || !v_tail)
        return KVARN_E_NULL;
    const bool packed = max_blocks > 0 && pool_blocks > 0;
    if (packed && (!block_table || !k_codes || !v_codes || !k_meta || !v_meta))
        return KVARN_E_NULL;
    if (misaligned(q_fp16) || misaligned(out) || misaligned(workspace) || misaligned(n_blocks) ||
        misaligned(tail_len) || misaligned(k_tail) || misaligned(v_tail) ||
        misaligned(block_table) || misaligned(k_codes) || misaligned(v_codes) ||
        misaligned(k_meta) || misaligned(v_meta))
        return KVARN_E_ALIGN;
    int ns = kvarn::attention_splits(batch, n_kv_heads, max_blocks);
    if (max_blocks == 0) ns = 0;
    if (workspace_bytes < kvarn::attention_workspace_bytes(batch, n_q_heads, D, ns + 1))
        return KVARN_E_WORKSPACE;
    if (batch == 0) return KVARN_OK;

    kvarn::AttnArgs a;
    a.q = static_cast<const uint16_t*>(q_fp16);
    a.kc = static_cast<const uint8_t*>(k_codes);
    a.vc = static_cast<const uint8_t*>(v_codes);
    a.km = static_cast<const uint16_t*>(k_meta);
    a.vm = static_cast<const uint16_t*>(v_meta);
    a.out = out;
    a.ws = static_cast<float*>(workspace);
    a.batch = batch;
    a.n_q_heads = n_q_heads;
    a.n_kv_heads = n_kv_heads;
    a.tiles_per_seq = max_blocks;
    // without a pool no packed tile is read: only the tail's partial slot
    a.n_splits = packed ? ns : 0;
    a.n_parts = (packed ? ns : 0) + 1;
    a.d0 = params->head_dim;
    a.sm_scale = sm_scale;
    a.table = block_table;
    a.nblk = n_blocks;
    a.tail_len = tail_len;
    a.k_tail = static_cast<const uint16_t*>(k_tail);
    a.v_tail = static_cast<const uint16_t*>(v_tail);
    a.pool_blocks = pool_blocks;
    hipError_t e = kvarn::launch_attention(a, D, params->k_bits, params->v_bits,
                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVARN_OK : KVARN_E_HIP;
}

}  // extern "C"

// ---- attention over an uncompressed fp16 cache (the baseline) ----

static kvarn_status check_fp16_attention(int32_t head_dim, int32_t batch, int32_t n_q_heads,
                                         int32_t n_kv_heads, int64_t seq_len, int* D) {
    if (head_dim < 33 || head_dim > 256 || (head_dim % 8) != 0) return KVARN_E_HEAD_DIM;
    if (seq_len < 0) return KVARN_E_SHAPE;
    // one (sequence, KV head) of K or V is addressed with 32-bit byte offsets
    if (seq_len * head_dim * 2 > INT32_MAX) return KVARN_E_SHAPE;
    kvarn_status st = check_attention_shape(batch, n_q_heads, n_kv_heads, 0);
    if (st != KVARN_OK) return st;
    if ((int64_t)batch * n_q_heads > INT32_MAX) return KVARN_E_SHAPE;
    const int64_t tiles = (seq_len + TILE - 1) / TILE;
    if (tiles > kMaxTiles || (int64_t)batch * n_kv_heads * tiles > kMaxTiles) return KVARN_E_SHAPE;
    int d = 64;
    while (d < head_dim) d *= 2;
    *D = d;
    return KVARN_OK;
}

kvarn_status kvarn_decode_attention_fp16_workspace(int32_t head_dim, int32_t batch,
                                                   int32_t n_q_heads, int32_t n_kv_heads,
                                                   int64_t seq_len, size_t* bytes) {
    if (!bytes) return KVARN_E_NULL;
    int D = 0;
    kvarn_status st = check_fp16_attention(head_dim, batch, n_q_heads, n_kv_heads, seq_len, &D);
    if (st != KVARN_OK) return st;
    const int ns = kvarn::attention_fp16_splits(batch, n_kv_heads, seq_len, D);
    *bytes = kvarn::attention_workspace_bytes(batch, n_q_heads, D, ns);
    return KVARN_OK;
}

kvarn_status kvarn_decode_attention_fp16(int32_t head_dim, int32_t batch, int32_t n_q_heads,
                                         int32_t n_kv_heads, int64_t seq_len, const void* q_fp16,
                                         const void* k_fp16, const void* v_fp16, float sm_scale,
                                         float* out, void* workspace, size_t workspace_bytes,
                                         void* stream) {
    int D = 0;
    kvarn_status st = check_fp16_attention(head_dim, batch, n_q_heads, n_kv_heads, seq_len, &D);
    if (st != KVARN_OK) return st;
    if (!q_fp16 || !out) return KVARN_E_NULL;
    if (seq_len > 0 && (!k_fp16 || !v_fp16 || !workspace)) return KVARN_E_NULL;
    if (misaligned(q_fp16) || misaligned(out) || misaligned(k_fp16) || misaligned(v_fp16) ||
        misaligned(workspace))
        return KVARN_E_ALIGN;
    const int ns = kvarn::attention_fp16_splits(batch, n_kv_heads, seq_len, D);
    if (ns > 0 && workspace_bytes < kvarn::attention_workspace_bytes(batch, n_q_heads, D, ns))
        return KVARN_E_WORKSPACE;
    if (batch == 0) return KVARN_OK;

    kvarn::Fp16AttnArgs a;
    a.q = static_cast<const uint16_t*>(q_fp16);
    a.k = static_cast<const uint16_t*>(k_fp16);
    a.v = static_cast<const uint16_t*>(v_fp16);
    a.out = out;
    a.ws = static_cast<float*>(workspace);
    a.batch = batch;
    a.n_q_heads = n_q_heads;
    a.n_kv_heads = n_kv_heads;
    a.seq_len = seq_len;
    a.n_splits = ns;
    a.d0 = head_dim;
    a.sm_scale = sm_scale;
    hipError_t e = kvarn::launch_attention_fp16(a, D, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVARN_OK : KVARN_E_HIP;
}
