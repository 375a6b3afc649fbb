/*
 * kvarn.h -- C ABI of the KVarN KV-cache quantizer hot path on MI355X (gfx950).
 *
 * The method (pages cited by title and section):
 *   - hotdry: "KVarN Hadamard 旋转与方差归一化：KV-cache 量化的校准算法实现"
 *     (blog.hotdry.top): §Hadamard 旋转 (per-tile Walsh-Hadamard rotation
 *     along the channels, computed as an O(n log n) transform), §迭代方差归一化
 *     (alternating column / row standard-deviation normalisation in log space,
 *     3-5 iterations), §非对称量化与尺度折叠 (asymmetric round-to-nearest, K
 *     4-bit with per-channel scales, V 2-bit with per-token scales, folded back
 *     on read), §可落地的实现参数 (the kvarn_k4v2_g128 preset, 128-token tiles,
 *     fp16).
 *   - deep: "KV cache 為什麼能壓到 4-bit／2-bit 還不掉準確度——從 variance
 *     normalization 講起" (vatt-ghern.pages.dev): the worked 2-bit example
 *     (zero point = min, scale = range / (2^b - 1)), the four-stage pipeline
 *     and the KEY/VALUE table, and the deployment knob table (tile = one
 *     128-token PagedAttention block, scales travel with their block).
 *   - digest: "KVarN: 方差归一化的KV-Cache量化缓解推理任务中的误差累积"
 *     (ai-feeds.com): §方法 module 3 (dequantise, then attention over the
 *     quantised cache), §局限 (head_dim padded to a power of two).
 *
 * Conventions shared by every entry point
 *   - A tile is 128 consecutive tokens x head_dim channels of K or of V for
 *     one (layer or sequence, KV head).  head_dim D0 is padded with zeros to
 *     D = the next power of two, at least 64 (D0 = 96 -> 128).
 *   - fp16 inputs and outputs are IEEE binary16, tokens-major:
 *     [n_tiles][128][D0].
 *   - Packed codes, format v1: the b-bit code of element e is stored at bit
 *     e*b of the tile's byte stream, least significant bit first.  K elements
 *     are numbered e = t*D + j (token-major); V elements e = j*128 + t
 *     (channel-major).  Per tile: 128*D*b/8 bytes.
 *   - Meta, binary16 per tile: K [SK (D) | ZK (D) | RK (128)],
 *     V [SV (128) | ZV (128) | CV (D)].  The rotated-domain value is
 *     K: RK_t * (code * SK_j + ZK_j),  V: CV_j * (code * SV_t + ZV_t).
 *   - Every device pointer must be 16-byte aligned.  Buffers are owned and
 *     allocated by the caller; the library allocates nothing, never prints
 *     and never aborts.  Its only global state is the static scratch of
 *     kvarn_decode_attention_noalloc (a device array per GPU and its cached
 *     device address); every other entry point keeps none.
 *   - Every argument is validated on the host before any launch.  Launches
 *     are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream); nothing synchronises.  A launch failure reported by the HIP
 *     runtime returns KVARN_E_HIP and leaves the outputs unspecified.
 *   - Inputs must be finite; a tile holding NaN or Inf gets unspecified
 *     output for that tile only.
 */
#ifndef KVARN_H
#define KVARN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVARN_OK = 0,
    KVARN_E_NULL = 1,      /* a required pointer is NULL, or a pointer set is partly NULL */
    KVARN_E_HEAD_DIM = 2,  /* head_dim outside 33..256 or not a multiple of 8 */
    KVARN_E_TILE = 3,      /* tile_tokens != 128 */
    KVARN_E_BITS = 4,      /* k_bits or v_bits not in {2, 4} */
    KVARN_E_ITERS = 5,     /* n_iters outside 0..16 */
    KVARN_E_SHAPE = 6,     /* negative or too large a count, or n_q_heads % n_kv_heads != 0 */
    KVARN_E_ALIGN = 7,     /* a pointer is not 16-byte aligned */
    KVARN_E_WORKSPACE = 8, /* attention workspace (or the static scratch) too small for the shape */
    KVARN_E_HIP = 9        /* the HIP runtime reported an error at launch */
} kvarn_status;

/* Problem statement of one KV-cache configuration. */
typedef struct {
    int32_t head_dim;    /* D0: 33..256, multiple of 8 */
    int32_t tile_tokens; /* must be 128: one tile = one 128-token block */
    int32_t k_bits;      /* 2 or 4 (preset k4v2: 4) */
    int32_t v_bits;      /* 2 or 4 (preset k4v2: 2) */
    int32_t n_iters;     /* normalisation iterations, 0..16 (the pages: 3-5) */
} kvarn_params;

/* Per-tile byte sizes of the packed format. */
typedef struct {
    int32_t padded_dim;    /* D */
    int64_t k_code_bytes;  /* 128 * D * k_bits / 8 */
    int64_t v_code_bytes;  /* 128 * D * v_bits / 8 */
    int64_t k_meta_bytes;  /* 2 * (2 * D + 128) */
    int64_t v_meta_bytes;  /* 2 * (256 + D) */
} kvarn_tile_layout;

/* Host only, pure: validates params and fills the per-tile layout. */
kvarn_status kvarn_get_layout(const kvarn_params *params, kvarn_tile_layout *layout);

/* Host only: parses "kvarn_k{K}v{V}_g{G}" (e.g. "kvarn_k4v2_g128") into params.
 * G must be 128.  Returns KVARN_E_BITS / KVARN_E_TILE / KVARN_E_NULL on a bad string. */
kvarn_status kvarn_params_from_preset(const char *preset, int32_t head_dim, int32_t n_iters,
                                      kvarn_params *params);

/* Quantise n_tiles tiles of K and of V (rotate, normalise, round, pack, fold).
 * Defined by: hotdry §Hadamard 旋转 (rotation of every token along the
 * channels), §迭代方差归一化 (n_iters rounds of column-then-row std
 * normalisation, factors accumulated in log space), §非对称量化与尺度折叠
 * (K per channel at k_bits, V per token at v_bits, the group-axis factor
 * folded into the group's scale and zero point); deep page, worked 2-bit
 * example (zero point = group min, scale = range / (2^b - 1), code =
 * round((v - min) / scale)).
 *   k_fp16, v_fp16   [n_tiles][128][head_dim] fp16, device, read only
 *   k_codes, v_codes [n_tiles][k|v_code_bytes] device, written
 *   k_meta, v_meta   [n_tiles][k|v_meta_bytes / 2] fp16, device, written
 * Either tensor may be skipped by passing all three of its pointers NULL;
 * a partly NULL set is KVARN_E_NULL.  n_tiles == 0 launches nothing. */
kvarn_status kvarn_quantize_tiles(const kvarn_params *params, int64_t n_tiles,
                                  const void *k_fp16, const void *v_fp16,
                                  void *k_codes, void *v_codes,
                                  void *k_meta, void *v_meta, void *stream);

/* Inverse of kvarn_quantize_tiles: unpack, apply the folded scales, undo the
 * rotation, keep the first head_dim channels, round to fp16 (nearest even).
 * Defined by: hotdry §非对称量化与尺度折叠 (the folded scales restore the
 * range on read) and §Hadamard 旋转 (the orthonormal transform is its own
 * inverse); digest §方法 module 3 (the cache is dequantised for attention).
 *   k_out, v_out [n_tiles][128][head_dim] fp16, device, written.
 * Pointer sets (codes, meta, out) of K or V may be all NULL to skip. */
kvarn_status kvarn_dequantize_tiles(const kvarn_params *params, int64_t n_tiles,
                                    const void *k_codes, const void *v_codes,
                                    const void *k_meta, const void *v_meta,
                                    void *k_out, void *v_out, void *stream);

/* Workspace (bytes) that kvarn_decode_attention needs for this shape. */
kvarn_status kvarn_decode_attention_workspace(const kvarn_params *params, int32_t batch,
                                              int32_t n_q_heads, int32_t n_kv_heads,
                                              int32_t tiles_per_seq, size_t *bytes);

/* One decode step of GQA attention over the packed cache.  Defined by:
 * digest §方法 module 3 (attention reads the dequantised cache); deep page,
 * stage card of the rotation (the orthonormal rotation keeps inner
 * products, so scores can be taken in the rotated domain) and section
 * "一次 16K context 的推論，記憶體都花到哪去了" (decode reads the whole cache
 * each step):
 *   out[b][h] = softmax(sm_scale * q[b][h] . K[b][g]^T) V[b][g],  g = h / (n_q_heads / n_kv_heads)
 * with K, V the dequantised cache (computed on the fly in the rotated domain,
 * never materialised).
 *   q        [batch][n_q_heads][head_dim] fp16, device
 *   codes / meta: tile i of (b, g) at index (b * n_kv_heads + g) * tiles_per_seq + i
 *   out      [batch][n_q_heads][head_dim] fp32, device, written
 *   workspace at least kvarn_decode_attention_workspace bytes, device, scratch. */
kvarn_status kvarn_decode_attention(const kvarn_params *params, int32_t batch,
                                    int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t tiles_per_seq, const void *q_fp16,
                                    const void *k_codes, const void *v_codes,
                                    const void *k_meta, const void *v_meta,
                                    float sm_scale, float *out, void *workspace,
                                    size_t workspace_bytes, void *stream);

/* ---- allocation-free variant, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation) ---- */

/* Bytes of the library's static scratch buffer: one file-scope device array
 * per GPU, held until the process ends. */
#define KVARN_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* kvarn_decode_attention with its split partials in the library's static
 * scratch instead of a caller workspace; arguments and
 * results are those of kvarn_decode_attention.  It allocates nothing: the
 * scratch of the current device is looked up once per device (the stream
 * must belong to the current device).  A shape whose workspace
 * (kvarn_decode_attention_workspace) exceeds KVARN_STATIC_SCRATCH_BYTES is
 * refused with KVARN_E_WORKSPACE before any launch.  Every call on one GPU
 * shares that GPU's scratch: calls that overlap on one GPU (different
 * streams, or different host threads without ordering) race; calls in one
 * stream are ordered.  Nothing in the scratch needs to start at zero. */
kvarn_status kvarn_decode_attention_noalloc(const kvarn_params *params, int32_t batch,
                                            int32_t n_q_heads, int32_t n_kv_heads,
                                            int32_t tiles_per_seq, const void *q_fp16,
                                            const void *k_codes, const void *v_codes,
                                            const void *k_meta, const void *v_meta,
                                            float sm_scale, float *out, void *stream);

/* ---- paged cache (deep page, the section on running inside vLLM's
 * PagedAttention: one 128-token page is one tile and its scales travel with
 * the page; the tokens that do not fill a page yet stay apart, in fp16, in a
 * decode workspace) ---- */

/* kvarn_quantize_tiles into chosen slots of a tile pool: input tile i of K and
 * of V is written to pool tile dst_tile[i] of the codes and meta arrays.
 *   dst_tile  [n_tiles] int64, device, read only; entries outside
 *             [0, pool_tiles) skip that input tile (nothing is written)
 *   k_codes.. [pool_tiles][...] as in kvarn_quantize_tiles
 * Two entries naming the same slot leave that slot unspecified. */
kvarn_status kvarn_quantize_tiles_to(const kvarn_params *params, int64_t n_tiles,
                                     const void *k_fp16, const void *v_fp16,
                                     const int64_t *dst_tile, int64_t pool_tiles,
                                     void *k_codes, void *v_codes,
                                     void *k_meta, void *v_meta, void *stream);

/* Workspace (bytes) that kvarn_decode_attention_paged needs for this shape. */
kvarn_status kvarn_decode_attention_paged_workspace(const kvarn_params *params, int32_t batch,
                                                    int32_t n_q_heads, int32_t n_kv_heads,
                                                    int32_t max_blocks, size_t *bytes);

/* One decode step of GQA attention over a paged packed cache plus an fp16 tail.
 * Sequence b's tokens are those of its n_blocks[b] blocks, in table order,
 * then the first tail_len[b] rows of its tail.
 *   block_table [batch][max_blocks] int32, device: physical block of logical
 *               block i of sequence b; physical block p holds the tiles
 *               p * n_kv_heads + g (g = KV head) of the pool arrays
 *   n_blocks    [batch] int32, device: used blocks, read as clamped to
 *               0..max_blocks
 *   tail_len    [batch] int32, device: 0..128 tail tokens (clamped)
 *   k_tail, v_tail [batch][n_kv_heads][128][head_dim] fp16, device
 *   pool arrays k_codes .. v_meta hold pool_blocks * n_kv_heads tiles
 *   q, out, sm_scale as in kvarn_decode_attention; a sequence with no tokens
 *   gets out = 0.
 * Table entries outside [0, pool_blocks) are read as block 0 (no access
 * outside the pool; that sequence's output is then unspecified). */
kvarn_status kvarn_decode_attention_paged(const kvarn_params *params, int32_t batch,
                                          int32_t n_q_heads, int32_t n_kv_heads,
                                          int32_t max_blocks, int64_t pool_blocks,
                                          const int32_t *block_table, const int32_t *n_blocks,
                                          const int32_t *tail_len, const void *q_fp16,
                                          const void *k_codes, const void *v_codes,
                                          const void *k_meta, const void *v_meta,
                                          const void *k_tail, const void *v_tail,
                                          float sm_scale, float *out, void *workspace,
                                          size_t workspace_bytes, void *stream);

/* ---- uncompressed fp16 cache: the baseline the packed cache is measured
 * against (hotdry page, section on the deployment parameters: throughput is
 * compared with an FP16 baseline; deep page, section
 * "一次 16K context 的推論，記憶體都花到哪去了": every decode step reads the
 * whole cache, so decode is bound by memory bandwidth) ---- */

/* Workspace (bytes) that kvarn_decode_attention_fp16 needs for this shape
 * (0 when seq_len == 0). */
kvarn_status kvarn_decode_attention_fp16_workspace(int32_t head_dim, int32_t batch,
                                                   int32_t n_q_heads, int32_t n_kv_heads,
                                                   int64_t seq_len, size_t *bytes);

/* One decode step of GQA attention over an fp16 cache:
 *   out[b][h] = softmax(sm_scale * q[b][h] . K[b][g]^T) V[b][g],  g = h / (n_q_heads / n_kv_heads)
 *   head_dim    D0: 33..256, multiple of 8 (no padding is involved)
 *   q           [batch][n_q_heads][head_dim] fp16, device
 *   k_fp16, v_fp16 [batch][n_kv_heads][seq_len][head_dim] fp16, device, read
 *               only; with seq_len = 128 * tiles_per_seq this is the tile
 *               layout that kvarn_quantize_tiles reads
 *   out         [batch][n_q_heads][head_dim] fp32, device, written
 *   workspace   at least kvarn_decode_attention_fp16_workspace bytes, device,
 *               scratch (may be NULL when seq_len == 0)
 * seq_len == 0 gives out = 0.  The GQA group holds at most 16 heads, and one
 * (sequence, KV head) of K holds at most 2^31 - 1 bytes
 * (seq_len * head_dim * 2), else KVARN_E_SHAPE. */
kvarn_status kvarn_decode_attention_fp16(int32_t head_dim, int32_t batch, int32_t n_q_heads,
                                         int32_t n_kv_heads, int64_t seq_len, const void *q_fp16,
                                         const void *k_fp16, const void *v_fp16, float sm_scale,
                                         float *out, void *workspace, size_t workspace_bytes,
                                         void *stream);

/* Static description of a status code. */
const char *kvarn_status_str(kvarn_status status);

#ifdef __cplusplus
}
#endif

#endif /* KVARN_H */
