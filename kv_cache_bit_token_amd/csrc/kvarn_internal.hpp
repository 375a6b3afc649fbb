// kvarn_internal.hpp -- launch interfaces between the C ABI (kvarn_abi.cpp)
// and the kernels.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvarn.h"

namespace kvarn {

// Workgroups per launch of the kernels that give each tile its own workgroup:
// at up to 512 threads each, far inside a dispatch's 2^32 work-items.  Larger
// tile counts are launched in chunks, each kernel taking its first tile as an
// argument.
constexpr int64_t kMaxGrid = (int64_t)1 << 22;

struct QuantArgs {
    const uint16_t* k;  // [n_k][128][d0] fp16 bits
    const uint16_t* v;  // [n_v][128][d0]
    uint8_t* kc;
    uint8_t* vc;
    uint16_t* km;
    uint16_t* vm;
    int64_t n_k;        // tiles of K to process (0 = skip K)
    int64_t n_v;        // tiles of V to process (0 = skip V)
    int d0;
    int n_iters;
    const int64_t* dst = nullptr;   // output slot of input tile i (nullptr: slot i)
    int64_t pool = 0;               // slots in the output arrays when dst is set
};

struct DequantArgs {
    const uint8_t* kc;
    const uint8_t* vc;
    const uint16_t* km;
    const uint16_t* vm;
    uint16_t* ko;
    uint16_t* vo;
    int64_t n_k;
    int64_t n_v;
    int d0;
};

struct AttnArgs {
    const uint16_t* q;   // [B][Hq][d0]
    const uint8_t* kc;
    const uint8_t* vc;
    const uint16_t* km;
    const uint16_t* vm;
    float* out;          // [B][Hq][d0]
    float* ws;           // split-K partials
    int batch;
    int n_q_heads;
    int n_kv_heads;
    int tiles_per_seq;
    int n_splits;        // splits per (b, g) of the packed tiles; split s takes tiles s, s + n_splits, ...
    int d0;
    float sm_scale;
    int n_parts = 0;     // partial slots per (b, h) in the workspace (n_splits, + 1 with a tail)
    // paged cache (table == nullptr: tile i of (b, g) at (b * n_kv_heads + g) * tiles_per_seq + i)
    const int32_t* table = nullptr;     // [batch][tiles_per_seq] physical block ids
    const int32_t* nblk = nullptr;      // [batch] used blocks
    const int32_t* tail_len = nullptr;  // [batch] fp16 tail tokens
    const uint16_t* k_tail = nullptr;   // [batch][n_kv_heads][128][d0]
    const uint16_t* v_tail = nullptr;
    int tail_in_grid = 0;               // set by the launcher: tails run as extra partial-kernel blocks
    int fuse_combine = 0;               // set by the launcher: each workgroup holds all splits of one (b, g) and merges them
    int64_t pool_blocks = 0;
};

// Decode attention over an uncompressed fp16 cache (the baseline).
struct Fp16AttnArgs {
    const uint16_t* q;   // [B][Hq][d0]
    const uint16_t* k;   // [B][Hkv][seq_len][d0]
    const uint16_t* v;
    float* out;          // [B][Hq][d0]
    float* ws;           // split-K partials [B][Hq][n_splits][D + 2]
    int batch;
    int n_q_heads;
    int n_kv_heads;
    int64_t seq_len;
    int n_splits;        // splits per (b, g); split s takes token steps s, s + n_splits, ...
    int d0;
    float sm_scale;
};

// Static device scratch of the allocation-free attention entry point: one
// array per GPU, resolved per device on first use (kvarn_scratch.hip).
constexpr size_t kStaticScratchBytes = KVARN_STATIC_SCRATCH_BYTES;
hipError_t static_scratch(void** ptr);

hipError_t launch_quantize(const QuantArgs& a, int D, int kb, int vb, hipStream_t s);
hipError_t launch_dequantize(const DequantArgs& a, int D, int kb, int vb, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, int D, int kb, int vb, hipStream_t s);

// Split-K plan of the decode attention for a shape (shared by the workspace
// query and the launch, so both agree).
int attention_splits(int batch, int n_kv_heads, int tiles_per_seq);
// Split partials [batch][n_q_heads][n_parts][D + 2] (max, sum, accumulator).
size_t attention_workspace_bytes(int batch, int n_q_heads, int D, int n_parts);

// Splits per (b, KV head) of the fp16-cache attention (token steps of
// 32 * 128 / D).
int attention_fp16_splits(int batch, int n_kv_heads, int64_t seq_len, int D);
hipError_t launch_attention_fp16(const Fp16AttnArgs& a, int D, hipStream_t s);

}  // namespace kvarn
