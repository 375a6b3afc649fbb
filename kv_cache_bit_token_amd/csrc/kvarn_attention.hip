// kvarn_attention.hip -- decode attention over the packed KVarN cache, gfx950.
//
// Method (digest page "KVarN: 方差归一化的KV-Cache量化...", "方法" module 3: the
// quantised cache takes part in attention after the scales are restored;
// deep-dive page, stage card "Hadamard rotation": the rotation is orthonormal,
// so q.k is unchanged; hotdry page "非对称量化与尺度折叠": per-channel K
// scales, per-token V scales, folded back on read).
//
// Everything runs in the rotated domain; nothing is dequantised to memory.
// With mk = 2^(k_bits-1), mv = 2^(v_bits-1):
//   qh  = H q / sqrt(D)                          per (b, query head), in each split's wave
//   s_t = sm * RK_t * ( sum_j (qh_j SK_j)(code_tj - mk) + sum_j qh_j (ZK_j + mk SK_j) )
//   online softmax over the tiles of a split
//   acc_j = CV_j * ( sum_t (p_t SV_t)(code_tj - mv) + sum_t p_t (ZV_t + mv SV_t) )
//   o = H (acc / l) / sqrt(D), first head_dim channels      (combine kernel)
// Centring the codes keeps both terms of each sum small (ZK is the group
// minimum, so the uncentred terms would be large and of opposite sign).
//
// Integer matrix cores.  Both code contractions run on
// v_mfma_i32_16x16x64_i8.  The codes enter centred and scaled, as signed
// bytes 2^(8-b) (code - 2^(b-1)) (b = k_bits or v_bits), which the unpack
// forms at no extra cost: shift the b-bit field to the top of its byte,
// flip its top bit, mask.  The other factor, q' = qh SK per head (or
// p' = p SV), is a fixed-point integer X = rint(q' 2^f), |X| < 2^30 (2^f a
// power of two per head and tile), written as four signed base-256 digits
// X = B3 2^24 + B2 2^16 + B1 2^8 + B0, B_i in [-128, 127]: the bytes of
// (X + 0x808080) ^ 0x808080.  The 16 rows of that operand are 4 query heads
// x 4 digits, so one instruction gives every lane the four exact int32
// digit sums of one (head, token) score or (head, channel) output, already
// centred; they are joined as (C3 2^8 + C2) 2^16 + (C1 2^8 + C0) with one
// rounding to fp32 (and one exact power-of-two rescale).
//   q.K^T : A = q' digits (4 heads x 4 digits) x 64 channels, B = K code
//           bytes (64 channels x 16 tokens), C = digit sums [head, digit][token];
//   p.V   : A = p' digits (4 heads x 4 digits) x 64 tokens, B = V code bytes
//           (64 tokens x 16 channels), C = digit sums [head, digit][channel].
// A lane (row / column l % 16, k-group l / 16) holds 16 bytes of a run of
// 16 contraction indices; the byte order inside a run follows the cheapest
// unpack of the packed codes (RunOrder), and the other operand follows it.
//
// Token order.  Lane l of a score or output tile holds head l / 16; its
// column c = l % 16 is, for the scores of 16-token block mb, token
// tau(mb, c) = r0(c) + delta(mb).  The map is chosen so that the 8 tokens
// a lane scores are exactly the 8 bytes it contributes to the p.V operand
// (two dwords of one run), so the softmax runs where the scores land and
// writes whole dwords of the p' image; the only LDS round trips per tile
// are the meta, the q' image and the p' image.
//
// Work split: each wavefront owns one split of one (b, KV head) and every
// query head of that head's GQA group; these waves do not synchronise with
// each other before their last tile.  Split s of n takes tiles s, s + n, s + 2n, ... of the
// sequence, so the n waves of a sequence read n neighbouring tiles at a time
// and the device reads a few hundred short windows instead of one long run
// per wave.  A paged call's fp16 tails run as
// extra 256-thread workgroups of the same grid where its workgroups have
// 256 threads (they synchronise only among their own waves), else as a
// kernel of their own.  Where a (b, KV head)'s splits fit one workgroup
// (no block table, no tails, at most 4 splits) they run as its waves and
// merge there, through LDS; otherwise a combine kernel merges the splits'
// (max, sum, acc).  Either way the merge undoes the rotation.
#include "kvarn_device.hpp"
#include "kvarn_internal.hpp"
#include "kvarn_rsrc.hpp"

namespace kvarn {

typedef int v4i_t __attribute__((ext_vector_type(4)));

// Splits in total: about two per SIMD.  Timed on a cache that no earlier
// pass has left in the last-level cache, four strided splits per sequence
// were fastest on the 64 x 8 x 16384 cache (0.149 ms, against 0.153 at eight
// and 0.158 at twelve); on 64 x 8 x 32768 the three counts were within the
// run-to-run spread.  Four divide both caches' 128 and 256 tiles evenly.
constexpr int kTargetWaves = 2048;
constexpr float kLog2e = 1.4426950408889634f;
// The combine kernel reads at most this many parts per (b, head) in one round trip.
constexpr int kCombineParts = 16;

// Splits per (b, KV head): about kTargetWaves in total, at most one per tile,
// and no more than the tile count needs at that many tiles per split.
int attention_splits(int batch, int n_kv_heads, int tiles_per_seq) {
    const int64_t pairs = (int64_t)batch * n_kv_heads;
    if (pairs <= 0 || tiles_per_seq <= 0) return 1;
    int64_t want = (kTargetWaves + pairs - 1) / pairs;
    if (want > tiles_per_seq) want = tiles_per_seq;
    if (want < 1) want = 1;
    const int64_t per = (tiles_per_seq + want - 1) / want;
    return (int)((tiles_per_seq + per - 1) / per);
}

size_t attention_workspace_bytes(int batch, int n_q_heads, int D, int n_parts) {
    return (size_t)batch * n_q_heads * n_parts * (D + 2) * sizeof(float);
}

// ---- packed codes -> centred bytes for the int8 matrix cores ----------------
// One run of 16 codes (the 16 contraction indices one lane group gives one
// instruction) becomes 4 dwords of signed bytes 2^(8-B) (c - 2^(B-1)):
//   4 bits (two packed dwords w0, w1):  dword 2q + h holds nibble h of each byte of w_q
//   2 bits (one packed dword w):         dword s      holds crumb s of each byte of w
// so byte n of dword j holds run position base(j) + stride * n.
template <int B> struct RunOrder;
template <> struct RunOrder<4> {
    static constexpr int kWords = 2;    // packed dwords per run
    static constexpr int kStride = 2;
    __host__ __device__ static constexpr int base(int j) { return 8 * (j / 2) + j % 2; }
};
template <> struct RunOrder<2> {
    static constexpr int kWords = 1;
    static constexpr int kStride = 4;
    __host__ __device__ static constexpr int base(int j) { return j; }
};

// The B-bit field at bit P of every byte of w, moved to the top of its byte
// with its top bit flipped: as a signed byte that is 2^(8-B) (c - 2^(B-1)).
template <int B, int P>
__device__ __forceinline__ int centred_field(uint32_t w) {
    constexpr uint32_t kTop = B == 4 ? 0xF0F0F0F0u : 0xC0C0C0C0u;
    return (int)(((w << (8 - B - P)) ^ 0x80808080u) & kTop);
}

template <int B>
__device__ __forceinline__ v4i_t code_bytes(const uint32_t* w) {
    if constexpr (B == 4) {
        return (v4i_t){centred_field<4, 0>(w[0]), centred_field<4, 4>(w[0]),
                       centred_field<4, 0>(w[1]), centred_field<4, 4>(w[1])};
    } else {
        return (v4i_t){centred_field<2, 0>(w[0]), centred_field<2, 2>(w[0]),
                       centred_field<2, 4>(w[0]), centred_field<2, 6>(w[0])};
    }
}

// Token of column c in 16-token block mb (tau = r0(c) + delta(mb)): column c
// = 4 g + j owns dword j of lane group g's two p.V runs (tokens 32 g + 16 m
// + base(j) + stride n, m = mb / 4, n = mb % 4), so its 8 scores are the 8
// bytes it writes into the p' image.
template <int VB>
__device__ __forceinline__ int tok_r0(int c) { return 32 * (c >> 2) + RunOrder<VB>::base(c & 3); }
template <int VB>
__host__ __device__ constexpr int tok_delta(int mb) { return 16 * (mb >> 2) + RunOrder<VB>::kStride * (mb & 3); }

// 2^x on the transcendental unit without the library's denormal-range
// guard: results below 2^-126 (softmax weights e^-87 below the running
// maximum) come out as zero instead of subnormal.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// reductions over aligned groups of W lanes (W = 8, 16, 32, 64)
template <int W>
__device__ __forceinline__ float grp_sum(float v) {
    v += dpp<DPP_XOR1>(v);
    v += dpp<DPP_XOR2>(v);
    v += dpp<DPP_HMIR>(v);
    if constexpr (W >= 16) v += dpp<DPP_ROR8>(v);
    if constexpr (W >= 32) v += __shfl_xor(v, 16);
    if constexpr (W >= 64) v += __shfl_xor(v, 32);
    return v;
}
template <int W>
__device__ __forceinline__ float grp_max(float v) {
    v = fmaxf(v, dpp<DPP_XOR1>(v));
    v = fmaxf(v, dpp<DPP_XOR2>(v));
    v = fmaxf(v, dpp<DPP_HMIR>(v));
    if constexpr (W >= 16) v = fmaxf(v, dpp<DPP_ROR8>(v));
    if constexpr (W >= 32) v = fmaxf(v, __shfl_xor(v, 16));
    if constexpr (W >= 64) v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}
// power-of-two scale s with max * s in [2^29, 2^30) (1 for max == 0): the
// fixed-point range of the four signed base-256 digits
__device__ __forceinline__ float fx_scale(float mx) {
    if (!(mx > 0.0f)) return 1.0f;
    int e;
    (void)frexpf(mx, &e);          // mx = m * 2^e, m in [0.5, 1)
    return ldexpf(1.0f, 30 - e);
}

// x = rint(v * s), |x| < 2^30, as its signed base-256 digits B0 .. B3 in
// bytes 0 .. 3: adding 128 below each of the upper three digit positions
// makes every lower byte hold B_i + 128, and flipping those bytes' top
// bits gives B_i in two's complement (the top byte is B3 as it is).
__device__ __forceinline__ uint32_t fx_digits(float v, float s) {
    const int x = (int)__builtin_rintf(v * s);
    return ((uint32_t)x + 0x808080u) ^ 0x808080u;
}

// 4 x 4 byte transpose: d[i] byte n = byte i of a[n] (digit i of value n).
__device__ __forceinline__ void digit_dwords(const uint32_t (&a)[4], uint32_t (&d)[4]) {
    const uint32_t t0 = __builtin_amdgcn_perm(a[1], a[0], 0x05010400u);   // a0.0 a1.0 a0.1 a1.1
    const uint32_t t1 = __builtin_amdgcn_perm(a[1], a[0], 0x07030602u);   // a0.2 a1.2 a0.3 a1.3
    const uint32_t u0 = __builtin_amdgcn_perm(a[3], a[2], 0x05010400u);
    const uint32_t u1 = __builtin_amdgcn_perm(a[3], a[2], 0x07030602u);
    d[0] = __builtin_amdgcn_perm(u0, t0, 0x05040100u);
    d[1] = __builtin_amdgcn_perm(u0, t0, 0x07060302u);
    d[2] = __builtin_amdgcn_perm(u1, t1, 0x05040100u);
    d[3] = __builtin_amdgcn_perm(u1, t1, 0x07060302u);
}

// Digit sums c[i] = sum B_i * centred code of one (head, index):
// sum x (code - mid) 2^(8-b) = ((c3 2^8 + c2) 2^16 + (c1 2^8 + c0)).
__device__ __forceinline__ float limb_join(v4i_t c) {
    const int hi = (c[3] << 8) + c[2];
    const int lo = (c[1] << 8) + c[0];
    return __builtin_fmaf((float)hi, 65536.0f, (float)lo);
}

// Per-wave LDS layout (bytes), for GQA group size G (RB = ceil(G / 4) row
// blocks of 4 heads): the tile's meta (K then V, adjacent), the q' digit
// image [rb][kc][slot][16 B] and the p' digit image [rb][m][slot][16 B]
// (both in the matrix-core operand layout, one 16-byte read per lane), and
// two per-head scalars of the scores (zero-point term, 1 / scale).
//
// Lane l reads slot l ^ s of an image, s = qa_swz(l / 16, kc) for q' and
// l / 16 for p'.  Each slot is stored as four dwords by four lanes; without
// the XOR, a half-wave's stores of one digit fill only 4 (q') or 8 (p') of
// the 32 banks that 4-byte stores are served by.  The XOR moves the slots
// of the storing lanes' different runs (q': run (gq, kc); p': lane group
// col / 4) onto different banks, and stays inside each 16-slot group, so a
// quarter wave still reads 16 distinct slots.
template <int D>
__host__ __device__ constexpr int qa_swz(int gq, int kc) { return (gq * (D / 64) + kc) & 7; }

template <int D>
struct AttnLds {
    static constexpr int KMH = 2 * D + TILE, VMH = 2 * TILE + D;
    static constexpr int NKC = D / 64;          // 64-channel runs of q.K^T per M-block
    __host__ __device__ static constexpr int rb(int G) { return (G + 3) / 4; }
    __host__ __device__ static constexpr int kmeta(int) { return 0; }
    __host__ __device__ static constexpr int vmeta(int) { return 2 * KMH; }
    __host__ __device__ static constexpr int qa(int) { return 2 * KMH + 2 * VMH; }
    __host__ __device__ static constexpr int pa(int G) { return qa(G) + rb(G) * NKC * 1024; }
    __host__ __device__ static constexpr int stats(int G) { return pa(G) + rb(G) * 2 * 1024; }
    __host__ __device__ static constexpr int bytes(int G) { return stats(G) + 8 * 4 * rb(G); }
};

// Natural-order Walsh-Hadamard transform of one D-vector held by one
// wavefront, lane l owning channels CPL l .. CPL l + CPL - 1 (CPL = D / 64),
// scaled by 1 / sqrt(D).  Stage h pairs channels j and j + h (j & h == 0)
// into (x_j + x_{j+h}, x_j - x_{j+h}), h = 1, 2, 4, ...: stages below CPL
// inside the lane, the others across lanes (partner lane l ^ (h / CPL); the
// upper member of a pair keeps partner - self).
template <int D>
__device__ __forceinline__ void wave_fwht(float (&v)[D / 64]) {
    constexpr int CPL = D / 64;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int h = 1; h < CPL; h <<= 1)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            if ((c & h) == 0) {
                const float x = v[c], y = v[c + h];
                v[c] = x + y;
                v[c + h] = x - y;
            }
#pragma unroll
    for (int h = CPL; h < D; h <<= 1) {
        const int lx = h / CPL;
        const bool upper = (lane & lx) != 0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float o = __shfl_xor(v[c], lx);
            v[c] = upper ? o - v[c] : v[c] + o;
        }
    }
    const float sc = 1.0f / __builtin_sqrtf((float)D);
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] *= sc;
}

// CPL consecutive fp16 channels of a query row as one load, and their floats.
template <int CPL> struct QRowChunk;
template <> struct QRowChunk<1> {
    using type = uint16_t;
    __device__ static void unpack(type w, float (&v)[1]) { v[0] = h2f_bits(w); }
};
template <> struct QRowChunk<2> {
    using type = uint32_t;
    __device__ static void unpack(type w, float (&v)[2]) {
        v[0] = h2f_bits((uint16_t)w);
        v[1] = h2f_bits((uint16_t)(w >> 16));
    }
};
template <> struct QRowChunk<4> {
    using type = uint2;
    __device__ static void unpack(type w, float (&v)[4]) {
        v[0] = h2f_bits((uint16_t)w.x);
        v[1] = h2f_bits((uint16_t)(w.x >> 16));
        v[2] = h2f_bits((uint16_t)w.y);
        v[3] = h2f_bits((uint16_t)(w.y >> 16));
    }
};

// The splits of one (b, KV head) as the waves of one workgroup (split =
// wave), merged there: each wave has written its (m, l, acc) per query head
// to ex[split][n][D + 2] in LDS and passed a barrier; wave w then merges
// heads w, w + n_splits, ... exactly as the combine kernel does (same
// reductions, same order) and writes their outputs.
template <int D>
__device__ void merge_splits_in_block(const AttnArgs& a, const float* ex, int b, int g, int G, int wave) {
    constexpr int CPL = D / 64;
    const int lane = threadIdx.x & 63;
    const int ns = a.n_splits;
    for (int n = wave; n < G; n += ns) {
        float ms = -INFINITY, ls = 0.0f;
        if (lane < ns) {
            ms = ex[((size_t)lane * G + n) * (D + 2)];
            ls = ex[((size_t)lane * G + n) * (D + 2) + 1];
        }
        float M = ms;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
        const float w = (ms != -INFINITY) ? exp2f((ms - M) * kLog2e) : 0.0f;
        float L = ls * w;
        float v[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[c] = 0.0f;
        for (int k = 0; k < ns; ++k) {
            const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
            const float* pk = ex + ((size_t)k * G + n) * (D + 2) + 2 + CPL * lane;
#pragma unroll
            for (int c = 0; c < CPL; ++c) v[c] = __builtin_fmaf(pk[c], wk, v[c]);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
        const float il = (L > 0.0f) ? 1.0f / L : 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[c] *= il;
        wave_fwht<D>(v);
        const size_t bh = (size_t)b * a.n_q_heads + g * G + n;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int j = CPL * lane + c;
            if (j < a.d0) a.out[bh * a.d0 + j] = v[c];
        }
    }
}

template <int D, int GM>
__device__ void attn_tail_block(const AttnArgs& a, int bg, uint8_t* lds);

template <int D, int KB, int VB, int GMAX>
__global__ __launch_bounds__(256) void attn_partial_kernel(AttnArgs a) {
    using L = AttnLds<D>;
    constexpr int NKC = D / 64;                 // 64-channel runs of q.K^T per M-block
    constexpr int NNB = D / 16;                 // 16-channel N-blocks of p.V
    constexpr int KROW = D * KB / 8;            // packed bytes of one token's K row
    constexpr int VROW = TILE * VB / 8;         // packed bytes of one channel's V row
    constexpr int KW = KROW / 16;               // dwords of a lane group's K chunk
    constexpr int VW = VROW / 16;               // dwords of a lane group's V chunk
    constexpr int KRW = RunOrder<KB>::kWords, VRW = RunOrder<VB>::kWords;
    constexpr int KCB = TILE * KROW, VCB = D * VROW;
    constexpr int RBMAX = GMAX / 4;             // row blocks of 4 query heads
    constexpr int QPH = D / 4;                  // q' tasks per head (4 channels each)
    constexpr int QR = (GMAX * QPH + 63) / 64;  // q' tasks per lane
    constexpr int MK = 1 << (KB - 1), MV = 1 << (VB - 1);

    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    // wave-uniform (scalar), so the split's tile indices and table reads are too
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wpb = blockDim.x >> 6;
    const int G = a.n_q_heads / a.n_kv_heads;
    const int RB = GMAX == 4 ? 1 : (G + 3) >> 2;   // row blocks in use (one below 5 heads)
    const int sgroups = (a.n_splits + wpb - 1) / wpb;
    if (a.tail_in_grid) {
        // the fp16 tails, one 256-thread block per (b, KV head), after the splits' blocks
        const int pblocks = a.batch * a.n_kv_heads * sgroups;
        if ((int)blockIdx.x >= pblocks) {
            attn_tail_block<D, GMAX>(a, (int)blockIdx.x - pblocks, smem);
            return;
        }
    }
    const int bg = blockIdx.x / sgroups;
    const int split = (blockIdx.x % sgroups) * wpb + wave;
    if (split >= a.n_splits) return;
    const int b = bg / a.n_kv_heads, g = bg % a.n_kv_heads;
    // tiles of this (b, g): all tiles_per_seq, or the sequence's used blocks
    int ntiles = a.tiles_per_seq;
    if (a.table) ntiles = min(max(a.nblk[b], 0), a.tiles_per_seq);
    // strided splits: step k of split s reads tile s + k * n_splits
    const int t0 = 0;
    const int t1 = split < ntiles ? (ntiles - split + a.n_splits - 1) / a.n_splits : 0;
    if (t0 >= t1) {
        // nothing in this split: an empty partial (m = -inf, l = 0, acc = 0)
        float* ex = reinterpret_cast<float*>(smem);
        if (a.fuse_combine) __syncthreads();
        for (int k = lane; k < G * (D + 2); k += 64) {
            const int n = k / (D + 2), e = k % (D + 2);
            float* p = a.fuse_combine
                ? ex + ((size_t)split * G + n) * (D + 2)
                : a.ws + (((size_t)b * a.n_q_heads + g * G + n) * a.n_parts + split) * (D + 2);
            p[e] = (e == 0) ? -INFINITY : 0.0f;
        }
        if (a.fuse_combine) {
            __syncthreads();
            merge_splits_in_block<D>(a, ex, b, g, G, wave);
        }
        return;
    }

    uint8_t* lds = smem + (size_t)wave * L::bytes(G);
    uint16_t* kmeta = reinterpret_cast<uint16_t*>(lds + L::kmeta(G));
    uint16_t* vmeta = reinterpret_cast<uint16_t*>(lds + L::vmeta(G));
    uint8_t* qaimg = lds + L::qa(G);
    uint8_t* paimg = lds + L::pa(G);
    float* st_qz = reinterpret_cast<float*>(lds + L::stats(G));   // [4 RB] zero-point term
    float* st_iq = st_qz + 4 * RB;                                   // [4 RB] 1 / (q' scale * code scale)

    const int col = lane & 15;      // matrix-core row / column of this lane
    const int lgr = lane >> 4;      // matrix-core lane group: head of a score or output tile

    // Loads run one tile ahead, each issued once its registers are free: the
    // next tile's meta right after this tile's meta is in LDS, its K codes
    // after the q.K^T products, its V codes after the p.V products.  Every
    // load is unconditional, so each wait covers a fixed number of younger
    // loads: past the last tile the code loads see an empty buffer range
    // (zeros, no memory traffic) and the meta is re-read.
    constexpr int KC = 2 * L::KMH / 16, VC = 2 * L::VMH / 16;   // 16-byte meta chunks
    constexpr int MCH = (KC + VC + 63) / 64;                      // chunks per lane
    uint32_t kw[TILE / 16][KW];   // K codes: 8 blocks of 16 tokens, one chunk per lane
    uint32_t vw[NNB][VW];         // V codes: D/16 N-blocks of 16 channels
    uint4 mt[MCH];                // meta chunks
    // paged cache: the split's first 64 block ids are read once, one per
    // lane, so a tile's id is a lane read instead of a scalar load on the
    // prefetch path
    int blk_lane = 0;
    if (a.table && t0 + lane < t1) blk_lane = a.table[(size_t)b * a.tiles_per_seq + split + (t0 + lane) * a.n_splits];
    // pool index of tile ti of this (b, g) (past the split's end: its last
    // tile; a paged table entry outside the pool reads block 0)
    auto tile_index = [&](int ti) -> int64_t {
        const int tc = ti < t1 ? ti : t1 - 1;
        const int lt = split + tc * a.n_splits;
        if (!a.table) return (int64_t)bg * a.tiles_per_seq + lt;
        int64_t blk = (tc - t0 < 64) ? __builtin_amdgcn_readlane(blk_lane, tc - t0)
                                     : a.table[(size_t)b * a.tiles_per_seq + lt];
        if (blk < 0 || blk >= a.pool_blocks) blk = 0;
        return blk * a.n_kv_heads + g;
    };
    // codes through per-tile buffer descriptors: per-lane offsets fixed, the
    // block moves the scalar offset (every read stays inside the whole tile)
    const int kvo = tok_r0<VB>(col) * KROW + lgr * (KROW / 4);   // token tau(., col), lane group lgr
    const int vvo = col * VROW + lgr * (VROW / 4);               // channel col, lane group lgr
    auto load_k = [&](int ti) {
        // past the split's last tile the range is empty: the loads return zero
        // without touching memory, and the wait counts stay the same
        const auto r = make_rsrc(a.kc + tile_index(ti) * KCB, ti < t1 ? (uint32_t)KCB : 0u);
#pragma unroll
        for (int mb = 0; mb < TILE / 16; ++mb) {
            const int so = tok_delta<VB>(mb) * KROW;
            if constexpr (KW >= 4) {
#pragma unroll
                for (int w = 0; w < KW; w += 4) {
                    const uint4 v = buf_load16<kPolicyNT>(r, kvo + 4 * w, so);
                    kw[mb][w] = v.x; kw[mb][w + 1] = v.y; kw[mb][w + 2] = v.z; kw[mb][w + 3] = v.w;
                }
            } else if constexpr (KW == 2) {
                const uint2 v = buf_load8<kPolicyNT>(r, kvo, so);
                kw[mb][0] = v.x; kw[mb][1] = v.y;
            } else {
                kw[mb][0] = buf_load4<kPolicyNT>(r, kvo, so);
            }
        }
    };
    auto load_v = [&](int ti) {
        const auto r = make_rsrc(a.vc + tile_index(ti) * VCB, ti < t1 ? (uint32_t)VCB : 0u);
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb) {
            const int so = 16 * nb * VROW;
            if constexpr (VW == 4) {
                const uint4 v = buf_load16<kPolicyNT>(r, vvo, so);
                vw[nb][0] = v.x; vw[nb][1] = v.y; vw[nb][2] = v.z; vw[nb][3] = v.w;
            } else {
                const uint2 v = buf_load8<kPolicyNT>(r, vvo, so);
                vw[nb][0] = v.x; vw[nb][1] = v.y;
            }
        }
    };
    auto load_meta = [&](int ti) {
        const int64_t tile = tile_index(ti);
        const uint4* km = reinterpret_cast<const uint4*>(a.km + tile * L::KMH);
        const uint4* vm = reinterpret_cast<const uint4*>(a.vm + tile * L::VMH);
#pragma unroll
        for (int r = 0; r < MCH; ++r) {
            int k = lane + 64 * r;
            if (k >= KC + VC) k = 0;   // spare lanes re-read chunk 0
            const uint4* src = (k < KC) ? km + k : vm + (k - KC);
            mt[r] = *src;
        }
    };
    // The first tile, then the group's fp16 queries, go out before anything
    // waits.  A query row is read in the layout of wave_fwht (lane l holds
    // channels CPL l .. CPL l + CPL - 1, zero past head_dim; head_dim is a
    // multiple of 8, so no lane straddles it).
    load_meta(t0);
    load_k(t0);
    load_v(t0);
    constexpr int CPL = D / 64;
    using QRaw = typename QRowChunk<CPL>::type;
    QRaw qraw[GMAX];
    {
        const uint16_t* qg = a.q + ((size_t)b * a.n_q_heads + g * G) * a.d0 + CPL * lane;
        const bool in_row = CPL * lane < a.d0;
#pragma unroll
        for (int n = 0; n < GMAX; ++n)
            qraw[n] = (n < G && in_row) ? *reinterpret_cast<const QRaw*>(qg + (size_t)n * a.d0) : QRaw{};
    }

    // softmax state and accumulator of head 4 rb + lgr (channel 16 nb + col)
    float m_run[RBMAX], l_run[RBMAX];
    float acc[RBMAX][NNB];
#pragma unroll
    for (int rb = 0; rb < RBMAX; ++rb) {
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.0f;
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb) acc[rb][nb] = 0.0f;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the first tile and the queries, once

    // Rotated queries H q / sqrt(D) of the group, one transform per head,
    // staged as floats [G][D] in the q' image region (G D 4 bytes fit in its
    // ceil(G / 4) 16 D bytes; the first tile's q' digits overwrite them only
    // after the gather below).  q' tasks: task t = lane + 64 r covers head
    // n = t / QPH and the 4 channels of dword j of run (lane group gq, chunk kc):
    //   channel gq D/4 + 16 kc + base(j) + stride n', n' = 0..3
    float qh[QR][4];
    {
        float* qst = reinterpret_cast<float*>(qaimg);
#pragma unroll
        for (int n = 0; n < GMAX; ++n) {
            if (n < G) {
                float v[CPL];
                QRowChunk<CPL>::unpack(qraw[n], v);
                wave_fwht<D>(v);
#pragma unroll
                for (int c = 0; c < CPL; ++c) qst[n * D + CPL * lane + c] = v[c];
            }
        }
        wave_sync();
#pragma unroll
        for (int r = 0; r < QR; ++r) {
            const int t = lane + 64 * r;
            const int n = t / QPH, rem = t % QPH;
            const int gq = rem / (D / 16), rem2 = rem % (D / 16);
            const int kc = rem2 >> 2, j = rem2 & 3;
            const bool live = n < G;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ch = gq * (D / 4) + 16 * kc + RunOrder<KB>::base(j) + RunOrder<KB>::kStride * e;
                qh[r][e] = live ? qst[(live ? n : 0) * D + ch] : 0.0f;   // index kept inside the image
            }
        }
        wave_sync();
    }

    for (int ti = t0; ti < t1; ++ti) {
        // ---- meta of the tile into the wave's LDS, then the next tile's meta ----
        static_assert(L::vmeta(0) == 16 * KC, "meta images must be adjacent");
#pragma unroll
        for (int r = 0; r < MCH; ++r) {
            const uint4 v = mt[r];
            if (lane + 64 * r < KC + VC) reinterpret_cast<uint4*>(kmeta)[lane + 64 * r] = v;
        }
        load_meta(ti + 1);
        wave_sync();

        // ---- q' = qh * SK as four signed base-256 digits, zero-point term ----
#pragma unroll
        for (int r = 0; r < QR; ++r) {
            const int t = lane + 64 * r;
            if (GMAX > 4 && t >= 4 * RB * QPH) break;    // past the padded group (uniform)
            const int n = t / QPH, rem = t % QPH;
            const int gq = rem / (D / 16), rem2 = rem % (D / 16);
            const int kc = rem2 >> 2, j = rem2 & 3;
            float qv[4];
            float zt = 0.0f, mx = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ch = gq * (D / 4) + 16 * kc + RunOrder<KB>::base(j) + RunOrder<KB>::kStride * e;
                const float sk = h2f_bits(kmeta[ch]);
                const float zk = h2f_bits(kmeta[D + ch]);
                qv[e] = qh[r][e] * sk;
                zt = __builtin_fmaf(qh[r][e], __builtin_fmaf((float)MK, sk, zk), zt);
                mx = fmaxf(mx, fabsf(qv[e]));
            }
            zt = grp_sum<QPH>(zt);
            mx = grp_max<QPH>(mx);
            const float sq = fx_scale(mx);
            uint32_t xd[4], d[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) xd[e] = fx_digits(qv[e], sq);
            digit_dwords(xd, d);
            // rows 4 (n % 4) + digit of run (gq, kc) in row block n / 4: slot
            // 16 gq + 4 (n % 4) + digit of image (n / 4, kc), swizzled
            const int sl = (16 * gq + 4 * (n & 3)) ^ qa_swz<D>(gq, kc);
            uint8_t* dst = qaimg + ((n >> 2) * NKC + kc) * 1024 + 4 * j;
#pragma unroll
            for (int dg = 0; dg < 4; ++dg) *reinterpret_cast<uint32_t*>(dst + 16 * (sl ^ dg)) = d[dg];
            if (rem == 0) {
                st_qz[n] = zt;
                st_iq[n] = 1.0f / (sq * (float)(256 >> KB));   // the codes enter as 2^(8-KB) (c - MK)
            }
        }
        wave_sync();

        float s[RBMAX][TILE / 16];   // scores of head 4 rb + lgr, token tau(mb, col)
        {
            // ---- q.K^T: digit sums on the integer matrix cores ----
            v4i_t qa[RBMAX][NKC];
#pragma unroll
            for (int rb = 0; rb < RBMAX; ++rb) {
                if (rb < RB) {
#pragma unroll
                    for (int kc = 0; kc < NKC; ++kc)
                        qa[rb][kc] = *reinterpret_cast<const v4i_t*>(
                            qaimg + (rb * NKC + kc) * 1024 + 16 * (lane ^ qa_swz<D>(lane >> 4, kc)));
                }
            }
            float qz[RBMAX], iq[RBMAX];
#pragma unroll
            for (int rb = 0; rb < RBMAX; ++rb) {
                const int h = rb < RB ? 4 * rb + lgr : 0;
                qz[rb] = st_qz[h]; iq[rb] = st_iq[h];
            }
#pragma unroll
            for (int mb = 0; mb < TILE / 16; ++mb) {
                v4i_t kb[NKC];
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc) kb[kc] = code_bytes<KB>(&kw[mb][KRW * kc]);
                const float rk = h2f_bits(kmeta[2 * D + tok_r0<VB>(col) + tok_delta<VB>(mb)]);
#pragma unroll
                for (int rb = 0; rb < RBMAX; ++rb) {
                    if (rb < RB) {
                        v4i_t c = {0, 0, 0, 0};
#pragma unroll
                        for (int kc = 0; kc < NKC; ++kc)
                            c = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[rb][kc], kb[kc], c, 0, 0, 0);
                        s[rb][mb] = a.sm_scale * rk * __builtin_fmaf(limb_join(c), iq[rb], qz[rb]);
                    }
                }
            }
        }
        load_k(ti + 1);

        // ---- online softmax of head 4 rb + lgr over the tile; p' digits into the image ----
        float al[RBMAX], ip[RBMAX], pz[RBMAX];
        {
            float sv[TILE / 16], zv[TILE / 16];
#pragma unroll
            for (int mb = 0; mb < TILE / 16; ++mb) {
                const int tok = tok_r0<VB>(col) + tok_delta<VB>(mb);
                sv[mb] = h2f_bits(vmeta[tok]);
                zv[mb] = h2f_bits(vmeta[TILE + tok]);
            }
#pragma unroll
            for (int rb = 0; rb < RBMAX; ++rb) {
                if (rb < RB) {
                    float mt = s[rb][0];
#pragma unroll
                    for (int mb = 1; mb < TILE / 16; ++mb) mt = fmaxf(mt, s[rb][mb]);
                    mt = grp_max<16>(mt);
                    const float mnew = fmaxf(m_run[rb], mt);
                    al[rb] = exp2_fast((m_run[rb] - mnew) * kLog2e);
                    float p[TILE / 16], lt = 0.0f, pzs = 0.0f, mxp = 0.0f;
#pragma unroll
                    for (int mb = 0; mb < TILE / 16; ++mb) {
                        p[mb] = exp2_fast((s[rb][mb] - mnew) * kLog2e);
                        lt += p[mb];
                        pzs = __builtin_fmaf(p[mb], __builtin_fmaf((float)MV, sv[mb], zv[mb]), pzs);
                        p[mb] *= sv[mb];            // p' = p SV
                        mxp = fmaxf(mxp, p[mb]);
                    }
                    lt = grp_sum<16>(lt);
                    pz[rb] = grp_sum<16>(pzs);
                    mxp = grp_max<16>(mxp);
                    m_run[rb] = mnew;
                    l_run[rb] = l_run[rb] * al[rb] + lt;
                    const float sp = fx_scale(mxp);
                    ip[rb] = 1.0f / (sp * (float)(256 >> VB));   // the codes enter as 2^(8-VB) (c - MV)
                    // run m of lane group col / 4, dword col % 4, rows 4 lgr + digit
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        uint32_t xd[4], d[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) xd[e] = fx_digits(p[4 * m + e], sp);
                        digit_dwords(xd, d);
                        // slot 16 (col / 4) + 4 lgr + digit, swizzled by col / 4
                        uint8_t* dst = paimg + (rb * 2 + m) * 1024 + 16 * (16 * (col >> 2) + 4 * lgr) + 4 * (col & 3);
#pragma unroll
                        for (int dg = 0; dg < 4; ++dg)
                            *reinterpret_cast<uint32_t*>(dst + 16 * (dg ^ (col >> 2))) = d[dg];
                    }
                }
            }
        }
        wave_sync();

        // ---- p.V: digit sums on the integer matrix cores, accumulator update ----
        {
            v4i_t pa[RBMAX][2];
#pragma unroll
            for (int rb = 0; rb < RBMAX; ++rb) {
                if (rb < RB) {
#pragma unroll
                    for (int m = 0; m < 2; ++m)
                        pa[rb][m] = *reinterpret_cast<const v4i_t*>(paimg + (rb * 2 + m) * 1024 + 16 * (lane ^ (lane >> 4)));
                }
            }
#pragma unroll
            for (int nb = 0; nb < NNB; ++nb) {
                const v4i_t vb0 = code_bytes<VB>(&vw[nb][0]);
                const v4i_t vb1 = code_bytes<VB>(&vw[nb][VRW]);
                const float cv = h2f_bits(vmeta[2 * TILE + 16 * nb + col]);
#pragma unroll
                for (int rb = 0; rb < RBMAX; ++rb) {
                    if (rb < RB) {
                        v4i_t c = {0, 0, 0, 0};
                        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(pa[rb][0], vb0, c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(pa[rb][1], vb1, c, 0, 0, 0);
                        const float upd = cv * __builtin_fmaf(limb_join(c), ip[rb], pz[rb]);
                        acc[rb][nb] = __builtin_fmaf(acc[rb][nb], al[rb], upd);
                    }
                }
            }
        }
        load_v(ti + 1);
        wave_sync();
    }

    // ---- partial result of this split: (m, l, acc[D]) per query head, to
    // the workspace, or (all splits of this (b, g) in this workgroup) to LDS
    // once every wave is done with its own region, merged in the block ----
    float* ex = reinterpret_cast<float*>(smem);
    if (a.fuse_combine) __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RBMAX; ++rb) {
        const int n = 4 * rb + lgr;
        if (rb < RB && n < G) {
            float* p = a.fuse_combine
                ? ex + ((size_t)split * G + n) * (D + 2)
                : a.ws + (((size_t)b * a.n_q_heads + g * G + n) * a.n_parts + split) * (D + 2);
#pragma unroll
            for (int nb = 0; nb < NNB; ++nb) p[2 + 16 * nb + col] = acc[rb][nb];
            if (col == 0) {
                p[0] = m_run[rb];
                p[1] = l_run[rb];
            }
        }
    }
    if (a.fuse_combine) {
        __syncthreads();
        merge_splits_in_block<D>(a, ex, b, g, G, wave);
    }
}

template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
    // one wavefront per (b, query head), four per workgroup
    constexpr int CPL = D / 64;
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);   // b * n_q_heads + h
    if (bh >= a.batch * a.n_q_heads) return;
    const float* p = a.ws + (size_t)bh * a.n_parts * (D + 2);
    float M = -INFINITY, L = 0.0f;
    float v[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] = 0.0f;
    if (a.n_parts <= kCombineParts) {
        // Few parts: every load goes out at once (lane s: part s's max and
        // sum; every lane: its CPL channels of each part's accumulator), so
        // the wave waits on memory once.  Same sums, in the same order, as
        // the general path below.
        float ms = -INFINITY, ls = 0.0f;
        if (lane < a.n_parts) {
            ms = p[(size_t)lane * (D + 2)];
            ls = p[(size_t)lane * (D + 2) + 1];
        }
        float pv[kCombineParts][CPL];
#pragma unroll
        for (int k = 0; k < kCombineParts; ++k)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                pv[k][c] = k < a.n_parts ? p[(size_t)(k < a.n_parts ? k : 0) * (D + 2) + 2 + CPL * lane + c]
                                         : 0.0f;   // the address stays inside this head's parts
        M = ms;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
        const float w = (ms != -INFINITY) ? exp2f((ms - M) * kLog2e) : 0.0f;
        L = ls * w;
#pragma unroll
        for (int k = 0; k < kCombineParts; ++k) {
            const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
#pragma unroll
            for (int c = 0; c < CPL; ++c) v[c] = __builtin_fmaf(pv[k][c], wk, v[c]);
        }
    } else {
        // global max over the parts (lanes stride the parts)
        for (int s = lane; s < a.n_parts; s += 64) M = fmaxf(M, p[(size_t)s * (D + 2)]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
        // the normaliser and the weighted sum of the parts' accumulators, CPL
        // channels per lane.  In each chunk of 64 parts, lane k computes part
        // k's weight and the loop reads it back lane by lane, so that the
        // accumulator loads of successive parts do not wait on one another.
        for (int base = 0; base < a.n_parts; base += 64) {
            const int s = base + lane;
            float w = 0.0f;
            if (s < a.n_parts) {
                const float ms = p[(size_t)s * (D + 2)];
                if (ms != -INFINITY) {
                    w = exp2f((ms - M) * kLog2e);
                    L += p[(size_t)s * (D + 2) + 1] * w;
                }
            }
            const int cnt = min(64, a.n_parts - base);
            const float* pb = p + (size_t)base * (D + 2) + 2 + CPL * lane;
#pragma unroll 4
            for (int k = 0; k < cnt; ++k) {
                const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
#pragma unroll
                for (int c = 0; c < CPL; ++c) v[c] = __builtin_fmaf(pb[(size_t)k * (D + 2) + c], wk, v[c]);
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
    const float il = (L > 0.0f) ? 1.0f / L : 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] *= il;
    wave_fwht<D>(v);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int j = CPL * lane + c;
        if (j < a.d0) a.out[(size_t)bh * a.d0 + j] = v[c];
    }
}

// ---- fp16 tail of a paged sequence (at most 128 tokens, not yet a tile) ----
// One 256-thread workgroup per (b, KV head): plain fp32 attention of the
// group's query heads over the tail's fp16 K and V, in the original channel
// domain (the scores are the same in either domain, the rotation being
// orthonormal).  Its partial (m, l, acc) goes to the last slot of the
// workspace with acc rotated (H acc / sqrt(D)), so that the combine kernel's
// final rotation returns it to the original domain together with the packed
// tiles' slots.  Query rows GM > G are zero and their results are dropped.
//   scores: thread pair (2t, 2t+1) holds token t, one half of the channels
//           each, every 16-byte load of the half in flight;
//   p . V:  thread (s, c) sums tokens s, s + NS, ... over channel chunk c
//           (8 channels, one 16-byte load per token); the NS token slices
//           are reduced across lanes, then across the four waves in LDS.
// LDS of one tail workgroup: q (then the summed acc) [GM][D], p [TILE][GM],
// per-wave max and sum [2][4][GM], final m and l [2][GM].
template <int D, int GM>
struct TailLds {
    static constexpr int kBytes = 4 * (GM * D + TILE * GM + 8 * GM + 2 * GM);
};

// The tail of (b, KV head) bg, by one 256-thread workgroup (lds: TailLds
// bytes, 16-byte aligned).
template <int D, int GM>
__device__ void attn_tail_block(const AttnArgs& a, int bg, uint8_t* lds) {
    constexpr int NT = 256;
    constexpr int HC = D / 2;                      // channels per score thread
    constexpr int CPR = D / 8;                     // 16-byte chunks of a padded row
    constexpr int NS = NT / CPR;                   // token slices of the p . V phase
    constexpr int TPS = TILE / NS;                 // tokens per slice
    constexpr int SPW = 64 / CPR;                  // slices per wave
    float* qs = reinterpret_cast<float*>(lds);     // q; then the summed acc
    float* ps = qs + GM * D;                       // p[t][n]
    float (*red)[4][GM] = reinterpret_cast<float (*)[4][GM]>(ps + TILE * GM);   // per-wave max and sum
    float (*ml)[GM] = reinterpret_cast<float (*)[GM]>(ps + TILE * GM + 8 * GM); // final m and l
    float* os = qs;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int b = bg / a.n_kv_heads, g = bg % a.n_kv_heads;
    const int G = a.n_q_heads / a.n_kv_heads;
    const int d0 = a.d0;
    const int T = min(max(a.tail_len[b], 0), TILE);
    const int slot = a.n_parts - 1;
    auto part = [&](int n) {
        return a.ws + (((size_t)b * a.n_q_heads + g * G + n) * a.n_parts + slot) * (D + 2);
    };
    if (T == 0) {
        for (int k = tid; k < G * (D + 2); k += NT)
            part(k / (D + 2))[k % (D + 2)] = (k % (D + 2) == 0) ? -INFINITY : 0.0f;
        return;
    }
    for (int k = tid; k < GM * D; k += NT) {
        const int n = k / D, j = k % D;
        qs[k] = (n < G && j < d0) ? h2f_bits(a.q[((size_t)b * a.n_q_heads + g * G + n) * d0 + j]) : 0.0f;
    }
    __syncthreads();
    const uint16_t* kt = a.k_tail + (size_t)bg * TILE * d0;
    const uint16_t* vt = a.v_tail + (size_t)bg * TILE * d0;

    // scores
    const int t = tid >> 1, h = tid & 1;
    float sc[GM];
#pragma unroll
    for (int n = 0; n < GM; ++n) sc[n] = 0.0f;
    if (t < T) {
        uint4 w[HC / 8];
#pragma unroll
        for (int c = 0; c < HC / 8; ++c) {
            const int j = h * HC + 8 * c;
            w[c] = (j < d0) ? *reinterpret_cast<const uint4*>(kt + (size_t)t * d0 + j)
                            : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int c = 0; c < HC / 8; ++c) {
            const uint32_t wd[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float kv = h2f_bits((uint16_t)((e & 1) ? (wd[e >> 1] >> 16) : (wd[e >> 1] & 0xFFFF)));
                const int j = h * HC + 8 * c + e;
#pragma unroll
                for (int n = 0; n < GM; ++n) sc[n] = __builtin_fmaf(qs[n * D + j], kv, sc[n]);
            }
        }
    }
#pragma unroll
    for (int n = 0; n < GM; ++n) sc[n] = a.sm_scale * (sc[n] + __shfl_xor(sc[n], 1));

    // softmax statistics over the T tokens (each token is held by two lanes)
#pragma unroll
    for (int n = 0; n < GM; ++n) {
        float mx = (t < T) ? sc[n] : -INFINITY;
        for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        if (lane == 0) red[0][wv][n] = mx;
    }
    __syncthreads();
    float pn[GM];
#pragma unroll
    for (int n = 0; n < GM; ++n) {
        const float mx = fmaxf(fmaxf(red[0][0][n], red[0][1][n]), fmaxf(red[0][2][n], red[0][3][n]));
        pn[n] = (t < T) ? exp2f((sc[n] - mx) * kLog2e) : 0.0f;
        float sum = h ? 0.0f : pn[n];
        for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
        if (lane == 0) red[1][wv][n] = sum;
        if (tid == 0) ml[0][n] = mx;
    }
    if (h == 0) {
#pragma unroll
        for (int n = 0; n < GM; ++n) ps[t * GM + n] = pn[n];
    }
    __syncthreads();
    if (tid < GM) ml[1][tid] = (red[1][0][tid] + red[1][1][tid]) + (red[1][2][tid] + red[1][3][tid]);

    // p . V
    const int c = tid % CPR, sl = tid / CPR;
    const bool cok = 8 * c < d0;
    uint4 v[TPS];
#pragma unroll
    for (int i = 0; i < TPS; ++i) {
        const int tt = sl + NS * i;
        v[i] = (cok && tt < T) ? *reinterpret_cast<const uint4*>(vt + (size_t)tt * d0 + 8 * c)
                               : make_uint4(0u, 0u, 0u, 0u);
    }
    float acc[GM][8];
#pragma unroll
    for (int n = 0; n < GM; ++n)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[n][e] = 0.0f;
#pragma unroll
    for (int i = 0; i < TPS; ++i) {
        const int tt = sl + NS * i;
        const uint32_t wd[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float vv = h2f_bits((uint16_t)((e & 1) ? (wd[e >> 1] >> 16) : (wd[e >> 1] & 0xFFFF)));
#pragma unroll
            for (int n = 0; n < GM; ++n) acc[n][e] = __builtin_fmaf(ps[tt * GM + n], vv, acc[n][e]);
        }
    }
    // slices of one wave: lanes c + CPR k
#pragma unroll
    for (int o = CPR; o < 64; o <<= 1)
#pragma unroll
        for (int n = 0; n < GM; ++n)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[n][e] += __shfl_xor(acc[n][e], o);
    // waves in turn (q is dead: every thread passed the statistics barriers)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        if (wv == w && lane < CPR) {
#pragma unroll
            for (int n = 0; n < GM; ++n)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    os[n * D + 8 * c + e] = (w == 0) ? acc[n][e] : os[n * D + 8 * c + e] + acc[n][e];
        }
        __syncthreads();
    }
    static_assert(SPW >= 1 && NS * CPR == NT, "tail thread mapping");
    // rotate each query's acc: H acc / sqrt(D)
#pragma unroll
    for (int hs = 1; hs < D; hs <<= 1) {
        for (int k = tid; k < G * (D / 2); k += NT) {
            const int r = k / (D / 2), pidx = k % (D / 2);
            const int lo = (pidx / hs) * 2 * hs + (pidx % hs), hi = lo + hs;
            const float x = os[r * D + lo], y = os[r * D + hi];
            os[r * D + lo] = x + y;
            os[r * D + hi] = x - y;
        }
        __syncthreads();
    }
    const float rs = 1.0f / __builtin_sqrtf((float)D);
    for (int k = tid; k < G * (D + 2); k += NT) {
        const int n = k / (D + 2), e = k % (D + 2);
        part(n)[e] = (e >= 2) ? os[n * D + e - 2] * rs : ml[e][n];
    }
}

// One workgroup per (b, KV head), when the tails are not run by the partial
// kernel's grid.
template <int D, int GM>
__global__ __launch_bounds__(256) void attn_tail_kernel(AttnArgs a) {
    __shared__ __align__(16) uint8_t lds[TailLds<D, GM>::kBytes];
    attn_tail_block<D, GM>(a, blockIdx.x, lds);
}

__global__ void fill_zero_kernel(float* out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = 0.0f;
}

template <int D, int KB, int VB, int GMAX>
static hipError_t launch_att(const AttnArgs& args, hipStream_t s) {
    AttnArgs a = args;
    const int G = a.n_q_heads / a.n_kv_heads;
    if (a.n_splits > 0) {
        const int per_wave = AttnLds<D>::bytes(G);
        int wpb = 65536 / per_wave;
        if (wpb > 4) wpb = 4;
        if (wpb < 1) wpb = 1;
        // Without a block table or tails, when a (b, g)'s splits fit one
        // workgroup, they run as its waves and merge there: no combine launch
        // and no partials in memory.  The merge's exchange, n_splits x G x
        // (D + 2) floats, fits the waves' LDS regions (each holds the q' image
        // of G heads, 16 D ceil(G / 4) bytes or more).
        if (!a.table && !a.tail_len && a.n_splits <= wpb &&
            (size_t)a.n_splits * G * (D + 2) * sizeof(float) <= (size_t)per_wave * a.n_splits) {
            wpb = a.n_splits;
            a.fuse_combine = 1;
        }
        const int64_t sgroups = (a.n_splits + wpb - 1) / wpb;
        int64_t blocks = (int64_t)a.batch * a.n_kv_heads * sgroups;
        // A paged call's fp16 tails run as extra blocks of the same grid where
        // those blocks have the tail's 256 threads and its LDS, so they overlap
        // the splits instead of following them.
        if (a.tail_len && wpb == 4 && TailLds<D, GMAX>::kBytes <= per_wave * wpb) {
            a.tail_in_grid = 1;
            blocks += (int64_t)a.batch * a.n_kv_heads;
        }
        hipLaunchKernelGGL((attn_partial_kernel<D, KB, VB, GMAX>), dim3((unsigned)blocks),
                           dim3(64 * wpb), (size_t)per_wave * wpb, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.tail_len && !a.tail_in_grid) {
        hipLaunchKernelGGL((attn_tail_kernel<D, GMAX>), dim3((unsigned)(a.batch * a.n_kv_heads)),
                           dim3(256), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.fuse_combine) return hipSuccess;
    hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((unsigned)((a.batch * a.n_q_heads + 3) / 4)),
                       dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int D, int KB, int VB>
static hipError_t launch_att_g(const AttnArgs& a, hipStream_t s) {
    const int G = a.n_q_heads / a.n_kv_heads;
    if (G <= 4) return launch_att<D, KB, VB, 4>(a, s);
    return launch_att<D, KB, VB, 16>(a, s);
}

template <int D>
static hipError_t launch_att_bits(const AttnArgs& a, int kb, int vb, hipStream_t s) {
    if (kb == 4 && vb == 2) return launch_att_g<D, 4, 2>(a, s);
    if (kb == 4 && vb == 4) return launch_att_g<D, 4, 4>(a, s);
    if (kb == 2 && vb == 2) return launch_att_g<D, 2, 2>(a, s);
    return launch_att_g<D, 2, 4>(a, s);
}

hipError_t launch_attention(const AttnArgs& a, int D, int kb, int vb, hipStream_t s) {
    if (a.tiles_per_seq == 0 && !a.tail_len) {
        const int64_t n = (int64_t)a.batch * a.n_q_heads * a.d0;
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           a.out, n);
        return hipGetLastError();
    }
    if (D == 64) return launch_att_bits<64>(a, kb, vb, s);
    if (D == 128) return launch_att_bits<128>(a, kb, vb, s);
    return launch_att_bits<256>(a, kb, vb, s);
}

}  // namespace kvarn
