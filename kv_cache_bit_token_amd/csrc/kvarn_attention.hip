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
//   qh  = H q / sqrt(D)                          once per (b, query head)
//   s_t = sm * RK_t * ( sum_j (qh_j SK_j)(code_tj - mk) + sum_j qh_j (ZK_j + mk SK_j) )
//   online softmax over the tiles of a split
//   acc_j = CV_j * ( sum_t (p_t SV_t)(code_tj - mv) + sum_t p_t (ZV_t + mv SV_t) )
//   o = H (acc / l) / sqrt(D), first head_dim channels      (combine kernel)
// Centring the codes keeps both terms of each sum small (ZK is the group
// minimum, so the uncentred terms would be large and of opposite sign).
//
// Matrix cores.  Both contractions run on v_mfma_f32_16x16x32_f16 (two
// 16-deep operands side by side); the layouts below are those of the 16-deep
// operands:
//   q.K^T : A = codes (16 tokens x 16 channels), B = q' (16 channels x the
//           GQA group's query heads, padded to 16), C = scores;
//   p.V   : A = p' (query heads x 16 tokens), B = codes (16 tokens x 16
//           channels), C = partial outputs.
// Codes become exact fp16 values (c - 2^(b-1)) with a magic-number unpack;
// q' = qh * SK and p' = p * SV are fp32 values split into fp16 hi + lo
// parts (each scaled by a power of two per tile), so each product is exact
// and the fp32 accumulation keeps fp32 accuracy.  The contraction axis is
// permuted so every lane reads one contiguous run of packed codes: the K
// row chunk of its token (16 bytes at K4, D = 128) and the V row chunk of
// its channel (8 bytes at V2); the same permutation orders q' and p'.
//
// Work split: each wavefront owns one split (a run of tiles) of one
// (b, KV head) and every query head of that head's GQA group; waves never
// synchronise with each other.  Per tile, small per-wave LDS images move
// q', the scores, p' and the p.V results between the matrix-core layouts and
// dense layouts in which all 64 lanes do the softmax and the updates.  A
// combine kernel merges the splits' (max, sum, acc) and undoes the rotation.
#include "kvarn_device.hpp"
#include "kvarn_internal.hpp"
#include "kvarn_rsrc.hpp"

namespace kvarn {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kTargetWaves = 8192;   // splits in flight: 8 waves per SIMD on 256 CUs
constexpr float kLog2e = 1.4426950408889634f;

void attention_plan(int batch, int n_kv_heads, int tiles_per_seq, int* n_splits,
                    int* tiles_per_split) {
    const int64_t pairs = (int64_t)batch * n_kv_heads;
    int ns = 1;
    if (pairs > 0 && tiles_per_seq > 0) {
        int64_t want = (kTargetWaves + pairs - 1) / pairs;
        if (want > tiles_per_seq) want = tiles_per_seq;
        if (want < 1) want = 1;
        ns = (int)want;
    }
    int tps = tiles_per_seq > 0 ? (tiles_per_seq + ns - 1) / ns : 0;
    if (tps > 0) ns = (tiles_per_seq + tps - 1) / tps;
    *n_splits = ns;
    *tiles_per_split = tps;
}

size_t attention_workspace_bytes(int batch, int n_q_heads, int D, int n_parts) {
    return (size_t)batch * n_q_heads * n_parts * (D + 2) * sizeof(float);
}

// byte offset of the rotated queries: the partials rounded up to 256 bytes
static size_t qrot_offset(int batch, int n_q_heads, int D, int n_parts) {
    return (attention_workspace_bytes(batch, n_q_heads, D, n_parts) + 255) & ~(size_t)255;
}

size_t packed_attention_workspace_bytes(int batch, int n_q_heads, int D, int n_parts) {
    return qrot_offset(batch, n_q_heads, D, n_parts) + (size_t)batch * n_q_heads * D * sizeof(float);
}

// ---- b-bit codes -> exact fp16 (code - 2^(b-1)) -----------------------------
// A packed dword holds N = 32/b codes.  Pair k takes codes k and k + N/2 (bits
// b*k and b*k + 16) into the two halves of a dword.  A code sitting at bit s
// of its half (s + b <= 10) is OR-ed as it stands into the mantissa of a
// magic fp16 whose unit in the last place is 2^-s, so the half reads
// magic + code exactly; one packed fp16 add then subtracts magic + 2^(b-1).
// Only the pairs whose bits lie above the mantissa need a shift, one shared
// per dword: 4-bit pairs 0, 1 sit at s = 0, 4 and pairs 2, 3 at s = 0, 4 of
// w >> 8; 2-bit pairs 0..4 at s = 0, 2, 4, 6, 8 and pairs 5..7 at s = 0, 2, 4
// of w >> 10.
template <int B> struct Codes;
template <> struct Codes<4> {
    static constexpr int N = 8, SPLIT = 2, HI_SHIFT = 8;
    static constexpr float MID = 8.0f;
};
template <> struct Codes<2> {
    static constexpr int N = 16, SPLIT = 5, HI_SHIFT = 10;
    static constexpr float MID = 2.0f;
};

// The magic halves of the SPLIT bit positions, both halves of a dword, held
// in vector registers for the whole kernel, and the code masks of both
// halves, held in scalar registers.  Both are made opaque to the compiler so
// it does not rematerialise them at every use; with the mask in a scalar
// register, (x & mask) | magic is one v_and_or_b32 (a literal mask would
// need an AND and an OR).
template <int B>
struct CodeMagic {
    uint32_t m[Codes<B>::SPLIT];
    uint32_t mask[Codes<B>::SPLIT];
    __device__ __forceinline__ void init() {
#pragma unroll
        for (int i = 0; i < Codes<B>::SPLIT; ++i) {
            const uint32_t f = (25u - (uint32_t)(B * i)) << 10;   // exponent field of 2^(10 - s)
            asm volatile("v_mov_b32 %0, %1" : "=v"(m[i]) : "s"(f | (f << 16)));
            const uint32_t mk = ((1u << B) - 1u) << (B * i);
            asm volatile("s_mov_b32 %0, %1" : "=s"(mask[i]) : "i"(mk | (mk << 16)));
        }
    }
};

// pair k of dword w (wh = w >> HI_SHIFT), as two fp16 values code - 2^(b-1)
template <int B>
__device__ __forceinline__ uint32_t code_pair(uint32_t w, uint32_t wh, int k, const CodeMagic<B>& cm) {
    using C = Codes<B>;
    const int i = k < C::SPLIT ? k : k - C::SPLIT;
    const int s = B * i;                                      // bit of the code in its half
    const uint32_t x = k < C::SPLIT ? w : wh;
    const uint32_t v = (x & cm.mask[i]) | cm.m[i];
    const _Float16 sub = (_Float16)(-((float)(1 << (10 - s)) + C::MID));
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, v) + (h2_t){sub, sub});
}

// Matrix operand kb (4 fp16 values) out of a lane's run of packed dwords.
// Operand kb uses dword d = kb / (N/4) and pairs 2*k2, 2*k2 + 1 (k2 = kb mod
// N/4); element e holds code 2*k2 + (e >> 1) + (N/2)*(e & 1) of that dword.
template <int B, int NW>
__device__ __forceinline__ h4_t code_operand(const uint32_t (&w)[NW], int kb, const CodeMagic<B>& cm) {
    constexpr int Q = Codes<B>::N / 4;
    const int d = kb / Q, k2 = kb % Q;
    const uint32_t wh = w[d] >> Codes<B>::HI_SHIFT;
    const uint32_t lo = code_pair<B>(w[d], wh, 2 * k2, cm);
    const uint32_t hi = code_pair<B>(w[d], wh, 2 * k2 + 1, cm);
    return __builtin_bit_cast(h4_t, make_uint2(lo, hi));
}

// Two 16-deep operands side by side as one 32-deep operand of
// v_mfma_f32_16x16x32_f16.  A and B pair their elements by (lane group,
// element) alike, so concatenating operands 2j and 2j + 1 on both sides sums
// exactly the products the two 16-deep instructions summed.
__device__ __forceinline__ h8_t cat8(h4_t x, h4_t y) {
    return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Runs of a dense task that covers operands kbase, kbase + 1 (kbase even) of a
// lane group: the 8 elements are run0 + 0..3 and run1 + 0..3, stored
// interleaved [r0_0, r1_0, r0_1, r1_1, r0_2, r1_2, r0_3, r1_3].
template <int B>
__device__ __forceinline__ int run0_of(int group_base, int kbase) {
    constexpr int N = Codes<B>::N, Q = N / 4;
    return group_base + N * (kbase / Q) + 2 * (kbase % Q);
}

// reductions over aligned groups of W lanes (W = 8, 16, 32)
template <int W>
__device__ __forceinline__ float grp_sum(float v) {
    v += dpp<DPP_XOR1>(v);
    v += dpp<DPP_XOR2>(v);
    v += dpp<DPP_HMIR>(v);
    if constexpr (W >= 16) v += dpp<DPP_ROR8>(v);
    if constexpr (W >= 32) v += __shfl_xor(v, 16);
    return v;
}
template <int W>
__device__ __forceinline__ float grp_max(float v) {
    v = fmaxf(v, dpp<DPP_XOR1>(v));
    v = fmaxf(v, dpp<DPP_XOR2>(v));
    v = fmaxf(v, dpp<DPP_HMIR>(v));
    if constexpr (W >= 16) v = fmaxf(v, dpp<DPP_ROR8>(v));
    if constexpr (W >= 32) v = fmaxf(v, __shfl_xor(v, 16));
    return v;
}

// power-of-two scale s with max * s < 2^10 (1 for max == 0)
__device__ __forceinline__ float pow2_scale(float mx) {
    if (!(mx > 0.0f)) return 1.0f;
    int e;
    (void)frexpf(mx, &e);          // mx = m * 2^e, m in [0.5, 1)
    return ldexpf(1.0f, 10 - e);
}

__device__ __forceinline__ void split_hi_lo(float x, _Float16& hi, _Float16& lo) {
    hi = (_Float16)x;
    lo = (_Float16)(x - (float)hi);
}

// Per-wave LDS layout (bytes), for GQA group size G (padded to GP = 4k).
template <int D>
struct AttnLds {
    static constexpr int KMH = 2 * D + TILE, VMH = 2 * TILE + D;
    static constexpr int NKB = D / 16;
    __host__ __device__ static constexpr int kmeta(int) { return 0; }
    __host__ __device__ static constexpr int vmeta(int) { return 2 * KMH; }
    __host__ __device__ static constexpr int bq(int) { return 2 * KMH + 2 * VMH; }
    __host__ __device__ static constexpr int sc(int G) { return bq(G) + 64 * G * NKB; }
    __host__ __device__ static constexpr int pa(int G) { return sc(G) + 512 * G; }
    __host__ __device__ static constexpr int pvc(int G) { return pa(G) + 512 * G; }
    __host__ __device__ static constexpr int stats(int G) { return pvc(G) + 4 * D * ((G + 3) & ~3); }
    __host__ __device__ static constexpr int bytes(int G) { return stats(G) + 16 * G + 16; }
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

// Rotated query of one (b, query head): H q / sqrt(D) over the padded width,
// once per head for every split that reads it.  One wavefront per head, four
// heads per workgroup.
template <int D>
__global__ __launch_bounds__(256) void attn_rotate_q_kernel(AttnArgs a) {
    constexpr int CPL = D / 64;
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);   // b * n_q_heads + h
    if (bh >= a.batch * a.n_q_heads) return;
    float v[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int j = CPL * lane + c;
        v[c] = (j < a.d0) ? h2f_bits(a.q[(size_t)bh * a.d0 + j]) : 0.0f;
    }
    wave_fwht<D>(v);
#pragma unroll
    for (int c = 0; c < CPL; ++c) a.qrot[(size_t)bh * D + CPL * lane + c] = v[c];
}

template <int D, int KB, int VB, int GMAX>
__global__ __launch_bounds__(256) void attn_partial_kernel(AttnArgs a) {
    using L = AttnLds<D>;
    constexpr int NKB = D / 16;                 // q.K^T operands per M-block (channels)
    constexpr int NVB = TILE / 16;              // p.V operands per N-block (tokens)
    constexpr int KROW = D * KB / 8;            // packed bytes of one token's K row
    constexpr int VROW = TILE * VB / 8;         // packed bytes of one channel's V row
    constexpr int KW = KROW / 16;               // dwords of a lane group's K chunk
    constexpr int VW = VROW / 16;               // dwords of a lane group's V chunk
    constexpr int KCB = TILE * KROW, VCB = D * VROW;
    constexpr int QT = D / 8;                   // dense tasks per query (channels)
    constexpr int QTMAX = (GMAX * QT + 63) / 64;
    constexpr int STMAX = (GMAX * 16 + 63) / 64;
    constexpr int CPL_E = D / 64;               // epilogue channels per lane
    constexpr float MK = Codes<KB>::MID, MV = Codes<VB>::MID;

    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    // wave-uniform (scalar), so the split's tile indices and table reads are too
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wpb = blockDim.x >> 6;
    const int G = a.n_q_heads / a.n_kv_heads;
    const int GP = (G + 3) & ~3;
    const int sgroups = (a.n_splits + wpb - 1) / wpb;
    const int bg = blockIdx.x / sgroups;
    const int split = (blockIdx.x % sgroups) * wpb + wave;
    if (split >= a.n_splits) return;
    const int b = bg / a.n_kv_heads, g = bg % a.n_kv_heads;
    // tiles of this (b, g): all tiles_per_seq, or the sequence's used blocks
    int ntiles = a.tiles_per_seq;
    if (a.table) ntiles = min(max(a.nblk[b], 0), a.tiles_per_seq);
    const int t0 = split * a.tiles_per_split;
    const int t1 = min(t0 + a.tiles_per_split, ntiles);
    if (t0 >= t1) {
        // nothing in this split: an empty partial (m = -inf, l = 0, acc = 0)
        for (int k = lane; k < G * (D + 2); k += 64) {
            const int n = k / (D + 2), e = k % (D + 2);
            float* p = a.ws + (((size_t)b * a.n_q_heads + g * G + n) * a.n_parts + split) * (D + 2);
            p[e] = (e == 0) ? -INFINITY : 0.0f;
        }
        return;
    }

    uint8_t* lds = smem + (size_t)wave * L::bytes(G);
    uint16_t* kmeta = reinterpret_cast<uint16_t*>(lds + L::kmeta(G));
    uint16_t* vmeta = reinterpret_cast<uint16_t*>(lds + L::vmeta(G));
    uint8_t* bqimg = lds + L::bq(G);
    float* sc = reinterpret_cast<float*>(lds + L::sc(G));
    uint8_t* paimg = lds + L::pa(G);
    float* pvc = reinterpret_cast<float*>(lds + L::pvc(G));
    float* st = reinterpret_cast<float*>(lds + L::stats(G));
    float* st_qz = st;              // [G] zero-point term of the scores
    float* st_iq = st + G;          // [G] 1 / q' scale
    float* st_al = st + 2 * G;      // [G] softmax rescale of this tile
    float* st_pz = st + 3 * G;      // [G] zero-point term of p.V
    float* st_ip = st + 4 * G;      // [1] 1 / p' scale

    const int mrow = lane & 15;     // MFMA row / column index of this lane
    const int mgrp = lane >> 4;     // MFMA k-group of this lane

    // Loads run one tile ahead, each issued once its registers are free: the
    // next tile's meta right after this tile's meta is in LDS, its K codes
    // after the q.K^T products, its V codes after the p.V products.  Every
    // load is unconditional, so each wait covers a fixed number of younger
    // loads: past the last tile the code loads see an empty buffer range
    // (zeros, no memory traffic) and the meta is re-read.
    constexpr int KC = 2 * L::KMH / 16, VC = 2 * L::VMH / 16;   // 16-byte meta chunks
    constexpr int MCH = (KC + VC + 63) / 64;                      // chunks per lane
    uint32_t kw[TILE / 16][KW];   // K codes: 8 M-blocks of 16 tokens, one run per lane
    uint32_t vw[NKB][VW];         // V codes: D/16 N-blocks of 16 channels
    uint4 mt[MCH];                // meta chunks
    // paged cache: the split's first 64 block ids are read once, one per
    // lane, so a tile's id is a lane read instead of a scalar load on the
    // prefetch path
    int blk_lane = 0;
    if (a.table && t0 + lane < t1) blk_lane = a.table[(size_t)b * a.tiles_per_seq + t0 + lane];
    // pool index of tile ti of this (b, g) (past the split's end: its last
    // tile; a paged table entry outside the pool reads block 0)
    auto tile_index = [&](int ti) -> int64_t {
        const int tc = ti < t1 ? ti : t1 - 1;
        if (!a.table) return (int64_t)bg * a.tiles_per_seq + tc;
        int64_t blk = (tc - t0 < 64) ? __builtin_amdgcn_readlane(blk_lane, tc - t0)
                                     : a.table[(size_t)b * a.tiles_per_seq + tc];
        if (blk < 0 || blk >= a.pool_blocks) blk = 0;
        return blk * a.n_kv_heads + g;
    };
    // codes through per-tile buffer descriptors: per-lane offsets fixed, the
    // block moves the scalar offset
    const int kvo = mrow * KROW + mgrp * (KROW / 4);
    const int vvo = mrow * VROW + mgrp * (VROW / 4);
    auto load_k = [&](int ti) {
        // past the split's last tile the range is empty: the loads return zero
        // without touching memory, and the wait counts stay the same
        const auto r = make_rsrc(a.kc + tile_index(ti) * KCB, ti < t1 ? (uint32_t)KCB : 0u);
#pragma unroll
        for (int mb = 0; mb < TILE / 16; ++mb) {
            const int so = 16 * mb * KROW;
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
        for (int nb = 0; nb < NKB; ++nb) {
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
    // The group's rotated queries (H q / sqrt(D), from the rotation kernel)
    // and then the first tile go out before anything waits.
    // task t: query n = t / QT; lane group gq = (t % QT) / (NKB / 2); pair pr
    float qh[QTMAX][8];
#pragma unroll
    for (int r = 0; r < QTMAX; ++r) {
        const int t = lane + 64 * r;
        const int n = t / QT, rem = t % QT;
        const int gq = rem / (NKB / 2), pr = rem % (NKB / 2);
        const int r0 = run0_of<KB>(gq * (D / 4), 2 * pr), r1 = r0 + Codes<KB>::N / 2;
        const float* src = a.qrot + ((size_t)b * a.n_q_heads + g * G + (n < G ? n : G - 1)) * D;
        const float4 lo = *reinterpret_cast<const float4*>(src + r0);
        const float4 hi = *reinterpret_cast<const float4*>(src + r1);
        const bool live = n < G;
        qh[r][0] = live ? lo.x : 0.0f; qh[r][1] = live ? lo.y : 0.0f;
        qh[r][2] = live ? lo.z : 0.0f; qh[r][3] = live ? lo.w : 0.0f;
        qh[r][4] = live ? hi.x : 0.0f; qh[r][5] = live ? hi.y : 0.0f;
        qh[r][6] = live ? hi.z : 0.0f; qh[r][7] = live ? hi.w : 0.0f;
    }
    load_meta(t0);
    load_k(t0);
    load_v(t0);

    // softmax state of the dense score tasks (task t: query t / 16)
    float m_run[STMAX], l_run[STMAX];
#pragma unroll
    for (int r = 0; r < STMAX; ++r) { m_run[r] = -INFINITY; l_run[r] = 0.0f; }
    // dense accumulator: channel lane + 64 * r, query n
    float acc[CPL_E][GMAX];
#pragma unroll
    for (int r = 0; r < CPL_E; ++r)
#pragma unroll
        for (int n = 0; n < GMAX; ++n) acc[r][n] = 0.0f;

    CodeMagic<KB> kmagic;
    CodeMagic<VB> vmagic;
    kmagic.init();
    vmagic.init();
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the first tile, once

    for (int ti = t0; ti < t1; ++ti) {
        // ---- meta of the tile into the wave's LDS, then the next tile's meta ----
        // (the K and V meta images are adjacent: chunk k lands at byte 16 k)
        static_assert(L::vmeta(0) == 16 * KC, "meta images must be adjacent");
#pragma unroll
        for (int r = 0; r < MCH; ++r) {
            const uint4 v = mt[r];
            if (lane + 64 * r < KC + VC) reinterpret_cast<uint4*>(kmeta)[lane + 64 * r] = v;
        }
        load_meta(ti + 1);
        wave_sync();

        // ---- q' = qh * SK (hi/lo, scaled), zero-point term ----
#pragma unroll
        for (int r = 0; r < QTMAX; ++r) {
            const int t = lane + 64 * r;
            const int n = t / QT, rem = t % QT;
            const int gq = rem / (NKB / 2), pr = rem % (NKB / 2);
            const int r0 = run0_of<KB>(gq * (D / 4), 2 * pr), r1 = r0 + Codes<KB>::N / 2;
            float qv[8];
            float zt = 0.0f, mx = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int ch = (e < 4 ? r0 : r1) + (e & 3);
                const float sk = h2f_bits(kmeta[ch]);
                const float zk = h2f_bits(kmeta[D + ch]);
                qv[e] = qh[r][e] * sk;
                zt = __builtin_fmaf(qh[r][e], __builtin_fmaf(MK, sk, zk), zt);
                mx = fmaxf(mx, fabsf(qv[e]));
            }
            zt = grp_sum<QT>(zt);
            mx = grp_max<QT>(mx);
            const float sq = pow2_scale(mx);
            if (n < G) {
                _Float16 hv[8], lv[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    split_hi_lo(qv[e] * sq, hv[2 * e], lv[2 * e]);
                    split_hi_lo(qv[4 + e] * sq, hv[2 * e + 1], lv[2 * e + 1]);
                }
                const int off = ((gq * G + n) * NKB + 2 * pr) * 8;
                *reinterpret_cast<uint4*>(bqimg + off) = __builtin_bit_cast(uint4, hv);
                *reinterpret_cast<uint4*>(bqimg + 32 * G * NKB + off) = __builtin_bit_cast(uint4, lv);
                if (rem == 0) { st_qz[n] = zt; st_iq[n] = 1.0f / sq; }
            }
        }
        wave_sync();
        // MFMA B operand: q' of head mrow; columns past the group repeat
        // head G - 1 and their scores are never stored
        h4_t bq_hi[NKB], bq_lo[NKB];
        {
            const int row = mrow < G ? mrow : G - 1;
#pragma unroll
            for (int k = 0; k < NKB; ++k) {
                const int off = ((mgrp * G + row) * NKB + k) * 8;
                bq_hi[k] = *reinterpret_cast<const h4_t*>(bqimg + off);
                bq_lo[k] = *reinterpret_cast<const h4_t*>(bqimg + 32 * G * NKB + off);
            }
        }

        // ---- scores: q.K^T on the matrix cores, per 16-token M-block ----
#pragma unroll
        for (int mb = 0; mb < TILE / 16; ++mb) {
            f4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < NKB; k += 2) {
                const h8_t av = cat8(code_operand<KB, KW>(kw[mb], k, kmagic),
                                     code_operand<KB, KW>(kw[mb], k + 1, kmagic));
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, cat8(bq_hi[k], bq_hi[k + 1]), c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, cat8(bq_lo[k], bq_lo[k + 1]), c, 0, 0, 0);
            }
            if (mrow < G)
                *reinterpret_cast<f4_t*>(sc + mrow * TILE + 16 * mb + 4 * mgrp) = c;
        }
        load_k(ti + 1);
        wave_sync();

        // ---- online softmax, dense: task t = (query t/16, lane group, pair) ----
#pragma unroll
        for (int r = 0; r < STMAX; ++r) {
            const int t = lane + 64 * r;
            const int n = t / 16, rem = t % 16;
            const int gv = rem / 4, pr = rem % 4;
            const int r0 = run0_of<VB>(32 * gv, 2 * pr), r1 = r0 + Codes<VB>::N / 2;
            const bool live = n < G;
            const int nn = live ? n : 0;
            const float iq = st_iq[nn], qz = st_qz[nn];
            float s[8], svv[8], zvv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int tok = (e < 4 ? r0 : r1) + (e & 3);
                const float rk = h2f_bits(kmeta[2 * D + tok]);
                svv[e] = h2f_bits(vmeta[tok]);
                zvv[e] = h2f_bits(vmeta[TILE + tok]);
                s[e] = a.sm_scale * rk * __builtin_fmaf(sc[nn * TILE + tok], iq, qz);
            }
            float mt = s[0], smax = 0.0f;
#pragma unroll
            for (int e = 1; e < 8; ++e) mt = fmaxf(mt, s[e]);
#pragma unroll
            for (int e = 0; e < 8; ++e) smax = fmaxf(smax, fabsf(svv[e]));
            mt = grp_max<16>(mt);
            smax = grp_max<16>(smax);
            const float mnew = fmaxf(m_run[r], mt);
            const float al = exp2f((m_run[r] - mnew) * kLog2e);
            const float sp = pow2_scale(smax);
            float p[8], lt = 0.0f, pz = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = exp2f((s[e] - mnew) * kLog2e);
                lt += p[e];
                pz = __builtin_fmaf(p[e], __builtin_fmaf(MV, svv[e], zvv[e]), pz);
            }
            lt = grp_sum<16>(lt);
            pz = grp_sum<16>(pz);
            m_run[r] = mnew;
            l_run[r] = l_run[r] * al + lt;
            if (live) {
                _Float16 hv[8], lv[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    split_hi_lo(p[e] * svv[e] * sp, hv[2 * e], lv[2 * e]);
                    split_hi_lo(p[4 + e] * svv[4 + e] * sp, hv[2 * e + 1], lv[2 * e + 1]);
                }
                const int off = ((gv * G + n) * NVB + 2 * pr) * 8;
                *reinterpret_cast<uint4*>(paimg + off) = __builtin_bit_cast(uint4, hv);
                *reinterpret_cast<uint4*>(paimg + 256 * G + off) = __builtin_bit_cast(uint4, lv);
                if (rem == 0) {
                    st_al[n] = al;
                    st_pz[n] = pz;
                    if (n == 0) st_ip[0] = 1.0f / sp;
                }
            }
        }
        wave_sync();
        // MFMA A operand: p' of head mrow; rows past the group repeat head
        // G - 1 and only rows of real heads are read back
        h4_t pa_hi[NVB], pa_lo[NVB];
        {
            const int row = mrow < G ? mrow : G - 1;
#pragma unroll
            for (int k = 0; k < NVB; ++k) {
                const int off = ((mgrp * G + row) * NVB + k) * 8;
                pa_hi[k] = *reinterpret_cast<const h4_t*>(paimg + off);
                pa_lo[k] = *reinterpret_cast<const h4_t*>(paimg + 256 * G + off);
            }
        }

        // ---- p.V on the matrix cores, per 16-channel N-block ----
#pragma unroll
        for (int nb = 0; nb < NKB; ++nb) {
            f4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < NVB; k += 2) {
                const h8_t bv = cat8(code_operand<VB, VW>(vw[nb], k, vmagic),
                                     code_operand<VB, VW>(vw[nb], k + 1, vmagic));
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(cat8(pa_hi[k], pa_hi[k + 1]), bv, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(cat8(pa_lo[k], pa_lo[k + 1]), bv, c, 0, 0, 0);
            }
            if (4 * mgrp < G)
                *reinterpret_cast<f4_t*>(pvc + (16 * nb + mrow) * GP + 4 * mgrp) = c;
        }
        load_v(ti + 1);
        wave_sync();

        // ---- dense update of the accumulator ----
        {
            const float ip = st_ip[0];
#pragma unroll
            for (int r = 0; r < CPL_E; ++r) {
                const int ch = lane + 64 * r;
                const float cv = h2f_bits(vmeta[2 * TILE + ch]);
#pragma unroll
                for (int n = 0; n < GMAX; ++n) {
                    if (n < G) {
                        const float upd = cv * __builtin_fmaf(pvc[ch * GP + n], ip, st_pz[n]);
                        acc[r][n] = __builtin_fmaf(acc[r][n], st_al[n], upd);
                    }
                }
            }
        }
        wave_sync();
    }

    // ---- partial result of this split: (m, l, acc[D]) per query head ----
#pragma unroll
    for (int r = 0; r < CPL_E; ++r) {
        const int ch = lane + 64 * r;
#pragma unroll
        for (int n = 0; n < GMAX; ++n) {
            if (n < G) {
                const int h = g * G + n;
                float* p = a.ws + (((size_t)b * a.n_q_heads + h) * a.n_parts + split) * (D + 2);
                p[2 + ch] = acc[r][n];
            }
        }
    }
#pragma unroll
    for (int r = 0; r < STMAX; ++r) {
        const int t = lane + 64 * r;
        const int n = t / 16;
        if (n < G && (t % 16) == 0) {
            const int h = g * G + n;
            float* p = a.ws + (((size_t)b * a.n_q_heads + h) * a.n_parts + split) * (D + 2);
            p[0] = m_run[r];
            p[1] = l_run[r];
        }
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
    // global max and the normaliser over the parts (lanes stride the parts)
    float M = -INFINITY;
    for (int s = lane; s < a.n_parts; s += 64) M = fmaxf(M, p[(size_t)s * (D + 2)]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float L = 0.0f;
    for (int s = lane; s < a.n_parts; s += 64) {
        const float ms = p[(size_t)s * (D + 2)];
        if (ms != -INFINITY) L += p[(size_t)s * (D + 2) + 1] * exp2f((ms - M) * kLog2e);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
    // weighted sum of the parts' accumulators, CPL channels per lane
    float v[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] = 0.0f;
    for (int s = 0; s < a.n_parts; ++s) {
        const float* ps = p + (size_t)s * (D + 2);
        const float ms = ps[0];
        if (ms == -INFINITY) continue;
        const float w = exp2f((ms - M) * kLog2e);
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[c] = __builtin_fmaf(ps[2 + CPL * lane + c], w, v[c]);
    }
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
template <int D, int GM>
__global__ __launch_bounds__(256) void attn_tail_kernel(AttnArgs a) {
    constexpr int NT = 256;
    constexpr int HC = D / 2;                      // channels per score thread
    constexpr int CPR = D / 8;                     // 16-byte chunks of a padded row
    constexpr int NS = NT / CPR;                   // token slices of the p . V phase
    constexpr int TPS = TILE / NS;                 // tokens per slice
    constexpr int SPW = 64 / CPR;                  // slices per wave
    __shared__ __align__(16) float qs[GM * D];     // q; then the summed acc
    __shared__ __align__(16) float ps[TILE * GM];  // p[t][n]
    __shared__ float red[2][4][GM];                // per-wave max and sum
    __shared__ float ml[2][GM];                    // final m and l
    float* os = qs;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int bg = blockIdx.x;
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

__global__ void fill_zero_kernel(float* out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = 0.0f;
}

template <int D, int KB, int VB, int GMAX>
static hipError_t launch_att(const AttnArgs& args, hipStream_t s) {
    AttnArgs a = args;
    const int G = a.n_q_heads / a.n_kv_heads;
    if (a.n_splits > 0) {
        // the rotated queries follow the split partials in the workspace
        a.qrot = reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) +
                                          qrot_offset(a.batch, a.n_q_heads, D, a.n_parts));
        hipLaunchKernelGGL((attn_rotate_q_kernel<D>), dim3((unsigned)((a.batch * a.n_q_heads + 3) / 4)),
                           dim3(256), 0, s, a);
        hipError_t e0 = hipGetLastError();
        if (e0 != hipSuccess) return e0;
        const int per_wave = AttnLds<D>::bytes(G);
        int wpb = 65536 / per_wave;
        if (wpb > 4) wpb = 4;
        if (wpb < 1) wpb = 1;
        const int64_t sgroups = (a.n_splits + wpb - 1) / wpb;
        const int64_t blocks = (int64_t)a.batch * a.n_kv_heads * sgroups;
        hipLaunchKernelGGL((attn_partial_kernel<D, KB, VB, GMAX>), dim3((unsigned)blocks),
                           dim3(64 * wpb), (size_t)per_wave * wpb, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.tail_len) {
        hipLaunchKernelGGL((attn_tail_kernel<D, GMAX>), dim3((unsigned)(a.batch * a.n_kv_heads)),
                           dim3(256), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
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
