// kvarn_dequantize.hip -- unpack + folded scales + inverse rotation, gfx950.
//
// Method (hotdry page "KVarN Hadamard 旋转与方差归一化", section
// "非对称量化与尺度折叠": the scales are multiplied back on read; digest page,
// "方法" module 3: dequantise restores the original scale): per tile, the
// rotated-domain value is
//     K: RK_t * (code * SK_j + ZK_j)      V: CV_j * (code * SV_t + ZV_t)
// and the orthonormal Hadamard matrix, symmetric and its own inverse, maps it
// back to the original channels; the first head_dim channels are rounded to
// fp16 (nearest even).
//
// 2*D threads per workgroup, same register layout and transform network as
// the quantiser (kvarn_device.hpp).  One workgroup per tile, K tiles then V
// tiles, launched in address order: the device writes fastest when the
// workgroups in flight write one narrow, advancing window of addresses, and
// the resident workgroups (three per CU) overlap one another's HBM
// latency with their arithmetic and stores.  K codes are
// token-major, so a lane's 16 channels of one token are one 8- (4-bit) or
// 4-byte (2-bit) word, read by that lane alone.  V codes are channel-major:
// a wavefront's tokens are a few bytes of every channel row, so the
// workgroup reads the tile's whole code block once, each wavefront 1 KB of
// consecutive bytes per load, and passes it through LDS; lanes holding
// neighbouring token groups then take whole words of their channel rows and
// swap bytes inside the wavefront.  (Read by each wavefront straight from
// memory, the partly used 128-byte lines of the V rows were fetched from HBM
// again when the cache dropped them between the wavefronts' reads.)  Code and
// meta loads carry the nontemporal hint, as the output stores do.  The
// per-token K factor RK_t and the 1/sqrt(D) scale are applied
// after the transform (they commute with it); for V, 1/sqrt(D) is folded
// into CV_j.
#include "kvarn_device.hpp"
#include "kvarn_internal.hpp"

namespace kvarn {

// Per-wavefront LDS region (2048 words): [0, 512) the V byte swap,
// [1536, 1536 + 4 * NC) the tile's meta as the wave needs it, and all of it
// for the output staging once both have been read.
constexpr int kWaveWords = 2048;
constexpr int kMetaWord = 1536;

// Meta of one tile for one wavefront of TW = 4096 / D tokens, gathered by
// the wave's lanes as 16-byte chunks (one global load per lane instead of
// every lane fetching its own copies):
//   K: SK (D halves) | ZK (D halves) | RK of the wave's tokens (TW halves)
//   V: SV of the wave's tokens | ZV of the wave's tokens | CV (D halves)
template <int D, bool IS_K>
struct MetaPlan {
    static constexpr int TW = 4096 / D;
    static constexpr int NC = IS_K ? D / 4 + TW / 8 : TW / 4 + D / 8;   // chunks
    static constexpr int NS = (NC + 63) / 64;                            // per lane
    // source offset (halves, within the tile's meta) of chunk e; tok0 =
    // first token of the wave
    __device__ static int src(int e, int tok0) {
        if (IS_K) return e < D / 4 ? 8 * e : 2 * D + tok0 + 8 * (e - D / 4);
        if (e < TW / 8) return tok0 + 8 * e;
        if (e < TW / 4) return TILE + tok0 + 8 * (e - TW / 8);
        return 2 * TILE + 8 * (e - TW / 4);
    }
};

// packed inputs of one tile held by one lane
template <int D, int BITS, bool IS_K> struct Packed;
template <int D, int BITS> struct Packed<D, BITS, true> {
    uint32_t c[TPL][BITS / 2];           // token 4*tb + i: 16 channels of block nb
    uint4 m[MetaPlan<D, true>::NS];      // meta chunks
};
template <int D, int BITS> struct Packed<D, BITS, false> {
    uint4 v[BITS / 2];                   // this thread's 16-byte pieces of the tile's code block
    uint4 m[MetaPlan<D, false>::NS];
};

// Word (channel row r, word w) of a V tile's code block in the workgroup's
// LDS copy.  Rows are 4 * VB words long; with L = log2(D):
//   2-bit: 16-byte word G holds word w of rows 4 (r >> 2) .. 4 (r >> 2) + 3,
//          G = (r >> 2 | w << (L - 2)) ^ (r >> 6) << (8 - L) ^ (w >> 2 & 1) << 2;
//   4-bit: 16-byte word G + 2 D ((r >> 3) & 1) holds word w of the four rows
//          that differ in bits 1 and 2 of r,
//          G = (r & 1 | (r >> 4) << 1 | w << (L - 3)) ^ (w >> 2 & 3) << 1 ^ (r >> 7).
// A lane's rows 16 nb + 4 j + n (2-bit) or 16 nb + 2 q + j (4-bit) of its
// word m are then one or two aligned 16-byte words, the 16-byte reads of a
// quarter wave and the 4-byte stores of a half wave (the stored pieces are
// 16 consecutive bytes of one row each) fall on distinct banks at every
// head_dim, and word w + i of a row sits i * VQ words after word w
// (w % 4 == 0, i < 4).
template <int D, int BITS>
struct VBlock {
    static constexpr int L = D == 64 ? 6 : D == 128 ? 7 : 8;
    static constexpr int WORDS = 4 * BITS * D;         // words of one tile's code block
    static constexpr int VQ = BITS == 2 ? D : D / 2;   // word step of w -> w + 1 (w % 4 < 3)
    __device__ static int addr(int r, int w) {
        if constexpr (BITS == 2) {
            const int G = ((r >> 2) | (w << (L - 2))) ^ ((r >> 6) << (8 - L)) ^ (((w >> 2) & 1) << 2);
            return 4 * G + (r & 3);
        } else {
            const int G = ((r & 1) | ((r >> 4) << 1) | (w << (L - 3))) ^ (((w >> 2) & 3) << 1) ^ (r >> 7);
            return 4 * (G + 2 * D * ((r >> 3) & 1)) + ((r >> 1) & 3);
        }
    }
};

// Global loads with the nontemporal hint: every code and meta byte is read
// once per call.  Inside the prefill step (the cache read after the
// quantiser's 5 GB) they took the kernel from 0.927 to 0.905 ms; the packed
// attention's meta loads, given the same hint, were slower.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_nt8(const void* p) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t ld_nt4(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

__device__ __forceinline__ float half_of(const uint32_t* pairs, int k) {
    return h2f_bits((uint16_t)((k & 1) ? (pairs[k >> 1] >> 16) : (pairs[k >> 1] & 0xFFFF)));
}
__device__ __forceinline__ void lds16(uint32_t* dst, const uint32_t* src) {
    const uint4 a = *reinterpret_cast<const uint4*>(src);
    const uint4 b = *reinterpret_cast<const uint4*>(src + 4);
    dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
    dst[4] = b.x; dst[5] = b.y; dst[6] = b.z; dst[7] = b.w;
}

template <int D, int BITS, bool IS_K>
__device__ __forceinline__ void load_tile(Packed<D, BITS, IS_K>& p, const uint8_t* __restrict__ codes,
                                          const uint16_t* __restrict__ meta, int tb, int nb) {
    using MP = MetaPlan<D, IS_K>;
    const int ln = threadIdx.x & 63;
    const int tok0 = (threadIdx.x >> 6) * MP::TW;
#pragma unroll
    for (int k = 0; k < MP::NS; ++k) {
        int e = ln + 64 * k;
        if (e >= MP::NC) e = 0;   // spare lanes re-read chunk 0 (keeps the load unconditional)
        p.m[k] = ld_nt16(meta + MP::src(e, tok0));
    }
    if constexpr (IS_K) {
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const uint8_t* src = codes + ((4 * tb + i) * D + 16 * nb) * BITS / 8;
            if constexpr (BITS == 4) {
                const uint2 w = ld_nt8(src);
                p.c[i][0] = w.x;
                p.c[i][1] = w.y;
            } else {
                p.c[i][0] = ld_nt4(src);
            }
        }
    } else {
        // the tile's code block, 16 bytes per thread and load: each wave reads
        // 1 KB of consecutive bytes
#pragma unroll
        for (int k = 0; k < BITS / 2; ++k)
            p.v[k] = ld_nt16(reinterpret_cast<const uint4*>(codes) + threadIdx.x + 2 * D * k);
    }
}

template <int D, int BITS, bool IS_K, bool FULL>
__device__ __forceinline__ void dequantize_tile(const Packed<D, BITS, IS_K>& p, int d0,
                                                uint16_t* __restrict__ out, uint32_t* xch,
                                                uint32_t* vb) {
    constexpr int R = D / CPL;
    constexpr uint32_t MASK = (1u << BITS) - 1;
    using N = Net<R>;
    using MP = MetaPlan<D, IS_K>;
    const int tid = threadIdx.x;
    const int cb = tid % R;
    const int tb = tid / R;
    const int ln = tid & 63;
    const int tbl = ln / R;                 // token group within the wave
    const int nb = cb ^ N::kF;             // rotated channel block read by this lane
    const int ob = N::nu(cb);              // output channel block held after the transform
    const float rsqrtD = 1.0f / __builtin_sqrtf((float)D);
    uint32_t* mw = xch + kMetaWord;        // the wave's meta words (2 halves each)

#pragma unroll
    for (int k = 0; k < MP::NS; ++k)
        if (ln + 64 * k < MP::NC) *reinterpret_cast<uint4*>(mw + 4 * (ln + 64 * k)) = p.m[k];

    float x[TPL][CPL];
    float rowscale[TPL];
    if constexpr (IS_K) {
        wave_sync();
        uint32_t sk[8], zk[8], rk[2];
        lds16(sk, mw + 8 * nb);
        lds16(zk, mw + D / 2 + 8 * nb);
        const uint2 r2 = *reinterpret_cast<const uint2*>(mw + D + 2 * tbl);
        rk[0] = r2.x;
        rk[1] = r2.y;
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            rowscale[i] = half_of(rk, i) * rsqrtD;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const uint32_t w = (BITS == 4) ? p.c[i][c >> 3] : p.c[i][0];
                const int sh = (BITS == 4) ? 4 * (c & 7) : 2 * c;
                const float code = (float)((w >> sh) & MASK);
                x[i][c] = __builtin_fmaf(code, half_of(sk, c), half_of(zk, c));
            }
        }
    } else {
        // The code block through LDS: every thread stores its 16-byte pieces
        // (channel row r, words w0 .. w0 + 3), then lane (tb, nb) reads word
        // m of the rows it swaps below, g[n] = row 16 nb + 4 j + n (2-bit,
        // m = tb / 4, j = tb % 4) or g[q] = row 16 nb + 2 q + j (4-bit,
        // m = tb / 2, j = tb % 2).  The workgroup dequantises one tile, so
        // the block is stored once and one barrier orders the reads after it.
        using VBk = VBlock<D, BITS>;
        uint32_t g[BITS == 2 ? 4 : 8];
#pragma unroll
        for (int k = 0; k < BITS / 2; ++k) {
            const int P = tid + 2 * D * k;   // 16-byte piece of the block
            const int a0 = BITS == 2 ? VBk::addr(P >> 1, 4 * (P & 1)) : VBk::addr(P >> 2, 4 * (P & 3));
            vb[a0] = p.v[k].x;
            vb[a0 + VBk::VQ] = p.v[k].y;
            vb[a0 + 2 * VBk::VQ] = p.v[k].z;
            vb[a0 + 3 * VBk::VQ] = p.v[k].w;
        }
        __syncthreads();
        if constexpr (BITS == 2) {
            const uint4 a = *reinterpret_cast<const uint4*>(vb + VBk::addr(16 * nb + 4 * (tb & 3), tb >> 2));
            g[0] = a.x; g[1] = a.y; g[2] = a.z; g[3] = a.w;
        } else {
            const uint4 a = *reinterpret_cast<const uint4*>(vb + VBk::addr(16 * nb + (tb & 1), tb >> 1));
            const uint4 b = *reinterpret_cast<const uint4*>(vb + VBk::addr(16 * nb + 8 + (tb & 1), tb >> 1));
            g[0] = a.x; g[1] = a.y; g[2] = a.z; g[3] = a.w;
            g[4] = b.x; g[5] = b.y; g[6] = b.z; g[7] = b.w;
        }

        // in-wave swap: lane (token group tb) gets word q = channels of its block
        // (2-bit: 4 channels 4q..4q+3, a byte each; 4-bit: channels 2q, 2q+1, two bytes each)
        constexpr int NW = BITS == 2 ? 4 : 8;
        uint32_t w[NW];
        if constexpr (BITS == 2) {
            const uint32_t A = __builtin_amdgcn_perm(g[1], g[0], 0x05010400u);
            const uint32_t B = __builtin_amdgcn_perm(g[1], g[0], 0x07030602u);
            const uint32_t C = __builtin_amdgcn_perm(g[3], g[2], 0x05010400u);
            const uint32_t E = __builtin_amdgcn_perm(g[3], g[2], 0x07030602u);
            *reinterpret_cast<uint4*>(xch + 4 * ln) =
                make_uint4(__builtin_amdgcn_perm(C, A, 0x05040100u), __builtin_amdgcn_perm(C, A, 0x07060302u),
                           __builtin_amdgcn_perm(E, B, 0x05040100u), __builtin_amdgcn_perm(E, B, 0x07060302u));
            wave_sync();
            const int j = tb & 3;
            const int base = ln - j * R;
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] = xch[4 * (base + q * R) + j];
        } else {
            *reinterpret_cast<uint4*>(xch + 8 * ln) = make_uint4(g[0], g[1], g[2], g[3]);
            *reinterpret_cast<uint4*>(xch + 8 * ln + 4) = make_uint4(g[4], g[5], g[6], g[7]);
            wave_sync();
            const int j = tb & 1;
            const int base = ln - j * R;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t r0 = xch[8 * base + q], r1 = xch[8 * (base + R) + q];
                w[q] = j ? __builtin_amdgcn_perm(r1, r0, 0x07060302u) : __builtin_amdgcn_perm(r1, r0, 0x05040100u);
            }
        }
        uint32_t sv[2], zv[2], cvw[8];
        {
            const uint2 s2 = *reinterpret_cast<const uint2*>(mw + 2 * tbl);
            const uint2 z2 = *reinterpret_cast<const uint2*>(mw + MP::TW / 2 + 2 * tbl);
            sv[0] = s2.x; sv[1] = s2.y;
            zv[0] = z2.x; zv[1] = z2.y;
            lds16(cvw, mw + MP::TW + 8 * nb);
        }
        float cv[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) cv[c] = half_of(cvw, c) * rsqrtD;
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const float svi = half_of(sv, i), zvi = half_of(zv, i);
            rowscale[i] = 1.0f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const uint32_t word = (BITS == 2) ? w[c >> 2] : w[c >> 1];
                const int sh = (BITS == 2) ? 8 * (c & 3) + 2 * i : 16 * (c & 1) + 4 * i;
                const float code = (float)((word >> sh) & MASK);
                x[i][c] = cv[c] * __builtin_fmaf(code, svi, zvi);
            }
        }
    }

    // ---- inverse rotation (same network) ----
    fwht_inlane(x);
    fwht_crosslane<R>(x, cb);

    // ---- fp16 store ----
    // The wave's 256/R tokens are one contiguous run of the output (d0
    // channels per row, 8 KB when d0 == D).  Stage it in the wave's LDS
    // region as 16-byte chunks and store it with fully contiguous 1 KB wave
    // stores.  16-byte LDS stores are served eight lanes at a time over 32
    // banks, and the eight lanes of a token group hold chunks 2 ob + h, which
    // fill only four of the eight 16-byte bank groups.  So with 16 or 32
    // chunks per row the chunk index is flipped in its lowest bit by bits 3
    // and 4 of the chunk, and in bit 3 by token-group parity: eight lanes then
    // hit eight distinct bank groups, and the quarter-wave 16-byte reads of 16
    // consecutive chunks stay conflict-free.  With another even count (head_dim
    // 64, or a padded width) bit 0 is flipped by token-group parity.  Padded
    // widths stage only their first d0 channels.
    {
        const int CPR = FULL ? D / 8 : d0 / 8;   // 16-byte chunks per output row
        const bool swz = FULL || (CPR & 1) == 0;
        auto slot = [&](int r, int ch) {
            if (!swz) return r * CPR + ch;
            if (CPR % 16 == 0)
                return r * CPR + (ch ^ (((ch >> 3) ^ (ch >> 4)) & 1) ^ (((r >> 2) & 1) << 3));
            return r * CPR + (ch ^ ((r >> 2) & 1));
        };
        const int ln = tid & 63;
        wave_sync();
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int r = 4 * (ln / R) + i;   // row within the wave's run
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int ch = 2 * ob + h;
                if (!FULL && ch >= CPR) continue;
                uint32_t o[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t lo = f2h_bits(x[i][8 * h + 2 * k] * rowscale[i]);
                    const uint32_t hi = f2h_bits(x[i][8 * h + 2 * k + 1] * rowscale[i]);
                    o[k] = lo | (hi << 16);
                }
                *reinterpret_cast<uint4*>(xch + 4 * slot(r, ch)) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
        wave_sync();
        const int run = (256 / R) * CPR;        // chunks in the wave's run
        uint4* dst = reinterpret_cast<uint4*>(out + (size_t)(tid >> 6) * (256 / R) * d0);
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
            const int g = ln + 64 * s2;
            if (!FULL && g >= run) break;
            const int r = g / CPR, ch = g % CPR;
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(xch + 4 * slot(r, ch)),
                                        reinterpret_cast<u32x4*>(dst + g));
        }
    }
}

// Workgroup b dequantises tile b0 + b of the concatenation [K tiles | V
// tiles].  The grid covers every tile (in launches of at most kMaxGrid
// workgroups), so the workgroups in flight write one narrow window of the
// outputs that advances in address order, the pattern the device writes
// fastest; the resident workgroups overlap one another's loads and stores.

template <int D, int KB, int VB, bool FULL>
__global__ __launch_bounds__(2 * D) void dequantize_kernel(DequantArgs a, int64_t b0) {
    __shared__ __align__(16) uint32_t xch[(2 * D / 64) * kWaveWords];
    __shared__ __align__(16) uint32_t vblk[VBlock<D, VB>::WORDS];   // the V tile's code block
    constexpr int R = D / CPL;
    const int tid = threadIdx.x;
    const int tb = tid / R;
    const int nb = (tid % R) ^ Net<R>::kF;   // rotated channel block read by this lane
    uint32_t* xw = xch + (tid >> 6) * kWaveWords;
    const int64_t b = b0 + blockIdx.x;
    if (b < a.n_k) {
        Packed<D, KB, true> p;
        load_tile<D, KB, true>(p, a.kc + b * (TILE * D * KB / 8), a.km + b * (2 * D + TILE), tb, nb);
        dequantize_tile<D, KB, true, FULL>(p, a.d0, a.ko + b * TILE * a.d0, xw, vblk);
    } else if (b < a.n_k + a.n_v) {
        const int64_t t = b - a.n_k;
        Packed<D, VB, false> p;
        load_tile<D, VB, false>(p, a.vc + t * (TILE * D * VB / 8), a.vm + t * (2 * TILE + D), tb, nb);
        dequantize_tile<D, VB, false, FULL>(p, a.d0, a.vo + t * TILE * a.d0, xw, vblk);
    }
}

template <int D, int KB, int VB>
static hipError_t launch_dq(const DequantArgs& a, hipStream_t s) {
    auto kern = (a.d0 == D) ? dequantize_kernel<D, KB, VB, true> : dequantize_kernel<D, KB, VB, false>;
    const int64_t total = a.n_k + a.n_v;
    for (int64_t b0 = 0; b0 < total; b0 += kMaxGrid) {
        const int64_t n = total - b0 < kMaxGrid ? total - b0 : kMaxGrid;
        hipLaunchKernelGGL(kern, dim3((unsigned)n), dim3(2 * D), 0, s, a, b0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int D>
static hipError_t launch_dq_bits(const DequantArgs& a, int kb, int vb, hipStream_t s) {
    if (kb == 4 && vb == 2) return launch_dq<D, 4, 2>(a, s);
    if (kb == 4 && vb == 4) return launch_dq<D, 4, 4>(a, s);
    if (kb == 2 && vb == 2) return launch_dq<D, 2, 2>(a, s);
    return launch_dq<D, 2, 4>(a, s);
}

hipError_t launch_dequantize(const DequantArgs& a, int D, int kb, int vb, hipStream_t s) {
    if (D == 64) return launch_dq_bits<64>(a, kb, vb, s);
    if (D == 128) return launch_dq_bits<128>(a, kb, vb, s);
    return launch_dq_bits<256>(a, kb, vb, s);
}

}  // namespace kvarn
