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
// One workgroup = one tile, 2*D threads, same register layout and transform
// network as the quantiser (kvarn_device.hpp).  The packed codes and meta
// of the tile are copied into LDS with 16-byte loads, each lane then reads
// its 4 tokens x 16 channels, transforms in registers and stores 32 bytes per
// token.  The per-token K factor RK_t and the 1/sqrt(D) scale are applied
// after the transform (they commute with it); for V, 1/sqrt(D) is folded
// into CV_j.
#include "kvarn_device.hpp"
#include "kvarn_internal.hpp"

namespace kvarn {

template <int D, int BITS, bool IS_K>
__device__ __forceinline__ void dequantize_tile(const uint8_t* __restrict__ codes_in,
                                                const uint16_t* __restrict__ meta_in, int d0,
                                                uint16_t* __restrict__ out, uint32_t* lds) {
    constexpr int R = D / CPL;
    constexpr int NT = 2 * D;
    constexpr int CODE_BYTES = TILE * D * BITS / 8;
    constexpr int META_HALVES = IS_K ? 2 * D + TILE : 2 * TILE + D;
    constexpr uint32_t MASK = (1u << BITS) - 1;
    using N = Net<R>;

    const int tid = threadIdx.x;
    const int cb = tid % R;
    const int tb = tid / R;
    const int nb = cb ^ N::kF;   // rotated channel block read by this lane
    const int ob = N::nu(cb);    // output channel block held after the transform
    const float rsqrtD = 1.0f / __builtin_sqrtf((float)D);

    // ---- stage the packed tile in LDS ----
    {
        const uint4* src = reinterpret_cast<const uint4*>(codes_in);
        uint4* dst = reinterpret_cast<uint4*>(lds);
        for (int k = tid; k < CODE_BYTES / 16; k += NT) dst[k] = src[k];
        const uint4* msrc = reinterpret_cast<const uint4*>(meta_in);
        uint4* mdst = reinterpret_cast<uint4*>(lds + CODE_BYTES / 4);
        for (int k = tid; k < META_HALVES / 8; k += NT) mdst[k] = msrc[k];
    }
    __syncthreads();
    const uint8_t* cimg = reinterpret_cast<const uint8_t*>(lds);
    const uint16_t* mimg = reinterpret_cast<const uint16_t*>(lds + CODE_BYTES / 4);

    // ---- unpack my 4 tokens x 16 channels ----
    float code[TPL][CPL];
    if constexpr (IS_K) {
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int t = 4 * tb + i;
            if constexpr (BITS == 4) {
                const uint2 w = *reinterpret_cast<const uint2*>(cimg + (t * D + 16 * nb) / 2);
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    code[i][c] = (float)((w.x >> (4 * c)) & MASK);
                    code[i][8 + c] = (float)((w.y >> (4 * c)) & MASK);
                }
            } else {
                const uint32_t w = *reinterpret_cast<const uint32_t*>(cimg + (t * D + 16 * nb) / 4);
#pragma unroll
                for (int c = 0; c < 16; ++c) code[i][c] = (float)((w >> (2 * c)) & MASK);
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int k = 16 * nb + c;
            uint32_t w;
            if constexpr (BITS == 2) w = cimg[(k * TILE + 4 * tb) / 4];
            else w = *reinterpret_cast<const uint16_t*>(cimg + (k * TILE + 4 * tb) / 2);
#pragma unroll
            for (int i = 0; i < TPL; ++i) code[i][c] = (float)((w >> (BITS * i)) & MASK);
        }
    }

    // ---- folded scales -> rotated-domain values ----
    float x[TPL][CPL];
    float rowscale[TPL];
    if constexpr (IS_K) {
        float sk[CPL], zk[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            sk[c] = h2f_bits(mimg[16 * nb + c]);
            zk[c] = h2f_bits(mimg[D + 16 * nb + c]);
        }
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            rowscale[i] = h2f_bits(mimg[2 * D + 4 * tb + i]) * rsqrtD;
#pragma unroll
            for (int c = 0; c < CPL; ++c) x[i][c] = __builtin_fmaf(code[i][c], sk[c], zk[c]);
        }
    } else {
        float cv[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) cv[c] = h2f_bits(mimg[2 * TILE + 16 * nb + c]) * rsqrtD;
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const float sv = h2f_bits(mimg[4 * tb + i]);
            const float zv = h2f_bits(mimg[TILE + 4 * tb + i]);
            rowscale[i] = 1.0f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) x[i][c] = cv[c] * __builtin_fmaf(code[i][c], sv, zv);
        }
    }

    // ---- inverse rotation (same network) ----
    fwht_inlane(x);
    fwht_crosslane<R>(x, cb);

    // ---- fp16 store of the first d0 channels ----
    if (16 * ob < d0) {
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            uint32_t w[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t lo = f2h_bits(x[i][2 * k] * rowscale[i]);
                const uint32_t hi = f2h_bits(x[i][2 * k + 1] * rowscale[i]);
                w[k] = lo | (hi << 16);
            }
            uint16_t* dst = out + (size_t)(4 * tb + i) * d0 + 16 * ob;
            *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
            if (16 * ob + 16 <= d0) *reinterpret_cast<uint4*>(dst + 8) = make_uint4(w[4], w[5], w[6], w[7]);
        }
    }
}

template <int D, int KB, int VB>
__global__ __launch_bounds__(2 * D) void dequantize_kernel(DequantArgs args) {
    constexpr int KBYTES = TILE * D * KB / 8 + 2 * (2 * D + TILE);
    constexpr int VBYTES = TILE * D * VB / 8 + 2 * (2 * TILE + D);
    constexpr int WORDS = (KBYTES > VBYTES ? KBYTES : VBYTES) / 4;
    __shared__ uint32_t lds[WORDS];
    const int64_t tile = blockIdx.x;
    if (tile < args.n_k) {
        dequantize_tile<D, KB, true>(args.kc + tile * (TILE * D * KB / 8),
                                     args.km + tile * (2 * D + TILE), args.d0,
                                     args.ko + tile * TILE * args.d0, lds);
    } else {
        const int64_t vt = tile - args.n_k;
        dequantize_tile<D, VB, false>(args.vc + vt * (TILE * D * VB / 8),
                                      args.vm + vt * (2 * TILE + D), args.d0,
                                      args.vo + vt * TILE * args.d0, lds);
    }
}

template <int D, int KB, int VB>
static hipError_t launch_dq(const DequantArgs& a, hipStream_t s) {
    const int64_t blocks = a.n_k + a.n_v;
    hipLaunchKernelGGL((dequantize_kernel<D, KB, VB>), dim3((unsigned)blocks), dim3(2 * D), 0, s, a);
    return hipGetLastError();
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
