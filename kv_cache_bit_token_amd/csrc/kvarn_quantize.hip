// kvarn_quantize.hip -- fused rotate + normalise + RTN + pack + fold, gfx950.
//
// Method (hotdry page "KVarN Hadamard 旋转与方差归一化", sections
// "Hadamard 旋转", "迭代方差归一化" and "非对称量化与尺度折叠"; deep-dive page
// "KV cache 為什麼能壓到 4-bit／2-bit ...", worked 2-bit example and the
// KEY/VALUE table): per 128-token tile, rotate every token along head_dim by
// the orthonormal Hadamard matrix, alternate column / row standard-deviation
// normalisation n_iters times with log-space factors, then asymmetric RTN
// per channel (K) or per token (V), fold the group-axis factor into the
// group's scale and zero point, pack the codes.
//
// One workgroup = one tile (K or V), 2*D threads, the tile held in VGPRs as
// fp32 (see kvarn_device.hpp for the lane layout and the transform).  The
// input is read from HBM exactly once; codes and meta are staged in LDS and
// written out with 16-byte stores.
//
// Arithmetic, equal to the stated method in exact arithmetic:
//  * The transform runs unscaled: X' = sqrt(D) * Xt.  The normalised tile is
//    invariant to a global scale, so only the stored column factor and the K
//    scale/zero absorb the sqrt(D), divided out once per group.
//  * Log-space accumulation l_c += ln(sigma_c(current values)) gives
//    exp(l_c) = std over tokens of X'[t][c] * exp(-l_r[t]); the kernel keeps
//    these products directly (C[c] = exp(l_c), R[t] = exp(l_r)) and
//    recomputes each std from X' and the current cross-axis factors, the
//    same quantity without an exp/log round trip.
//  * A K group (one channel) is scaled by its own column factor, which
//    cancels in its codes and folds back in SK, ZK: the kernel quantises
//    X' * (1/R[t]) directly.  Likewise V quantises X' * (1/C[c]) and the row
//    factor cancels, so V skips the last row pass (its result is not used).
//  * Standard deviations are two-pass (mean first, then centred sum of
//    squares), population (divide by the group size).
#include "kvarn_device.hpp"
#include "kvarn_internal.hpp"

namespace kvarn {

template <int D, int BITS, bool IS_K>
__device__ __forceinline__ void quantize_tile(const uint16_t* __restrict__ xin, int d0, int n_iters,
                                              uint8_t* __restrict__ codes_out,
                                              uint16_t* __restrict__ meta_out, float* lds) {
    constexpr int R = D / CPL;          // lanes per row-group
    constexpr int NT = 2 * D;           // threads
    constexpr int L = (1 << BITS) - 1;  // top code
    constexpr int CODE_BYTES = TILE * D * BITS / 8;
    constexpr int META_HALVES = IS_K ? 2 * D + TILE : 2 * TILE + D;
    using N = Net<R>;

    const int tid = threadIdx.x;
    const int cb = tid % R;
    const int tb = tid / R;
    const int nb = cb ^ N::kF;      // natural channel block loaded by this lane
    const int ob = N::nu(cb);       // Sylvester channel block held after the transform
    const float sqrtD = __builtin_sqrtf((float)D);
    const float rsqrtD = 1.0f / sqrtD;

    float* part = lds;                    // [32][D] column partials
    float* colv = lds + 32 * D;           // [D] broadcast of column stats
    float* colv2 = colv + D;              // [D]

    // ---------------- load (one HBM read) + pad ----------------
    float x[TPL][CPL];
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
        const uint16_t* row = xin + (size_t)(4 * tb + i) * d0;
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
            const int ch0 = 16 * nb + 8 * hlf;
            if (ch0 + 8 <= d0) {
                uint4 w = *reinterpret_cast<const uint4*>(row + ch0);
                uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    x[i][8 * hlf + 2 * k] = h2f_bits((uint16_t)(ws[k] & 0xFFFF));
                    x[i][8 * hlf + 2 * k + 1] = h2f_bits((uint16_t)(ws[k] >> 16));
                }
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) x[i][8 * hlf + k] = 0.0f;
            }
        }
    }

    // ---------------- rotation (unscaled) ----------------
    fwht_inlane(x);
    fwht_crosslane<R>(x, cb);

    // ---------------- normalisation ----------------
    float a[TPL];      // 1 / R[t] for my tokens
    float Rt[TPL];     // R[t] = exp(l_r[t])
#pragma unroll
    for (int i = 0; i < TPL; ++i) { a[i] = 1.0f; Rt[i] = 1.0f; }
    float b[CPL];      // 1 / C[c] for my channels (unscaled units)
#pragma unroll
    for (int c = 0; c < CPL; ++c) b[c] = rsqrtD;

    // reducer role: position p = tid >> 1 (lane-position space), half hh
    const int rp = tid >> 1, rh = tid & 1;
    float Cp = sqrtD;   // column factor of position rp, unscaled units (exp(l_c) * sqrt(D))

    for (int it = 0; it < n_iters; ++it) {
        // ---- column pass: mean over tokens of x * a ----
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < TPL; ++i) s = __builtin_fmaf(x[i][c], a[i], s);
            part[tb * D + 16 * cb + c] = s;
        }
        __syncthreads();
        float cmean;
        {
            float s = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k) s += part[(rh * 16 + k) * D + rp];
            s += dpp<DPP_XOR1>(s);
            cmean = s * (1.0f / TILE);
            if (rh == 0) colv[rp] = cmean;
        }
        __syncthreads();
        float m[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) m[c] = colv[16 * cb + c];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float q = 0.0f;
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                float d = __builtin_fmaf(x[i][c], a[i], -m[c]);
                q = __builtin_fmaf(d, d, q);
            }
            part[tb * D + 16 * cb + c] = q;
        }
        __syncthreads();
        {
            float q = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k) q += part[(rh * 16 + k) * D + rp];
            q += dpp<DPP_XOR1>(q);
            const float sd = __builtin_sqrtf(q * (1.0f / TILE));
            if (!is_flat(sd, cmean)) Cp = sd;
            if (rh == 0) colv[rp] = 1.0f / Cp;
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < CPL; ++c) b[c] = colv[16 * cb + c];

        // ---- row pass (V does not use the last one) ----
        if (!IS_K && it == n_iters - 1) break;
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            float s = 0.0f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) s = __builtin_fmaf(x[i][c], b[c], s);
            const float rmean = rg_sum<R>(s) * (1.0f / D);
            float q = 0.0f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                float d = __builtin_fmaf(x[i][c], b[c], -rmean);
                q = __builtin_fmaf(d, d, q);
            }
            const float sd = __builtin_sqrtf(rg_sum<R>(q) * (1.0f / D));
            if (!is_flat(sd, rmean)) Rt[i] = sd;
            a[i] = 1.0f / Rt[i];
        }
    }

    // ---------------- gauge of the stored factors ----------------
    // The normalised tile depends on l_r[t] + l_c[c] only.  The mean column
    // log-factor is moved into the row factors (G = geometric mean of the
    // column factors) so the stored fp16 factors stay in range even when the
    // iteration drifts the two sets apart.  Codes are unaffected; only the
    // stored SK/ZK/RK (K) and SV/ZV/CV (V) see G.
    float* gsum = lds + 66 * D;
    float G, invG;
    {
        float s = logf(Cp * rsqrtD);   // both lanes of a position: the sum is 2x
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
        if ((tid & 63) == 0) gsum[tid >> 6] = s;
        __syncthreads();
        float tot = 0.0f;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) tot += gsum[w];
        const float mean_lc = tot * (0.5f / D);
        G = expf(mean_lc);
        invG = expf(-mean_lc);
    }

    // ---------------- quantisation parameters ----------------
    uint8_t* cimg = reinterpret_cast<uint8_t*>(lds);                  // packed code image
    uint16_t* mimg = reinterpret_cast<uint16_t*>(lds + CODE_BYTES / 4);  // meta image
    uint32_t code[TPL][CPL];

    if constexpr (IS_K) {
        // K: one group per channel, over the 128 tokens: values v = x * a[t]
        float v[TPL][CPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i)
#pragma unroll
            for (int c = 0; c < CPL; ++c) v[i][c] = x[i][c] * a[i];
        __syncthreads();   // LDS part[] reuse
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float mn = v[0][c], mx = v[0][c];
#pragma unroll
            for (int i = 1; i < TPL; ++i) { mn = fminf(mn, v[i][c]); mx = fmaxf(mx, v[i][c]); }
            part[tb * D + 16 * cb + c] = mn;
            part[32 * D + 2 * D + tb * D + 16 * cb + c] = mx;   // second buffer after colv/colv2
        }
        __syncthreads();
        float zk, sk;
        {
            float mn = part[(rh * 16) * D + rp], mx = part[32 * D + 2 * D + (rh * 16) * D + rp];
#pragma unroll
            for (int k = 1; k < 16; ++k) {
                mn = fminf(mn, part[(rh * 16 + k) * D + rp]);
                mx = fmaxf(mx, part[32 * D + 2 * D + (rh * 16 + k) * D + rp]);
            }
            mn = fminf(mn, dpp<DPP_XOR1>(mn));
            mx = fmaxf(mx, dpp<DPP_XOR1>(mx));
            zk = mn;
            sk = (mx - mn) / (float)L;
            const float inv = (mx > mn) ? 1.0f / sk : 0.0f;
            if (rh == 0) { colv[rp] = inv; colv2[rp] = -zk * inv; }
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float inv = colv[16 * cb + c], off = colv2[16 * cb + c];
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                float u = __builtin_fmaf(v[i][c], inv, off);
                float r = __builtin_rintf(u);
                r = fminf(fmaxf(r, 0.0f), (float)L);
                code[i][c] = (uint32_t)r;
            }
        }
        __syncthreads();   // image overwrites part[]
        // meta: SK, ZK by the reducers (rotated channel index), RK by lane cb == 0
        if (rh == 0) {
            const int k = 16 * N::nu(rp >> 4) + (rp & 15);
            mimg[k] = f2h_bits(sk * rsqrtD * invG);
            mimg[D + k] = f2h_bits(zk * rsqrtD * invG);
        }
        if (cb == 0) {
#pragma unroll
            for (int i = 0; i < TPL; ++i) mimg[2 * D + 4 * tb + i] = f2h_bits(Rt[i] * G);
        }
    } else {
        // V: one group per token, over the D channels: values v = x * b[c]
        float v[TPL][CPL];
        float inv[TPL], off[TPL], zv[TPL], sv[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            float mn = 3.0e38f, mx = -3.0e38f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                v[i][c] = x[i][c] * b[c];
                mn = fminf(mn, v[i][c]);
                mx = fmaxf(mx, v[i][c]);
            }
            mn = rg_min<R>(mn);
            mx = rg_max<R>(mx);
            zv[i] = mn;
            sv[i] = (mx - mn) / (float)L;
            inv[i] = (mx > mn) ? 1.0f / sv[i] : 0.0f;
            off[i] = -mn * inv[i];
        }
#pragma unroll
        for (int i = 0; i < TPL; ++i)
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                float u = __builtin_fmaf(v[i][c], inv[i], off[i]);
                float r = __builtin_rintf(u);
                r = fminf(fmaxf(r, 0.0f), (float)L);
                code[i][c] = (uint32_t)r;
            }
        __syncthreads();   // image overwrites part[]
        if (cb == 0) {
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                mimg[4 * tb + i] = f2h_bits(sv[i] * G);
                mimg[TILE + 4 * tb + i] = f2h_bits(zv[i] * G);
            }
        }
        if (rh == 0) {
            const int k = 16 * N::nu(rp >> 4) + (rp & 15);
            mimg[2 * TILE + k] = f2h_bits(Cp * rsqrtD * invG);
        }
    }

    // ---------------- pack into the LDS image ----------------
    if constexpr (IS_K) {
        // token-major: token t, channels 16*ob .. +15 are contiguous
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int t = 4 * tb + i;
            if constexpr (BITS == 4) {
                uint32_t w0 = 0, w1 = 0;
#pragma unroll
                for (int c = 0; c < 8; ++c) { w0 |= code[i][c] << (4 * c); w1 |= code[i][8 + c] << (4 * c); }
                *reinterpret_cast<uint2*>(cimg + (t * D + 16 * ob) / 2) = make_uint2(w0, w1);
            } else {
                uint32_t w = 0;
#pragma unroll
                for (int c = 0; c < 16; ++c) w |= code[i][c] << (2 * c);
                *reinterpret_cast<uint32_t*>(cimg + (t * D + 16 * ob) / 4) = w;
            }
        }
    } else {
        // channel-major: channel k, tokens 4*tb .. +3 are contiguous
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int k = 16 * ob + c;
            if constexpr (BITS == 2) {
                uint32_t w = 0;
#pragma unroll
                for (int i = 0; i < TPL; ++i) w |= code[i][c] << (2 * i);
                cimg[(k * TILE + 4 * tb) / 4] = (uint8_t)w;
            } else {
                uint32_t w = 0;
#pragma unroll
                for (int i = 0; i < TPL; ++i) w |= code[i][c] << (4 * i);
                *reinterpret_cast<uint16_t*>(cimg + (k * TILE + 4 * tb) / 2) = (uint16_t)w;
            }
        }
    }
    __syncthreads();

    // ---------------- coalesced copy-out ----------------
    {
        const uint4* src = reinterpret_cast<const uint4*>(cimg);
        uint4* dst = reinterpret_cast<uint4*>(codes_out);
        for (int k = tid; k < CODE_BYTES / 16; k += NT) dst[k] = src[k];
        const uint4* msrc = reinterpret_cast<const uint4*>(mimg);
        uint4* mdst = reinterpret_cast<uint4*>(meta_out);
        for (int k = tid; k < META_HALVES / 8; k += NT) mdst[k] = msrc[k];
    }
}

// LDS floats needed: part [32][D] + colv/colv2 [2][D] + the K max buffer
// [32][D] + 16 gauge partials; the code and meta images reuse the front.
template <int D>
constexpr int quant_lds_floats() { return 32 * D + 2 * D + 32 * D + 16; }

template <int D, int KB, int VB>
__global__ __launch_bounds__(2 * D) void quantize_kernel(QuantArgs args) {
    __shared__ float lds[quant_lds_floats<D>()];
    const int64_t tile = blockIdx.x;
    if (tile < args.n_k) {
        quantize_tile<D, KB, true>(args.k + tile * TILE * args.d0, args.d0, args.n_iters,
                                   args.kc + tile * (TILE * D * KB / 8),
                                   args.km + tile * (2 * D + TILE), lds);
    } else {
        const int64_t vt = tile - args.n_k;
        quantize_tile<D, VB, false>(args.v + vt * TILE * args.d0, args.d0, args.n_iters,
                                    args.vc + vt * (TILE * D * VB / 8),
                                    args.vm + vt * (2 * TILE + D), lds);
    }
}

template <int D, int KB, int VB>
static hipError_t launch_q(const QuantArgs& a, hipStream_t s) {
    const int64_t blocks = a.n_k + a.n_v;
    hipLaunchKernelGGL((quantize_kernel<D, KB, VB>), dim3((unsigned)blocks), dim3(2 * D), 0, s, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_q_bits(const QuantArgs& a, int kb, int vb, hipStream_t s) {
    if (kb == 4 && vb == 2) return launch_q<D, 4, 2>(a, s);
    if (kb == 4 && vb == 4) return launch_q<D, 4, 4>(a, s);
    if (kb == 2 && vb == 2) return launch_q<D, 2, 2>(a, s);
    return launch_q<D, 2, 4>(a, s);
}

hipError_t launch_quantize(const QuantArgs& a, int D, int kb, int vb, hipStream_t s) {
    if (D == 64) return launch_q_bits<64>(a, kb, vb, s);
    if (D == 128) return launch_q_bits<128>(a, kb, vb, s);
    return launch_q_bits<256>(a, kb, vb, s);
}

}  // namespace kvarn
