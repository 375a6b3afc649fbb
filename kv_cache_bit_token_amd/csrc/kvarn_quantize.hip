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
// input is read from HBM exactly once; codes and meta are written straight
// from registers.
//
// Arithmetic, equal to the stated method in exact arithmetic:
//  * The transform runs unscaled: X' = sqrt(D) * Xt.  The normalised tile is
//    invariant to a global scale, so only the stored column factor and the K
//    scale/zero absorb the sqrt(D), divided out once per group.
//  * Log-space accumulation l_c += ln(sigma_c(current values)) gives
//    exp(l_c) = std over tokens of X'[t][c] * exp(-l_r[t]); the kernel keeps
//    these factors directly, as reciprocals (1/C[c] = exp(-l_c), 1/R[t] =
//    exp(-l_r), C and R themselves formed once at the end), and recomputes
//    each std from X' and the current cross-axis factors: the same quantity
//    without an exp/log round trip.
//  * Each std comes from the raw moments sum(v) and sum(v^2) of v = X' * f
//    (f the cross-axis factor) in one pass; the factor's reciprocal is the
//    hardware reciprocal square root of the variance (about 1 ulp).  Where
//    the mean is large next to the spread (4 mean^2 >= var, which includes
//    var <= 0 and so every flat group) the moments lose accuracy to
//    cancellation, and that pass is recomputed with the two-pass centred
//    formula: per tile for a column pass, per token for a row pass.
//  * A K group (one channel) is scaled by its own column factor, which
//    cancels in its codes and folds back in SK, ZK: the kernel quantises
//    X' * (1/R[t]) directly.  Likewise V quantises X' * (1/C[c]) and the row
//    factor cancels, so V skips the last row pass (its result is not used).
//  * A code is u = (v - z) * (L / range) rounded to the nearest integer, ties to even,
//    by the unsigned-byte conversion (which also clamps to [0, 255]), packed
//    four to a register and merged with shifts.
#include "kvarn_device.hpp"
#include "kvarn_internal.hpp"

namespace kvarn {

// round-to-nearest-even of u into byte SEL of acc (clamped to 0..255)
template <int SEL>
__device__ __forceinline__ uint32_t cvt_u8(float u, uint32_t acc) {
    return __builtin_amdgcn_cvt_pk_u8_f32(u, SEL, acc);
}

// Sum of v and of v^2 over n values v = x[k] * f[k] of one lane: one
// rounding per written operation (no contraction), so every caller forms
// the same bits.
template <int N>
__device__ __forceinline__ void lane_moments(const float (&x)[N], const float (&f)[N], float& s1,
                                             float& s2) {
#pragma clang fp contract(off)
    float v = x[0] * f[0];
    s1 = v;
    s2 = v * v;
#pragma unroll
    for (int k = 1; k < N; ++k) {
        v = x[k] * f[k];
        s1 = s1 + v;
        s2 = __builtin_fmaf(v, v, s2);
    }
}

// One 8-byte LDS read kept apart from its neighbours (the empty asm with a
// memory clobber stops the compiler from pairing reads into one two-address
// read: paired reads of the reducer pattern conflict in the LDS banks,
// single ones do not).
__device__ __forceinline__ float2 lds_read_single(const float2* p) {
    const float2 v = *p;
    asm volatile("" ::: "memory");
    return v;
}

template <int D, int BITS, bool IS_K, bool FULL>
__device__ __forceinline__ void quantize_tile(const uint16_t* __restrict__ xin, int d0, int n_iters,
                                              uint8_t* __restrict__ codes_out,
                                              uint16_t* __restrict__ meta_out, float* lds) {
    constexpr int R = D / CPL;          // lanes per row-group
    constexpr int NT = 2 * D;           // threads
    constexpr int L = (1 << BITS) - 1;  // top code
    using N = Net<R>;

    const int tid = threadIdx.x;
    const int cb = tid % R;
    const int tb = tid / R;
    const int nb = cb ^ N::kF;      // natural channel block loaded by this lane
    const int ob = N::nu(cb);       // Sylvester channel block held after the transform
    const float sqrtD = __builtin_sqrtf((float)D);
    const float rsqrtD = 1.0f / sqrtD;

    // Column partials (float2 per channel slot): thread n keeps its 16 at
    // entries [PST n, PST n + 16).  The odd stride puts the 32 lanes of a
    // half-wave on distinct bank pairs when they store the same slot.  The
    // reducer of lane position rp, half rh, sums the token groups
    // tb = k % DL + rh DL + (k / DL) 2 DL (k < 16, DL = 16 / R), so that the
    // two halves of a half-wave read entries 16 apart: no collision either.
    constexpr int PST = CPL + 1;
    constexpr int DL = 16 / R;
    float2* part = reinterpret_cast<float2*>(lds);   // [2D][PST]
    // Broadcast image padded to 20 floats per 16-channel block: the eight
    // blocks a wavefront reads with 16-byte loads then start on distinct
    // banks (unpadded, blocks 64 floats apart shared them, two-way).
    constexpr int CVN = D + D / 4;
    float* colv = lds + 4 * PST * D;                 // [CVN] broadcast of column stats
    float* colv2 = colv + CVN;                       // [CVN]
    int* flag = reinterpret_cast<int*>(colv2 + CVN); // [1] column-pass fallback request
    float* gsum = colv2 + CVN + 4;                   // [16] gauge partials

    // ---------------- load (one HBM read) + pad + first butterfly ----------------
    // FULL: d0 == D, no padding channels
    float x[TPL][CPL];
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
        const uint16_t* row = xin + (size_t)(4 * tb + i) * d0;
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
            const int ch0 = 16 * nb + 8 * hlf;
            uint4 w = make_uint4(0u, 0u, 0u, 0u);
            if (FULL || ch0 + 8 <= d0) w = *reinterpret_cast<const uint4*>(row + ch0);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int k = 0; k < 4; ++k)
                h2_butterfly(ws[k], x[i][8 * hlf + 2 * k], x[i][8 * hlf + 2 * k + 1]);
        }
    }

    // ---------------- rotation (unscaled) ----------------
    fwht_inlane<2>(x);
    fwht_crosslane<R>(x, cb);

    // ---------------- normalisation ----------------
    // Only the reciprocal factors are carried through the iterations:
    // R[t] = exp(l_r[t]) = 1 / a[t] and C = 1 / Cinv are formed once at the end.
    float a[TPL];                   // 1 / R[t] for my tokens
#pragma unroll
    for (int i = 0; i < TPL; ++i) a[i] = 1.0f;
    float b[CPL];                   // 1 / C[c] for my channels (unscaled units)
#pragma unroll
    for (int c = 0; c < CPL; ++c) b[c] = rsqrtD;

    // reducer role: position p = tid >> 1 (lane-position space), half rh
    const int rp = tid >> 1, rh = tid & 1;
    const int cwp = rp + 4 * (rp >> 4);   // my reducer position in the padded broadcast image
    const int crb = 20 * cb;              // my channel block in the padded broadcast image
    const float2* rpart = part + PST * (16 * rh + (rp >> 4)) + (rp & 15);
    float2* wpart = part + PST * tid;
    float Cinv = rsqrtD;   // 1 / column factor of position rp, unscaled units (exp(-l_c) / sqrt(D))
    if (tid == 0) *flag = 0;

    for (int it = 0; it < n_iters; ++it) {
        // ---- column pass: raw moments over tokens of x * a ----
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            // the sums start from the first term, not from 0 (no add of 0)
            const float v0 = x[0][c] * a[0];
            float s1 = v0, s2 = v0 * v0;
#pragma unroll
            for (int i = 1; i < TPL; ++i) {
                const float v = x[i][c] * a[i];
                s1 += v;
                s2 = __builtin_fmaf(v, v, s2);
            }
            wpart[c] = make_float2(s1, s2);
        }
        __syncthreads();
        const float Cinv_prev = Cinv;
        float cmean;
        {
            const float2 v0 = lds_read_single(rpart);
            float s1 = v0.x, s2 = v0.y;
#pragma unroll
            for (int k = 1; k < 16; ++k) {
                const float2 v = lds_read_single(rpart + PST * R * (k % DL + (k / DL) * 2 * DL));
                s1 += v.x;
                s2 += v.y;
            }
            s1 += dpp<DPP_XOR1>(s1);
            s2 += dpp<DPP_XOR1>(s2);
            // m2 = 2 mean, so t = 4 mean^2 serves both the variance and the test
            const float m2 = s1 * (2.0f / TILE);
            const float t = m2 * m2;
            cmean = 0.5f * m2;
            const float var = __builtin_fmaf(t, -0.25f, s2 * (1.0f / TILE));
            // accurate unless the mean dominates the spread (4 mean^2 >= var,
            // which also covers var <= 0)
            const bool ok = t < var;
            const float ci = __builtin_amdgcn_rsqf(var);
            Cinv = ok ? ci : Cinv;
            if (!ok) *flag = 1;
            if (rh == 0) colv[cwp] = Cinv;
        }
        __syncthreads();
        if (*flag) {
            // fallback: centred two-pass stds for every column of this pass
            // (the means are those of the raw pass)
            if (rh == 0) colv2[cwp] = cmean;
            __syncthreads();   // every thread has read the flag
            if (tid == 0) *flag = 0;
            float m[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) m[c] = colv2[crb + c];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                float q = 0.0f;
#pragma unroll
                for (int i = 0; i < TPL; ++i) {
                    const float d = __builtin_fmaf(x[i][c], a[i], -m[c]);
                    q = __builtin_fmaf(d, d, q);
                }
                wpart[c].x = q;
            }
            __syncthreads();
            {
                float q = 0.0f;
#pragma unroll
                for (int k = 0; k < 16; ++k) q += rpart[PST * R * (k % DL + (k / DL) * 2 * DL)].x;
                q += dpp<DPP_XOR1>(q);
                const float sd = __builtin_sqrtf(q * (1.0f / TILE));
                Cinv = is_flat(sd, cmean) ? Cinv_prev : 1.0f / sd;
                if (rh == 0) colv[cwp] = Cinv;
            }
            __syncthreads();
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) b[c] = colv[crb + c];

        // ---- row pass (V does not use the last one) ----
        if (!IS_K && it == n_iters - 1) break;
        // Per token: the row-group sums of the moments, each all-reduced
        // across the R lanes, and the centred fallback where the raw moments
        // are not accurate (4 mean^2 >= var; uniform across the row-group).
        auto row_pass_per_token = [&]() {
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                float s1, s2;
                lane_moments<CPL>(x[i], b, s1, s2);
                s1 = rg_sum<R>(s1);
                s2 = rg_sum<R>(s2);
                const float m2 = s1 * (2.0f / D);   // 2 mean
                const float t = m2 * m2;            // 4 mean^2
                const float var = __builtin_fmaf(t, -0.25f, s2 * (1.0f / D));
                float ai = __builtin_amdgcn_rsqf(var);
                if (!(t < var)) {
                    const float mean = 0.5f * m2;
                    float q = 0.0f;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        const float d = __builtin_fmaf(x[i][c], b[c], -mean);
                        q = __builtin_fmaf(d, d, q);
                    }
                    const float sd = __builtin_sqrtf(rg_sum<R>(q) * (1.0f / D));
                    ai = is_flat(sd, mean) ? a[i] : 1.0f / sd;
                }
                a[i] = ai;
            }
        };
        if constexpr (R >= 16) {
            // D = 256: the reduce-scatter below would cost this width its
            // occupancy (more VGPRs than 4 waves per SIMD allow)
            row_pass_per_token();
        } else {
            float s1[TPL], s2[TPL];
#pragma unroll
            for (int i = 0; i < TPL; ++i) lane_moments<CPL>(x[i], b, s1[i], s2[i]);
            // Reduce-scatter over the xor-1 and xor-2 steps of the row-group
            // sum, then an all-reduce of the one token left over the xor-7
            // step (R = 8).  With lane bits c0 c1 c2 of cb, the selectors are
            // b0 = c0 ^ c2 (tokens 0, 1 stay where b0 = 0, tokens 2, 3 where
            // b0 = 1) and b1 = c1 ^ c2, so each lane ends with token
            // u = 2 b0 + b1.  Each selector flips across its own step and
            // stays fixed across xor 7, so that step pairs lanes holding the
            // same token.  Every sum pairs the same lanes in the same order as
            // the per-token all-reduce: the results are the same bits, with 8
            // cross-lane adds instead of 24 and one reciprocal square root per
            // lane instead of four.
            const int c2 = (cb >> 2) & 1;
            const bool b0 = (cb & 1) ^ c2, b1 = ((cb >> 1) & 1) ^ c2;
            float r1[2], r2[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                r1[j] = (b0 ? s1[j + 2] : s1[j]) + dpp<DPP_XOR1>(b0 ? s1[j] : s1[j + 2]);
                r2[j] = (b0 ? s2[j + 2] : s2[j]) + dpp<DPP_XOR1>(b0 ? s2[j] : s2[j + 2]);
            }
            float u1 = (b1 ? r1[1] : r1[0]) + dpp<DPP_XOR2>(b1 ? r1[0] : r1[1]);
            float u2 = (b1 ? r2[1] : r2[0]) + dpp<DPP_XOR2>(b1 ? r2[0] : r2[1]);
            if constexpr (R >= 8) { u1 += dpp<DPP_HMIR>(u1); u2 += dpp<DPP_HMIR>(u2); }
            const float m2 = u1 * (2.0f / D);   // 2 mean
            const float t = m2 * m2;            // 4 mean^2
            const float var = __builtin_fmaf(t, -0.25f, u2 * (1.0f / D));
            if (__builtin_amdgcn_ballot_w64(!(t < var)) == 0) {
                // every token of the wave is accurate: gather the 4 factors
                const float au = __builtin_amdgcn_rsqf(var);
                const float g = dpp<DPP_XOR2>(au);                 // token u ^ 1
                const float A0 = b1 ? g : au, A1 = b1 ? au : g;   // tokens 2 b0, 2 b0 + 1
                const float h0 = dpp<DPP_XOR1>(A0), h1 = dpp<DPP_XOR1>(A1);
                a[0] = b0 ? h0 : A0;
                a[1] = b0 ? h1 : A1;
                a[2] = b0 ? A0 : h0;
                a[3] = b0 ? A1 : h1;
            } else {
                // some token of the wave needs the centred fallback
                row_pass_per_token();
            }
        }
    }

    // ---------------- gauge of the stored factors ----------------
    // The normalised tile depends on l_r[t] + l_c[c] only.  The mean column
    // log-factor is moved into the row factors (G = geometric mean of the
    // column factors) so the stored fp16 factors stay in range even when the
    // iteration drifts the two sets apart.  Codes are unaffected; only the
    // stored SK/ZK/RK (K) and SV/ZV/CV (V) see G.
    // Base-2 logarithms and powers on the hardware units: G only moves the
    // stored factors, so its own last-place error never reaches a code.
    float G, invG;
    {
        // log2 of the column factor; both lanes of a position: the sum is 2x
        float s = -__builtin_amdgcn_logf(Cinv * sqrtD);
        s = rg_sum<16>(s);   // sum over each 16-lane DPP row
        s = lane_f(s, 0) + lane_f(s, 16) + lane_f(s, 32) + lane_f(s, 48);
        if ((tid & 63) == 0) gsum[tid >> 6] = s;
        __syncthreads();
        float tot = gsum[0];
#pragma unroll
        for (int w = 1; w < NT / 64; ++w) tot += gsum[w];
        const float mean_l2 = tot * (0.5f / D);
        G = __builtin_amdgcn_exp2f(mean_l2);
        invG = __builtin_amdgcn_exp2f(-mean_l2);
    }
    // Sylvester channel index of the reducer's lane position
    const int kpos = 16 * N::nu(rp >> 4) + (rp & 15);

    // ---------------- quantisation, packing, stores ----------------
    if constexpr (IS_K) {
        // K: one group per channel, over the 128 tokens: values v = x * a[t]
#pragma unroll
        for (int i = 0; i < TPL; ++i)
#pragma unroll
            for (int c = 0; c < CPL; ++c) x[i][c] *= a[i];
        // (min, max) partials, same layout as the column moments
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float mn = fminf(fminf(x[0][c], x[1][c]), fminf(x[2][c], x[3][c]));
            float mx = fmaxf(fmaxf(x[0][c], x[1][c]), fmaxf(x[2][c], x[3][c]));
            wpart[c] = make_float2(mn, mx);
        }
        __syncthreads();
        {
            float2 v[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) v[k] = lds_read_single(rpart + PST * R * (k % DL + (k / DL) * 2 * DL));
            float mn = min3f(v[0].x, v[1].x, v[2].x), mx = max3f(v[0].y, v[1].y, v[2].y);
#pragma unroll
            for (int k = 3; k < 15; k += 2) {
                mn = min3f(mn, v[k].x, v[k + 1].x);
                mx = max3f(mx, v[k].y, v[k + 1].y);
            }
            mn = min3f(mn, v[15].x, dpp<DPP_XOR1>(min3f(mn, v[15].x, v[15].x)));
            mx = max3f(mx, v[15].y, dpp<DPP_XOR1>(max3f(mx, v[15].y, v[15].y)));
            const float zk = mn;
            const float range = mx - mn;
            const float sk = range * (1.0f / (float)L);
            const float inv = (range > 0.0f) ? (float)L * __builtin_amdgcn_rcpf(range) : 0.0f;
            if (rh == 0) {
                colv[cwp] = inv;
                colv2[cwp] = -zk * inv;
                meta_out[kpos] = f2h_bits(sk * rsqrtD * invG);        // SK
                meta_out[D + kpos] = f2h_bits(zk * rsqrtD * invG);    // ZK
            }
        }
        __syncthreads();
        if (cb == 0) {   // RK of my 4 tokens
            float rk[TPL];   // R[t] G
#pragma unroll
            for (int i = 0; i < TPL; ++i) rk[i] = G * __builtin_amdgcn_rcpf(a[i]);
            const uint32_t lo = f2h_bits(rk[0]) | ((uint32_t)f2h_bits(rk[1]) << 16);
            const uint32_t hi = f2h_bits(rk[2]) | ((uint32_t)f2h_bits(rk[3]) << 16);
            *reinterpret_cast<uint2*>(meta_out + 2 * D + 4 * tb) = make_uint2(lo, hi);
        }
        float inv[CPL], off[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) { inv[c] = colv[crb + c]; off[c] = colv2[crb + c]; }
        // token-major stream: token t, channels 16*ob .. +15 are contiguous
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            float u[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) u[c] = __builtin_fmaf(x[i][c], inv[c], off[c]);
            const int t = 4 * tb + i;
            if constexpr (BITS == 4) {
                uint32_t w[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float* q = u + 8 * h;
                    const uint32_t ev = cvt_u8<3>(q[6], cvt_u8<2>(q[4], cvt_u8<1>(q[2], cvt_u8<0>(q[0], 0u))));
                    const uint32_t od = cvt_u8<3>(q[7], cvt_u8<2>(q[5], cvt_u8<1>(q[3], cvt_u8<0>(q[1], 0u))));
                    w[h] = ev | (od << 4);
                }
                *reinterpret_cast<uint2*>(codes_out + (t * D + 16 * ob) / 2) = make_uint2(w[0], w[1]);
            } else {
                uint32_t p[4];
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    p[m] = cvt_u8<3>(u[12 + m], cvt_u8<2>(u[8 + m], cvt_u8<1>(u[4 + m], cvt_u8<0>(u[m], 0u))));
                *reinterpret_cast<uint32_t*>(codes_out + (t * D + 16 * ob) / 4) =
                    p[0] | (p[1] << 2) | (p[2] << 4) | (p[3] << 6);
            }
        }
    } else {
        // V: one group per token, over the D channels: values v = x * b[c]
        float inv[TPL], off[TPL], mn[TPL], mx[TPL];
        uint32_t sv2[TPL / 2], zv2[TPL / 2];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) x[i][c] *= b[c];
            mn[i] = x[i][0];
            mx[i] = x[i][0];
#pragma unroll
            for (int c = 1; c < CPL; ++c) { mn[i] = fminf(mn[i], x[i][c]); mx[i] = fmaxf(mx[i], x[i][c]); }
        }
        rg_minmax4<R, false>(mn);
        rg_minmax4<R, true>(mx);
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const float range = mx[i] - mn[i];
            const float sv = range * (1.0f / (float)L);
            inv[i] = (range > 0.0f) ? (float)L * __builtin_amdgcn_rcpf(range) : 0.0f;
            off[i] = -mn[i] * inv[i];
            const uint32_t hs = f2h_bits(sv * G), hz = f2h_bits(mn[i] * G);
            if (i & 1) { sv2[i / 2] |= hs << 16; zv2[i / 2] |= hz << 16; }
            else       { sv2[i / 2] = hs;        zv2[i / 2] = hz; }
        }
        if (cb == 0) {   // SV, ZV of my 4 tokens
            *reinterpret_cast<uint2*>(meta_out + 4 * tb) = make_uint2(sv2[0], sv2[1]);
            *reinterpret_cast<uint2*>(meta_out + TILE + 4 * tb) = make_uint2(zv2[0], zv2[1]);
        }
        if (rh == 0) meta_out[2 * TILE + kpos] = f2h_bits(invG * rsqrtD * __builtin_amdgcn_rcpf(Cinv));   // CV

        // Channel-major stream: channel k's codes of tokens 4*tb .. +3 form
        // BITS/2 bytes at k * (TILE * BITS / 8) + (BITS / 2) * tb.  Each lane packs
        // its channels, then lanes that hold neighbouring token groups of the
        // same channels swap through LDS (a transpose inside one wavefront)
        // so that every lane stores whole 32-bit words.  The partials are no
        // longer read by any wave (last read before the gauge barrier).
        constexpr int ROWB = TILE * BITS / 8;   // bytes per channel row
        uint32_t* xch = reinterpret_cast<uint32_t*>(lds);
        if constexpr (BITS == 2) {
            // p[q]: byte n = channel 16*ob + 4q + n, tokens 4*tb .. +3
            uint32_t p[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t t4[TPL];
#pragma unroll
                for (int i = 0; i < TPL; ++i) {
                    const float* xr = x[i] + 4 * q;
                    t4[i] = cvt_u8<3>(__builtin_fmaf(xr[3], inv[i], off[i]),
                            cvt_u8<2>(__builtin_fmaf(xr[2], inv[i], off[i]),
                            cvt_u8<1>(__builtin_fmaf(xr[1], inv[i], off[i]),
                            cvt_u8<0>(__builtin_fmaf(xr[0], inv[i], off[i]), 0u))));
                }
                p[q] = t4[0] | (t4[1] << 2) | (t4[2] << 4) | (t4[3] << 6);
            }
            // group of 4 lanes: token groups tb = 4m + j, same channel block
            *reinterpret_cast<uint4*>(xch + 4 * tid) = make_uint4(p[0], p[1], p[2], p[3]);
            wave_sync();
            const int j = tb & 3;
            const int base = tid - j * R;   // lane of token group 4m
            uint32_t r[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) r[jj] = xch[4 * (base + jj * R) + j];
            // 4x4 byte transpose: g[n] byte jj = r[jj] byte n
            const uint32_t A = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);
            const uint32_t B = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);
            const uint32_t C = __builtin_amdgcn_perm(r[3], r[2], 0x05010400u);
            const uint32_t E = __builtin_amdgcn_perm(r[3], r[2], 0x07030602u);
            const uint32_t g[4] = {__builtin_amdgcn_perm(C, A, 0x05040100u),
                                   __builtin_amdgcn_perm(C, A, 0x07060302u),
                                   __builtin_amdgcn_perm(E, B, 0x05040100u),
                                   __builtin_amdgcn_perm(E, B, 0x07060302u)};
            const int m = tb >> 2;
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const int k = 16 * ob + 4 * j + n;
                *reinterpret_cast<uint32_t*>(codes_out + k * ROWB + 4 * m) = g[n];
            }
        } else {
            // p[q]: channel 16*ob + 2q + e -> bytes 2e (tokens 0,1), 2e + 1 (tokens 2,3)
            uint32_t p[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int c0 = 2 * q, c1 = 2 * q + 1;
                const uint32_t ev = cvt_u8<3>(__builtin_fmaf(x[2][c1], inv[2], off[2]),
                                    cvt_u8<2>(__builtin_fmaf(x[0][c1], inv[0], off[0]),
                                    cvt_u8<1>(__builtin_fmaf(x[2][c0], inv[2], off[2]),
                                    cvt_u8<0>(__builtin_fmaf(x[0][c0], inv[0], off[0]), 0u))));
                const uint32_t od = cvt_u8<3>(__builtin_fmaf(x[3][c1], inv[3], off[3]),
                                    cvt_u8<2>(__builtin_fmaf(x[1][c1], inv[1], off[1]),
                                    cvt_u8<1>(__builtin_fmaf(x[3][c0], inv[3], off[3]),
                                    cvt_u8<0>(__builtin_fmaf(x[1][c0], inv[1], off[1]), 0u))));
                p[q] = ev | (od << 4);
            }
            // pairs of lanes: token groups tb = 2m + j
            *reinterpret_cast<uint4*>(xch + 8 * tid) = make_uint4(p[0], p[1], p[2], p[3]);
            *reinterpret_cast<uint4*>(xch + 8 * tid + 4) = make_uint4(p[4], p[5], p[6], p[7]);
            wave_sync();
            const int j = tb & 1;
            const int base = tid - j * R;
            const int m = tb >> 1;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t r0 = xch[8 * base + q], r1 = xch[8 * (base + R) + q];
                // channel 2q + j: halfword j of each lane's word
                const uint32_t g = j ? __builtin_amdgcn_perm(r1, r0, 0x07060302u)
                                     : __builtin_amdgcn_perm(r1, r0, 0x05040100u);
                const int k = 16 * ob + 2 * q + j;
                *reinterpret_cast<uint32_t*>(codes_out + k * ROWB + 4 * m) = g;
            }
        }
    }
}

// LDS floats: partials [2D][17] float2 + colv/colv2 [2][D + D/4] + flag/pad
// 4 + gauge 16; the V code exchange reuses the front.
template <int D>
constexpr int quant_lds_floats() { return 4 * (CPL + 1) * D + 2 * (D + D / 4) + 4 + 16; }

template <int D, int KB, int VB, bool FULL>
__global__ __launch_bounds__(2 * D) void quantize_kernel(QuantArgs args, int64_t b0) {
    __shared__ __align__(16) float lds[quant_lds_floats<D>()];
    const int64_t tile = b0 + blockIdx.x;   // K tiles, then V tiles
    const bool is_k = tile < args.n_k;
    const int64_t src = is_k ? tile : tile - args.n_k;
    // output slot: the tile itself, or its entry of dst (out-of-range entries
    // skip the tile; the test is uniform over the workgroup)
    int64_t slot = src;
    if (args.dst) {
        slot = args.dst[src];
        if (slot < 0 || slot >= args.pool) return;
    }
    if (is_k) {
        quantize_tile<D, KB, true, FULL>(args.k + src * TILE * args.d0, args.d0, args.n_iters,
                                         args.kc + slot * (TILE * D * KB / 8),
                                         args.km + slot * (2 * D + TILE), lds);
    } else {
        quantize_tile<D, VB, false, FULL>(args.v + src * TILE * args.d0, args.d0, args.n_iters,
                                          args.vc + slot * (TILE * D * VB / 8),
                                          args.vm + slot * (2 * TILE + D), lds);
    }
}

// One workgroup per tile, in launches of at most kMaxGrid workgroups.
template <int D, int KB, int VB>
static hipError_t launch_q(const QuantArgs& a, hipStream_t s) {
    auto kern = (a.d0 == D) ? quantize_kernel<D, KB, VB, true> : quantize_kernel<D, KB, VB, false>;
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
