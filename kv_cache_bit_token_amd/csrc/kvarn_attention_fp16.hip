// kvarn_attention_fp16.hip -- decode attention over an uncompressed fp16
// cache, gfx950: the baseline that the packed cache is measured against.
//
// Pages: hotdry page "KVarN Hadamard 旋转与方差归一化", section on the
// deployment parameters (throughput is compared with an FP16 baseline);
// deep page, section "一次 16K context 的推論，記憶體都花到哪去了" (every
// decode step reads the whole cache from HBM, so decode is bound by memory
// bandwidth and a smaller cache makes it faster).
//
//   out[b][h] = softmax(sm_scale * q[b][h] . K[b][g]^T) V[b][g]
//
// Work split: each wavefront owns one split of one (b, KV head) and every
// query head of its GQA group; split s of n takes token steps s, s + n,
// s + 2n, ..., so the n waves of a sequence read neighbouring steps at a
// time.  Waves do not synchronise before their last step; only the merge
// below uses LDS.  A step is TS = 32 * 128 / D tokens, so K and
// V of one step are 128 bytes per lane each.
//
// Matrix cores, v_mfma_f32_16x16x16_f16 (lane l: row / column l % 16,
// k-group l / 16):
//   q.K^T : A = K (16 tokens x 16 channels), B = q (16 channels x the
//           group's query heads, zero-padded to 16), C = scores[token][head];
//   p.V   : A = p (heads x 16 tokens), B = V (16 tokens x 16 channels).
// The C layout of q.K^T (lane: head l % 16, tokens 4 (l / 16) + i) is the A
// layout of p.V, so the probabilities never leave the lane.  fp16 q and K
// products are exact in fp32; p is split into fp16 hi + lo so the p.V
// products keep fp32 accuracy.  The contraction axis of q.K^T is permuted so
// that each lane reads whole 16-byte chunks (channels 8 (4 c + l / 16) ..
// + 7 for chunk c, and every load instruction covers 64 contiguous bytes of
// 16 rows); the output channels of p.V are permuted so that each lane reads
// one contiguous run of a V row (channels VCPL * (l % 16) .. + VCPL - 1).
//
// Loads run one step ahead: the next step's K right after this step's
// q.K^T, its V right after this step's p.V; every load is unconditional
// (rows past the sequence end read zero through a range-checked descriptor)
// so each wait covers a fixed number of younger loads.  Up to four splits
// of a (b, KV head) run as the waves of one workgroup and merge there
// through LDS; more splits go through a combine kernel.
#include "kvarn_device.hpp"
#include "kvarn_internal.hpp"
#include "kvarn_rsrc.hpp"

namespace kvarn {

namespace {

typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));

// Splits in total: about two per SIMD.  With strided splits this measured
// fastest on the 64 x 8 x 16384 and 64 x 8 x 32768 caches (four splits per
// sequence); 6, 8 or 12 splits per sequence were 4-20 % slower.
constexpr int kFp16TargetWaves = 2048;
constexpr float kLog2eF = 1.4426950408889634f;

template <int D>
struct Fp16Step {
    static constexpr int TS = 32 * 128 / D;     // tokens per step
    static constexpr int NMB = TS / 16;         // 16-token blocks per step
    static constexpr int NCH = D / 32;          // 16-byte K chunks per lane and token
    static constexpr int NKB = D / 16;          // q.K^T operands per block
    static constexpr int VCPL = D / 16;         // V channels per lane (= p.V N-blocks)
    static constexpr int VQ = VCPL / 8 > 0 ? VCPL / 8 : 1;   // 16-byte V loads per token
};

// fp16 half k of a run of dwords
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {   // {a.lo, b.lo}
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {   // {a.hi, b.hi}
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// The splits of one (b, KV head) as the waves of one workgroup (MERGE),
// merged there: each wave has written its (m, l, acc) per query head to
// ex[split][n][D + 2] in LDS and passed a barrier; the workgroup's threads
// then form the outputs exactly as the combine kernel does (same sums, same
// order).
template <int D>
__device__ void fp16_merge_in_block(const Fp16AttnArgs& a, const float* ex, int b, int g, int G) {
    const int ns = a.n_splits;
    for (int k = threadIdx.x; k < G * a.d0; k += blockDim.x) {
        const int n = k / a.d0, j = k % a.d0;
        float M = -INFINITY;
        for (int s = 0; s < ns; ++s) M = fmaxf(M, ex[((size_t)s * G + n) * (D + 2)]);
        float L = 0.0f;
        for (int s = 0; s < ns; ++s) {
            const float ms = ex[((size_t)s * G + n) * (D + 2)];
            if (ms != -INFINITY) L += ex[((size_t)s * G + n) * (D + 2) + 1] * exp2f((ms - M) * kLog2eF);
        }
        float v = 0.0f;
        for (int s = 0; s < ns; ++s) {
            const float ms = ex[((size_t)s * G + n) * (D + 2)];
            if (ms != -INFINITY) v += ex[((size_t)s * G + n) * (D + 2) + 2 + j] * exp2f((ms - M) * kLog2eF);
        }
        a.out[((size_t)b * a.n_q_heads + g * G + n) * a.d0 + j] = (L > 0.0f) ? v / L : 0.0f;
    }
}

template <int D, bool MERGE>
__global__ __launch_bounds__(256) void attn_fp16_partial_kernel(Fp16AttnArgs a) {
    using S = Fp16Step<D>;
    constexpr int TS = S::TS, NMB = S::NMB, NCH = S::NCH, NKB = S::NKB, VCPL = S::VCPL;
    constexpr int VW = VCPL / 2;                // dwords of V per lane and token
    const int lane = threadIdx.x & 63;
    // wave-uniform (scalar) so that the step's descriptors stay in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wpb = blockDim.x >> 6;
    const int G = a.n_q_heads / a.n_kv_heads;
    const int sgroups = (a.n_splits + wpb - 1) / wpb;
    const int bg = blockIdx.x / sgroups;
    const int split = (blockIdx.x % sgroups) * wpb + wave;
    if (split >= a.n_splits) return;
    const int b = bg / a.n_kv_heads, g = bg % a.n_kv_heads;
    const int64_t T = a.seq_len;
    const int64_t nsteps = (T + TS - 1) / TS;
    // strided splits: the k-th step of split s is step s + k * n_splits
    const int64_t s0 = 0;
    const int64_t s1 = split < nsteps ? (nsteps - split + a.n_splits - 1) / a.n_splits : 0;
    auto step_of = [&](int64_t k) { return (int64_t)split + (k < s1 ? k : s1 - 1) * a.n_splits; };
    // the split's partial: in the workspace, or (MERGE) in LDS for the workgroup
    extern __shared__ __align__(16) float ex[];
    auto part = [&](int n) {
        if constexpr (MERGE) return ex + ((size_t)split * G + n) * (D + 2);
        return a.ws + (((size_t)b * a.n_q_heads + g * G + n) * a.n_splits + split) * (D + 2);
    };
    if (s0 >= s1) {
        for (int k = lane; k < G * (D + 2); k += 64)
            part(k / (D + 2))[k % (D + 2)] = (k % (D + 2) == 0) ? -INFINITY : 0.0f;
        if constexpr (MERGE) {
            __syncthreads();
            fp16_merge_in_block<D>(a, ex, b, g, G);
        }
        return;
    }
    const int mrow = lane & 15, mgrp = lane >> 4;
    const int d0 = a.d0;

    // q operand: head mrow, chunk c = channels 8 (4 c + mgrp) .. + 7; chunks
    // past head_dim are zero, so the K chunks read there (the next row's
    // leading channels, or zero past the last row) contribute nothing; V
    // channels past head_dim only feed output columns that are never stored.
    uint4 qr[NCH];
    {
        const bool live = mrow < G;
        const uint16_t* qrow = a.q + ((size_t)b * a.n_q_heads + g * G + (live ? mrow : 0)) * d0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int ch = 8 * (4 * c + mgrp);
            const uint4 w = *reinterpret_cast<const uint4*>(qrow + min(ch, d0 - 8));
            qr[c] = (live && ch < d0) ? w : make_uint4(0u, 0u, 0u, 0u);
        }
    }

    // Buffer descriptors, one per step: base at the step's first row of this
    // (b, g), range up to the sequence end.  Every row and chunk offset sits
    // in the per-lane offset, which the hardware checks against the range
    // (the scalar offset is not checked, so it stays 0): a load past the last
    // row returns zero without touching memory, and a partial last step needs
    // no clamping.
    const int rowb = 2 * d0;
    const uint16_t* kbase = a.k + (size_t)bg * T * d0;
    const uint16_t* vbase = a.v + (size_t)bg * T * d0;
    // K: token 16 mb + mrow, chunk c at byte 16 (4 c + mgrp) of the row
    const int kvo = mrow * rowb + 16 * mgrp;
    // V: token 16 kb + 4 mgrp + e, channels VCPL * mrow ..
    const int vvo = 4 * mgrp * rowb + 2 * VCPL * mrow;
    uint4 kr[NMB][NCH];
    uint32_t vr[NMB][4][VW];
    auto load_k = [&](int64_t k) {
        const int64_t r0 = step_of(k) * TS;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(kbase + r0 * d0, (uint32_t)((T - r0) * rowb));
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
            for (int c = 0; c < NCH; ++c)
                kr[mb][c] = buf_load16<kPolicyNT>(r, kvo + 16 * mb * rowb + 64 * c, 0);
        }
    };
    auto load_v = [&](int64_t k) {
        const int64_t r0 = step_of(k) * TS;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(vbase + r0 * d0, (uint32_t)((T - r0) * rowb));
#pragma unroll
        for (int kb2 = 0; kb2 < NMB; ++kb2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int vo = vvo + (16 * kb2 + e) * rowb;
                if constexpr (VCPL == 4) {
                    const uint2 w = buf_load8<kPolicyNT>(r, vo, 0);
                    vr[kb2][e][0] = w.x;
                    vr[kb2][e][1] = w.y;
                } else {
#pragma unroll
                    for (int u = 0; u < VCPL / 8; ++u) {
                        const uint4 w = buf_load16<kPolicyNT>(r, vo + 16 * u, 0);
                        vr[kb2][e][4 * u + 0] = w.x;
                        vr[kb2][e][4 * u + 1] = w.y;
                        vr[kb2][e][4 * u + 2] = w.z;
                        vr[kb2][e][4 * u + 3] = w.w;
                    }
                }
            }
        }
    };

    float m_run = -INFINITY, l_run = 0.0f;   // head mrow
    f4_t acc[VCPL];                          // heads 4 mgrp + i, channel VCPL * mrow + nb
#pragma unroll
    for (int nb = 0; nb < VCPL; ++nb) acc[nb] = (f4_t){0.0f, 0.0f, 0.0f, 0.0f};

    load_k(s0);
    load_v(s0);
    for (int64_t st = s0; st < s1; ++st) {
        // ---- scores (tokens past the sequence end masked) ----
        const int rem = (int)min(T - step_of(st) * TS, (int64_t)TS);
        float s[NMB][4];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
            f4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < NKB; ++k) {
                const uint4 w = kr[mb][k >> 1];
                const uint4 qw = qr[k >> 1];
                const h4_t av = __builtin_bit_cast(h4_t, (k & 1) ? make_uint2(w.z, w.w) : make_uint2(w.x, w.y));
                const h4_t bv = __builtin_bit_cast(h4_t, (k & 1) ? make_uint2(qw.z, qw.w) : make_uint2(qw.x, qw.y));
                c = __builtin_amdgcn_mfma_f32_16x16x16f16(av, bv, c, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) s[mb][i] = (16 * mb + 4 * mgrp + i < rem) ? a.sm_scale * c[i] : -INFINITY;
        }
        load_k(st + 1);
        // keep the V-side work below (it waits for this step's V loads)
        // from being hoisted above the K-side work
        __builtin_amdgcn_sched_barrier(0);

        // ---- online softmax of head mrow over the step ----
        float mt = s[0][0];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mt = fmaxf(mt, s[mb][i]);
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mnew = fmaxf(m_run, mt);
        const float al = exp2f((m_run - mnew) * kLog2eF);
        const bool live = mrow < G;
        float lt = 0.0f;
        h4_t pa_hi[NMB], pa_lo[NMB];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = live ? exp2f((s[mb][i] - mnew) * kLog2eF) : 0.0f;
                lt += p;
                const _Float16 hi = (_Float16)p;
                pa_hi[mb][i] = hi;
                pa_lo[mb][i] = (_Float16)(p - (float)hi);
            }
        }
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        m_run = mnew;
        l_run = l_run * al + lt;
        __builtin_amdgcn_sched_barrier(0);

        // ---- acc = acc * alpha + p.V ----
        float ai[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ai[i] = __shfl(al, 4 * mgrp + i);
#pragma unroll
        for (int nb = 0; nb < VCPL; ++nb) {
            f4_t c = acc[nb];
#pragma unroll
            for (int i = 0; i < 4; ++i) c[i] *= ai[i];
            const int dw = nb >> 1;
#pragma unroll
            for (int k = 0; k < NMB; ++k) {
                const uint32_t x0 = (nb & 1) ? pair_hi(vr[k][0][dw], vr[k][1][dw]) : pair_lo(vr[k][0][dw], vr[k][1][dw]);
                const uint32_t x1 = (nb & 1) ? pair_hi(vr[k][2][dw], vr[k][3][dw]) : pair_lo(vr[k][2][dw], vr[k][3][dw]);
                const h4_t bv = __builtin_bit_cast(h4_t, make_uint2(x0, x1));
                c = __builtin_amdgcn_mfma_f32_16x16x16f16(pa_hi[k], bv, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x16f16(pa_lo[k], bv, c, 0, 0, 0);
            }
            acc[nb] = c;
        }
        load_v(st + 1);
    }

    // ---- partial result: (m, l, acc[D]) per query head ----
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int n = 4 * mgrp + i;
        if (n < G) {
            float* p = part(n);
#pragma unroll
            for (int nb = 0; nb < VCPL; ++nb) p[2 + VCPL * mrow + nb] = acc[nb][i];
        }
    }
    if (mgrp == 0 && mrow < G) {
        float* p = part(mrow);
        p[0] = m_run;
        p[1] = l_run;
    }
    if constexpr (MERGE) {
        __syncthreads();
        fp16_merge_in_block<D>(a, ex, b, g, G);
    }
}

template <int D>
__global__ __launch_bounds__(256) void attn_fp16_combine_kernel(Fp16AttnArgs a) {
    const int bh = blockIdx.x;   // b * n_q_heads + h
    const int ns = a.n_splits;
    const float* p = a.ws + (size_t)bh * ns * (D + 2);
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, p[s * (D + 2)]);
    float L = 0.0f;
    for (int s = 0; s < ns; ++s) {
        const float ms = p[s * (D + 2)];
        if (ms != -INFINITY) L += p[s * (D + 2) + 1] * exp2f((ms - M) * kLog2eF);
    }
    for (int j = threadIdx.x; j < a.d0; j += blockDim.x) {
        float v = 0.0f;
        for (int s = 0; s < ns; ++s) {
            const float ms = p[s * (D + 2)];
            if (ms != -INFINITY) v += p[s * (D + 2) + 2 + j] * exp2f((ms - M) * kLog2eF);
        }
        a.out[(size_t)bh * a.d0 + j] = (L > 0.0f) ? v / L : 0.0f;
    }
}

// Any GQA group of up to 16 heads fills the 16 columns of the matrix-core
// tiles, so one instantiation per head_dim serves every group size.
template <int D>
hipError_t launch_f16(const Fp16AttnArgs& a, hipStream_t s) {
    if (a.n_splits > 0 && a.n_splits <= 4) {
        // a (b, g)'s splits fit one workgroup: they run as its waves and merge
        // there through n_splits x G x (D + 2) floats of LDS, no combine launch
        const int G = a.n_q_heads / a.n_kv_heads;
        const size_t lds = (size_t)a.n_splits * G * (D + 2) * sizeof(float);
        hipLaunchKernelGGL((attn_fp16_partial_kernel<D, true>), dim3((unsigned)((int64_t)a.batch * a.n_kv_heads)),
                           dim3(64 * a.n_splits), lds, s, a);
        return hipGetLastError();
    }
    if (a.n_splits > 0) {
        constexpr int wpb = 4;
        const int64_t sgroups = (a.n_splits + wpb - 1) / wpb;
        const int64_t blocks = (int64_t)a.batch * a.n_kv_heads * sgroups;
        hipLaunchKernelGGL((attn_fp16_partial_kernel<D, false>), dim3((unsigned)blocks), dim3(64 * wpb),
                           0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((attn_fp16_combine_kernel<D>), dim3((unsigned)(a.batch * a.n_q_heads)), dim3(128),
                       0, s, a);
    return hipGetLastError();
}

}  // namespace

int attention_fp16_splits(int batch, int n_kv_heads, int64_t seq_len, int D) {
    const int64_t ts = 32 * 128 / D;
    const int64_t nsteps = seq_len > 0 ? (seq_len + ts - 1) / ts : 0;
    const int64_t pairs = (int64_t)batch * n_kv_heads;
    if (nsteps == 0 || pairs == 0) return 0;
    int64_t want = (kFp16TargetWaves + pairs - 1) / pairs;
    if (want > nsteps) want = nsteps;
    if (want < 1) want = 1;
    const int64_t per = (nsteps + want - 1) / want;
    return (int)((nsteps + per - 1) / per);
}

hipError_t launch_attention_fp16(const Fp16AttnArgs& a, int D, hipStream_t s) {
    if ((int64_t)a.batch * a.n_q_heads == 0) return hipSuccess;
    if (D == 64) return launch_f16<64>(a, s);
    if (D == 128) return launch_f16<128>(a, s);
    return launch_f16<256>(a, s);
}

}  // namespace kvarn
