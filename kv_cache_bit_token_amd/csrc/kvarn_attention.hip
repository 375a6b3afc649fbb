// kvarn_attention.hip -- decode attention over the packed KVarN cache, gfx950.
//
// Method (digest page "KVarN: 方差归一化的KV-Cache量化...", "方法" module 3: the
// quantised cache takes part in attention after the scales are restored;
// deep-dive page, stage card "Hadamard rotation": the rotation is orthonormal,
// so q.k is unchanged; hotdry page "非对称量化与尺度折叠": per-channel K
// scales, per-token V scales, folded back on read).
//
// Everything runs in the rotated domain; nothing is dequantised to memory:
//   qh = H q / sqrt(D)                       (once per (b, head), zero-padded)
//   s_t = sm_scale * RK_t * (sum_j (qh_j SK_j) (code_tj - mk) + sum_j qh_j (ZK_j + mk SK_j))
//   online softmax over the tiles of a split
//   acc_j = CV_j (sum_t p_t SV_t (code_tj - mv) + sum_t p_t (ZV_t + mv SV_t))
//   o = H (acc / l) / sqrt(D), first head_dim channels      (combine kernel)
// mk = (2^k_bits - 1)/2 and mv = (2^v_bits - 1)/2 centre the codes: ZK is the
// group minimum, so sum_j qh_j SK_j code_tj and sum_j qh_j ZK_j are large
// and of opposite sign; centred, neither term carries the cancellation and
// the fp32 score keeps its accuracy when the scores are large.
// Split-K: each workgroup owns one (b, KV head, split) and all the query
// heads of that KV head's GQA group; a combine kernel merges the splits'
// (max, sum, acc) partials and applies the inverse rotation.
#include "kvarn_device.hpp"
#include "kvarn_internal.hpp"

namespace kvarn {

constexpr int ATT_THREADS = 256;
constexpr int kTargetBlocks = 2048;   // enough workgroups to fill 256 CUs several times

void attention_plan(int batch, int n_kv_heads, int tiles_per_seq, int* n_splits,
                    int* tiles_per_split) {
    const int64_t pairs = (int64_t)batch * n_kv_heads;
    int ns = 1;
    if (pairs > 0 && tiles_per_seq > 0) {
        int64_t want = (kTargetBlocks + pairs - 1) / pairs;
        if (want > tiles_per_seq) want = tiles_per_seq;
        if (want < 1) want = 1;
        ns = (int)want;
    }
    int tps = tiles_per_seq > 0 ? (tiles_per_seq + ns - 1) / ns : 0;
    if (tps > 0) ns = (tiles_per_seq + tps - 1) / tps;
    *n_splits = ns;
    *tiles_per_split = tps;
}

size_t attention_workspace_bytes(int batch, int n_q_heads, int D, int n_splits) {
    return (size_t)batch * n_q_heads * n_splits * (D + 2) * sizeof(float);
}

// In-LDS Walsh-Hadamard transform of `rows` vectors of length D (natural
// order), scaled by 1/sqrt(D).
template <int D>
__device__ void lds_fwht(float* v, int rows) {
    const int tid = threadIdx.x;
    for (int h = 1; h < D; h <<= 1) {
        for (int k = tid; k < rows * D / 2; k += blockDim.x) {
            const int r = k / (D / 2), p = k % (D / 2);
            const int lo = (p / h) * 2 * h + (p % h), hi = lo + h;
            const float a = v[r * D + lo], b = v[r * D + hi];
            v[r * D + lo] = a + b;
            v[r * D + hi] = a - b;
        }
        __syncthreads();
    }
    const float sc = 1.0f / __builtin_sqrtf((float)D);
    for (int k = tid; k < rows * D; k += blockDim.x) v[k] *= sc;
    __syncthreads();
}

template <int D, int KB, int VB>
__global__ __launch_bounds__(ATT_THREADS) void attn_partial_kernel(AttnArgs a) {
    constexpr int KCB = TILE * D * KB / 8, VCB = TILE * D * VB / 8;
    constexpr int KMH = 2 * D + TILE, VMH = 2 * TILE + D;
    constexpr uint32_t KMASK = (1u << KB) - 1, VMASK = (1u << VB) - 1;
    constexpr float MK = 0.5f * (float)KMASK, MV = 0.5f * (float)VMASK;
    constexpr int GMAX = 16;
    __shared__ float qrot[GMAX * D];
    __shared__ float qs[GMAX * D];
    __shared__ float sc[GMAX * TILE];
    __shared__ float qz[GMAX], pz[GMAX], alpha[GMAX], mrun[GMAX], lrun[GMAX];
    __shared__ uint4 kimg[(KCB + 2 * KMH) / 16];
    __shared__ uint4 vimg[(VCB + 2 * VMH) / 16];

    const int tid = threadIdx.x;
    const int G = a.n_q_heads / a.n_kv_heads;
    const int blk = blockIdx.x;
    const int split = blk % a.n_splits;
    const int bg = blk / a.n_splits;
    const int b = bg / a.n_kv_heads, g = bg % a.n_kv_heads;
    const int t0 = split * a.tiles_per_split;
    int t1 = t0 + a.tiles_per_split;
    if (t1 > a.tiles_per_seq) t1 = a.tiles_per_seq;

    // rotated queries of the group
    for (int k = tid; k < G * D; k += ATT_THREADS) {
        const int hh = k / D, j = k % D;
        const int h = g * G + hh;
        qrot[k] = (j < a.d0) ? h2f_bits(a.q[((size_t)b * a.n_q_heads + h) * a.d0 + j]) : 0.0f;
    }
    if (tid < G) { mrun[tid] = -INFINITY; lrun[tid] = 0.0f; }
    __syncthreads();
    lds_fwht<D>(qrot, G);

    float acc[GMAX * D / ATT_THREADS > 0 ? GMAX * D / ATT_THREADS : 1];
    const int npairs = G * D;
#pragma unroll
    for (int r = 0; r < (int)(sizeof(acc) / sizeof(float)); ++r) acc[r] = 0.0f;

    const uint8_t* kcode = reinterpret_cast<const uint8_t*>(kimg);
    const uint16_t* kmeta = reinterpret_cast<const uint16_t*>(kcode + KCB);
    const uint8_t* vcode = reinterpret_cast<const uint8_t*>(vimg);
    const uint16_t* vmeta = reinterpret_cast<const uint16_t*>(vcode + VCB);

    for (int ti = t0; ti < t1; ++ti) {
        const int64_t tile = (int64_t)bg * a.tiles_per_seq + ti;
        {
            const uint4* src = reinterpret_cast<const uint4*>(a.kc + tile * KCB);
            for (int k = tid; k < KCB / 16; k += ATT_THREADS) kimg[k] = src[k];
            const uint4* msrc = reinterpret_cast<const uint4*>(a.km + tile * KMH);
            for (int k = tid; k < 2 * KMH / 16; k += ATT_THREADS) kimg[KCB / 16 + k] = msrc[k];
            const uint4* vsrc = reinterpret_cast<const uint4*>(a.vc + tile * VCB);
            for (int k = tid; k < VCB / 16; k += ATT_THREADS) vimg[k] = vsrc[k];
            const uint4* vmsrc = reinterpret_cast<const uint4*>(a.vm + tile * VMH);
            for (int k = tid; k < 2 * VMH / 16; k += ATT_THREADS) vimg[VCB / 16 + k] = vmsrc[k];
        }
        __syncthreads();
        // q folded with the per-channel K scale; zero-point term per head
        for (int k = tid; k < G * D; k += ATT_THREADS) qs[k] = qrot[k] * h2f_bits(kmeta[k % D]);
        if (tid < G) {
            float z = 0.0f;
            for (int j = 0; j < D; ++j)
                z = __builtin_fmaf(qrot[tid * D + j],
                                   __builtin_fmaf(MK, h2f_bits(kmeta[j]), h2f_bits(kmeta[D + j])), z);
            qz[tid] = z;
        }
        __syncthreads();
        // scores
        for (int k = tid; k < G * TILE; k += ATT_THREADS) {
            const int hh = k / TILE, t = k % TILE;
            float s = 0.0f;
            for (int j = 0; j < D; ++j) {
                const int64_t e = (int64_t)t * D + j;
                const uint32_t c = (kcode[(e * KB) >> 3] >> ((e * KB) & 7)) & KMASK;
                s = __builtin_fmaf(qs[hh * D + j], (float)c - MK, s);
            }
            sc[k] = a.sm_scale * h2f_bits(kmeta[2 * D + t]) * (s + qz[hh]);
        }
        __syncthreads();
        // online softmax, one wave per head
        {
            const int w = tid / 64, lane = tid % 64;
            for (int hh = w; hh < G; hh += ATT_THREADS / 64) {
                float m = fmaxf(sc[hh * TILE + lane], sc[hh * TILE + 64 + lane]);
                for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
                const float mnew = fmaxf(mrun[hh], m);
                const float p0 = __expf(sc[hh * TILE + lane] - mnew);
                const float p1 = __expf(sc[hh * TILE + 64 + lane] - mnew);
                float l = p0 + p1;
                const float sv0 = h2f_bits(vmeta[lane]), sv1 = h2f_bits(vmeta[64 + lane]);
                const float zv0 = h2f_bits(vmeta[TILE + lane]), zv1 = h2f_bits(vmeta[TILE + 64 + lane]);
                float z = p0 * __builtin_fmaf(MV, sv0, zv0) + p1 * __builtin_fmaf(MV, sv1, zv1);
                for (int o = 32; o > 0; o >>= 1) { l += __shfl_xor(l, o); z += __shfl_xor(z, o); }
                sc[hh * TILE + lane] = p0 * sv0;
                sc[hh * TILE + 64 + lane] = p1 * sv1;
                if (lane == 0) {
                    const float al = __expf(mrun[hh] - mnew);
                    alpha[hh] = al;
                    lrun[hh] = lrun[hh] * al + l;
                    mrun[hh] = mnew;
                    pz[hh] = z;
                }
            }
        }
        __syncthreads();
        // p V accumulation (per channel, over the tile's tokens)
#pragma unroll
        for (int r = 0; r < (int)(sizeof(acc) / sizeof(float)); ++r) {
            const int k = tid + r * ATT_THREADS;
            if (k < npairs) {
                const int hh = k / D, j = k % D;
                float s = 0.0f;
                for (int t = 0; t < TILE; ++t) {
                    const int64_t e = (int64_t)j * TILE + t;
                    const uint32_t c = (vcode[(e * VB) >> 3] >> ((e * VB) & 7)) & VMASK;
                    s = __builtin_fmaf(sc[hh * TILE + t], (float)c - MV, s);
                }
                acc[r] = acc[r] * alpha[hh] + h2f_bits(vmeta[2 * TILE + j]) * (s + pz[hh]);
            }
        }
        __syncthreads();
    }

    // partial out: [b][h][split][D + 2] = (m, l, acc)
#pragma unroll
    for (int r = 0; r < (int)(sizeof(acc) / sizeof(float)); ++r) {
        const int k = tid + r * ATT_THREADS;
        if (k < npairs) {
            const int hh = k / D, j = k % D;
            const int h = g * G + hh;
            float* p = a.ws + (((size_t)b * a.n_q_heads + h) * a.n_splits + split) * (D + 2);
            p[2 + j] = acc[r];
            if (j == 0) { p[0] = mrun[hh]; p[1] = lrun[hh]; }
        }
    }
}

template <int D>
__global__ __launch_bounds__(ATT_THREADS) void attn_combine_kernel(AttnArgs a) {
    __shared__ float o[D];
    __shared__ float wsum[1];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x;   // b * n_q_heads + h
    const float* p = a.ws + (size_t)bh * a.n_splits * (D + 2);
    float M = -INFINITY;
    for (int s = 0; s < a.n_splits; ++s) M = fmaxf(M, p[s * (D + 2)]);
    float L = 0.0f;
    for (int s = 0; s < a.n_splits; ++s) {
        const float ms = p[s * (D + 2)];
        if (ms != -INFINITY) L += p[s * (D + 2) + 1] * __expf(ms - M);
    }
    if (tid == 0) wsum[0] = L;
    for (int j = tid; j < D; j += ATT_THREADS) {
        float v = 0.0f;
        for (int s = 0; s < a.n_splits; ++s) {
            const float ms = p[s * (D + 2)];
            if (ms != -INFINITY) v += p[s * (D + 2) + 2 + j] * __expf(ms - M);
        }
        o[j] = (L > 0.0f) ? v / L : 0.0f;
    }
    __syncthreads();
    lds_fwht<D>(o, 1);
    for (int j = tid; j < a.d0; j += ATT_THREADS) a.out[(size_t)bh * a.d0 + j] = o[j];
}

__global__ void fill_zero_kernel(float* out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = 0.0f;
}

template <int D, int KB, int VB>
static hipError_t launch_att(const AttnArgs& a, hipStream_t s) {
    const int64_t blocks = (int64_t)a.batch * a.n_kv_heads * a.n_splits;
    hipLaunchKernelGGL((attn_partial_kernel<D, KB, VB>), dim3((unsigned)blocks), dim3(ATT_THREADS),
                       0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((unsigned)(a.batch * a.n_q_heads)),
                       dim3(ATT_THREADS), 0, s, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_att_bits(const AttnArgs& a, int kb, int vb, hipStream_t s) {
    if (kb == 4 && vb == 2) return launch_att<D, 4, 2>(a, s);
    if (kb == 4 && vb == 4) return launch_att<D, 4, 4>(a, s);
    if (kb == 2 && vb == 2) return launch_att<D, 2, 2>(a, s);
    return launch_att<D, 2, 4>(a, s);
}

hipError_t launch_attention(const AttnArgs& a, int D, int kb, int vb, hipStream_t s) {
    if (a.tiles_per_seq == 0) {
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
