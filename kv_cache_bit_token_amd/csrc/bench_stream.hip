// bench_stream.hip -- streaming reference kernels for the benchmark (not part
// of the KVarN library's ABI; built into its own libkvarn_streamref.so).
//
// A plain kernel that moves the same bytes as a KVarN stage, with no
// arithmetic to speak of, measures what this device actually delivers for
// that read/write mix: the "achievable" rate that the stage's HBM fraction is
// read against, beside the nominal 8 TB/s.  One unit = read `rq` 16-byte
// words, write `wq` 16-byte words (per tile pair: quantize reads 65 536 B and
// writes 13 824 B; dequantize the reverse; attention only reads).  Every
// written word depends on the words the same thread read, so neither side can
// be dropped by the compiler.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void stream_mix_kernel(const uint4* __restrict__ src,
                                                         uint4* __restrict__ dst, int64_t units,
                                                         int rq, int wq, uint32_t* sink) {
    uint4 acc = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        const uint4* s = src + u * rq;
        for (int i = threadIdx.x; i < rq; i += blockDim.x) {
            const uint4 v = s[i];
            acc.x ^= v.x; acc.y ^= v.y; acc.z ^= v.z; acc.w ^= v.w;
        }
        uint4* d = dst + u * wq;
        for (int i = threadIdx.x; i < wq; i += blockDim.x)
            d[i] = make_uint4(acc.x ^ (uint32_t)i, acc.y, acc.z, acc.w);
    }
    // read-only mixes: one word per thread that sees a nonzero sum (never, for
    // the benchmark's inputs, but the compiler cannot know)
    if (wq == 0 && (acc.x & acc.y & acc.z & acc.w) == 0xFFFFFFFFu) sink[threadIdx.x] = acc.x;
}

// The same with the word counts fixed at compile time (loops fully unrolled:
// a thread's loads all in flight before its stores), for the tile-pair mixes
// at head_dim 128.  NT: stores carry the nontemporal hint.
template <int RQ, int WQ, bool NT>
__global__ __launch_bounds__(256) void stream_mix_fixed(const uint4* __restrict__ src,
                                                        uint4* __restrict__ dst, int64_t units,
                                                        uint32_t* sink) {
    constexpr int RL = (RQ + 255) / 256, WL = (WQ + 255) / 256;
    uint4 acc = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        const uint4* s = src + u * RQ;
        uint4 v[RL > 0 ? RL : 1];
#pragma unroll
        for (int k = 0; k < RL; ++k) {
            const int i = threadIdx.x + 256 * k;
            v[k] = (i < RQ) ? s[i] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int k = 0; k < RL; ++k) { acc.x ^= v[k].x; acc.y ^= v[k].y; acc.z ^= v[k].z; acc.w ^= v[k].w; }
        if constexpr (WQ > 0) {
            uint4* d = dst + u * WQ;
#pragma unroll
            for (int k = 0; k < WL; ++k) {
                const int i = threadIdx.x + 256 * k;
                if (i < WQ) {
                    if constexpr (NT) {
                        using u32x4 = uint32_t __attribute__((ext_vector_type(4)));
                        const u32x4 w = {acc.x ^ (uint32_t)i, acc.y, acc.z, acc.w};
                        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(d + i));
                    } else {
                        d[i] = make_uint4(acc.x ^ (uint32_t)i, acc.y, acc.z, acc.w);
                    }
                }
            }
        }
    }
    if (WQ == 0 && (acc.x & acc.y & acc.z & acc.w) == 0xFFFFFFFFu) sink[threadIdx.x] = acc.x;
}

// Phased variant: each workgroup reads the words of NB units (all loads in
// flight together), then writes the NB units' outputs with nontemporal
// stores, so every workgroup alternates long read and write bursts instead
// of interleaving them unit by unit.
template <int RQ, int WQ, int NB>
__global__ __launch_bounds__(256) void stream_mix_phased(const uint4* __restrict__ src,
                                                         uint4* __restrict__ dst, int64_t units,
                                                         uint32_t* sink) {
    constexpr int RL = (NB * RQ + 255) / 256, WL = (WQ + 255) / 256;
    using u32x4 = uint32_t __attribute__((ext_vector_type(4)));
    uint4 acc = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t u0 = (int64_t)blockIdx.x * NB; u0 < units; u0 += (int64_t)gridDim.x * NB) {
        const int nb = (int)((units - u0) < NB ? (units - u0) : NB);
        const uint4* s = src + u0 * RQ;
        uint4 v[RL];
#pragma unroll
        for (int k = 0; k < RL; ++k) {
            const int i = threadIdx.x + 256 * k;
            v[k] = (i < nb * RQ) ? s[i] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int k = 0; k < RL; ++k) { acc.x ^= v[k].x; acc.y ^= v[k].y; acc.z ^= v[k].z; acc.w ^= v[k].w; }
        for (int un = 0; un < nb; ++un) {
            uint4* d = dst + (u0 + un) * WQ;
#pragma unroll
            for (int k = 0; k < WL; ++k) {
                const int i = threadIdx.x + 256 * k;
                if (i < WQ) {
                    const u32x4 w = {acc.x ^ (uint32_t)i, acc.y ^ (uint32_t)un, acc.z, acc.w};
                    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(d + i));
                }
            }
        }
    }
    if ((acc.x & acc.y & acc.z & acc.w) == 0xFFFFFFFFu) sink[threadIdx.x] = acc.x;
}

// Vector-ALU reference: eight independent fp32 multiply-add chains per
// lane, 16 v_fma per loop trip with VGPR operands, nothing else but the loop
// counter.  It measures the issue rate of plain fp32 multiply-adds at a
// chosen number of waves per SIMD (the grid size), the arithmetic
// counterpart of the streaming kernels above.  Lane 0 of every wave also
// records its shader-clock and 100 MHz wall-clock ticks, which give the
// engine clock the chip ran at.
__global__ __launch_bounds__(256) void valu_fma_kernel(float* __restrict__ out,
                                                       long long* __restrict__ ticks, int iters,
                                                       float a, float b) {
    float r[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = (float)threadIdx.x * 1e-3f + (float)k;
    // the multiplier and addend in VGPRs: an SGPR operand keeps the SIMD from
    // issuing two of these instructions in one slot
    asm volatile("" : "+v"(a), "+v"(b));
    const long long c0 = clock64(), w0 = wall_clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k) r[k] = __builtin_fmaf(r[k], a, b);
#pragma unroll
        for (int k = 0; k < 8; ++k) r[k] = __builtin_fmaf(r[k], a, b);
    }
    const long long c1 = clock64(), w1 = wall_clock64();
    float t = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) t += r[k];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = t;
    if ((threadIdx.x & 63) == 0) {
        const size_t wv = (size_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
        ticks[2 * wv] = c1 - c0;
        ticks[2 * wv + 1] = w1 - w0;
    }
}

// One VALU instruction class, 16 per loop trip over eight registers (the
// classes the KVarN kernels use most): the per-class issue rate.  Values are
// meaningless; only the timing is used.
#define KVARN_X8(INSN)                                                                          \
    asm volatile(INSN(0) INSN(1) INSN(2) INSN(3) INSN(4) INSN(5) INSN(6) INSN(7)               \
                 INSN(0) INSN(1) INSN(2) INSN(3) INSN(4) INSN(5) INSN(6) INSN(7)               \
                 : "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3), "+v"(r4), "+v"(r5), "+v"(r6),       \
                   "+v"(r7)                                                                     \
                 : "v"(a), "v"(b), "s"(sa))
#define I_FMA(n) "v_fma_f32 %" #n ", %" #n ", %8, %9\n"
#define I_FMA_S(n) "v_fma_f32 %" #n ", %" #n ", %10, %9\n"
#define I_DPP(n) "s_nop 1\n v_fmac_f32_dpp %" #n ", %" #n ", %8 row_ror:8 row_mask:0xf bank_mask:0xf\n"
#define I_CVT(n) "v_cvt_pk_u8_f32 %" #n ", %8, 1, %" #n "\n"
#define I_ANDOR(n) "v_and_or_b32 %" #n ", %" #n ", %8, %9\n"
#define I_PKADD(n) "v_pk_add_f16 %" #n ", %" #n ", %8\n"
#define I_MIN(n) "v_min_f32 %" #n ", %" #n ", %8\n"
#define I_FMAMIX(n) "v_fma_mix_f32 %" #n ", %" #n ", %8, %9 op_sel_hi:[1,0,0]\n"

template <int CLS>
__global__ __launch_bounds__(256) void valu_class_kernel(float* __restrict__ out, int iters, float a,
                                                         float b, float sa) {
    float r0 = (float)threadIdx.x * 1e-3f + 1.0f, r1 = r0 + 1.0f, r2 = r0 + 2.0f, r3 = r0 + 3.0f;
    float r4 = r0 + 4.0f, r5 = r0 + 5.0f, r6 = r0 + 6.0f, r7 = r0 + 7.0f;
    for (int it = 0; it < iters; ++it) {
        if constexpr (CLS == 0) KVARN_X8(I_FMA);
        else if constexpr (CLS == 1) KVARN_X8(I_FMA_S);
        else if constexpr (CLS == 2) KVARN_X8(I_DPP);
        else if constexpr (CLS == 3) KVARN_X8(I_CVT);
        else if constexpr (CLS == 4) KVARN_X8(I_ANDOR);
        else if constexpr (CLS == 5) KVARN_X8(I_PKADD);
        else if constexpr (CLS == 6) KVARN_X8(I_MIN);
        else KVARN_X8(I_FMAMIX);
    }
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = r0 + r1 + r2 + r3 + r4 + r5 + r6 + r7;
}

}  // namespace

// Runs the vector-ALU reference: `blocks` workgroups of 256 threads (four
// waves), each lane issuing 16 * iters fp32 multiply-adds.  out holds
// blocks * 256 floats, ticks 2 * blocks * 4 int64 (per wave: shader-clock
// ticks, 100 MHz wall-clock ticks); device pointers.  Returns the hipError_t
// of the launch.
extern "C" int kvarn_valu_reference(void* out, void* ticks, int32_t blocks, int32_t iters,
                                    void* stream) {
    if (!out || !ticks || blocks <= 0 || iters < 0) return 1;
    hipLaunchKernelGGL(valu_fma_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<float*>(out),
                       static_cast<long long*>(ticks), iters, 0.999999f, 1e-6f);
    return (int)hipGetLastError();
}

// Instruction classes of kvarn_valu_class_reference, in `cls` order.
static const char* const kValuClassNames[] = {
    "v_fma_f32", "v_fma_f32 (SGPR operand)", "v_fmac_f32_dpp", "v_cvt_pk_u8_f32",
    "v_and_or_b32", "v_pk_add_f16", "v_min_f32", "v_fma_mix_f32"};

extern "C" int kvarn_valu_class_count() { return 8; }
extern "C" const char* kvarn_valu_class_name(int32_t cls) {
    return (cls >= 0 && cls < 8) ? kValuClassNames[cls] : "";
}

// Runs class `cls`: `blocks` workgroups of 256 threads, 16 * iters
// instructions per lane; out holds blocks * 256 floats.  Returns the
// hipError_t of the launch, 1 for bad arguments.
extern "C" int kvarn_valu_class_reference(int32_t cls, void* out, int32_t blocks, int32_t iters,
                                          void* stream) {
    if (!out || blocks <= 0 || iters < 0 || cls < 0 || cls >= 8) return 1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    float* o = static_cast<float*>(out);
    const dim3 g((unsigned)blocks), t(256);
    const float a = 1.0001f, b = 0.5f, sa = 0.999f;
    switch (cls) {
    case 0: hipLaunchKernelGGL(valu_class_kernel<0>, g, t, 0, st, o, iters, a, b, sa); break;
    case 1: hipLaunchKernelGGL(valu_class_kernel<1>, g, t, 0, st, o, iters, a, b, sa); break;
    case 2: hipLaunchKernelGGL(valu_class_kernel<2>, g, t, 0, st, o, iters, a, b, sa); break;
    case 3: hipLaunchKernelGGL(valu_class_kernel<3>, g, t, 0, st, o, iters, a, b, sa); break;
    case 4: hipLaunchKernelGGL(valu_class_kernel<4>, g, t, 0, st, o, iters, a, b, sa); break;
    case 5: hipLaunchKernelGGL(valu_class_kernel<5>, g, t, 0, st, o, iters, a, b, sa); break;
    case 6: hipLaunchKernelGGL(valu_class_kernel<6>, g, t, 0, st, o, iters, a, b, sa); break;
    default: hipLaunchKernelGGL(valu_class_kernel<7>, g, t, 0, st, o, iters, a, b, sa); break;
    }
    return (int)hipGetLastError();
}

// Streams `units` units through a grid of `blocks` workgroups of 256 threads
// (each takes units blockIdx, blockIdx + blocks, ...: a persistent grid when
// blocks < units, one unit per workgroup in address order when blocks ==
// units); with `unrolled` 1 (2: nontemporal stores), the tile-pair and
// single-tile mixes at head_dim 128 use the compile-time kernels (others fall
// back to the loop kernel); `unrolled` 3 / 4 run the dequantize mix phased, 4 / 8 units
// read before their writes.  src holds units * rq words, dst units * wq words, sink 256
// words; device pointers, 16-byte aligned.  Returns the hipError_t of the
// launch (0 on success).
extern "C" int kvarn_stream_reference(const void* src, void* dst, int64_t units, int32_t rq,
                                      int32_t wq, int32_t blocks, int32_t unrolled, void* sink,
                                      void* stream) {
    if (units <= 0) return 0;
    if (!src || (wq > 0 && !dst) || !sink || rq < 0 || wq < 0 || blocks <= 0) return 1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const uint4* s4 = static_cast<const uint4*>(src);
    uint4* d4 = static_cast<uint4*>(dst);
    uint32_t* k4 = static_cast<uint32_t*>(sink);
    const bool nt = unrolled == 2;
#define KVARN_FIXED(RQ_, WQ_)                                                                   \
    if (unrolled && rq == RQ_ && wq == WQ_) {                                                  \
        if (nt)                                                                                 \
            hipLaunchKernelGGL((stream_mix_fixed<RQ_, WQ_, true>), dim3((unsigned)blocks),      \
                               dim3(256), 0, st, s4, d4, units, k4);                            \
        else                                                                                    \
            hipLaunchKernelGGL((stream_mix_fixed<RQ_, WQ_, false>), dim3((unsigned)blocks),     \
                               dim3(256), 0, st, s4, d4, units, k4);                            \
        return (int)hipGetLastError();                                                          \
    }
    if (unrolled >= 3 && rq == 864 && wq == 4096) {
        if (unrolled == 3)
            hipLaunchKernelGGL((stream_mix_phased<864, 4096, 4>), dim3((unsigned)blocks), dim3(256),
                               0, st, s4, d4, units, k4);
        else
            hipLaunchKernelGGL((stream_mix_phased<864, 4096, 8>), dim3((unsigned)blocks), dim3(256),
                               0, st, s4, d4, units, k4);
        return (int)hipGetLastError();
    }
    if (unrolled >= 3) return 1;
    KVARN_FIXED(4096, 864)
    KVARN_FIXED(864, 4096)
    KVARN_FIXED(864, 0)
    KVARN_FIXED(4096, 0)
    KVARN_FIXED(0, 4096)
    KVARN_FIXED(2048, 432)
    KVARN_FIXED(432, 2048)
    KVARN_FIXED(432, 0)
    KVARN_FIXED(2048, 0)
    KVARN_FIXED(0, 2048)
#undef KVARN_FIXED
    hipLaunchKernelGGL(stream_mix_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4*>(src),
                       static_cast<uint4*>(dst), units, rq, wq, static_cast<uint32_t*>(sink));
    return (int)hipGetLastError();
}
