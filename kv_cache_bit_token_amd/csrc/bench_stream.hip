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
// at head_dim 128.
template <int RQ, int WQ>
__global__ __launch_bounds__(256) void stream_mix_fixed(const uint4* __restrict__ src,
                                                        uint4* __restrict__ dst, int64_t units,
                                                        uint32_t* sink) {
    constexpr int RL = (RQ + 255) / 256, WL = (WQ + 255) / 256;
    uint4 acc = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        const uint4* s = src + u * RQ;
        uint4 v[RL];
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
                if (i < WQ) d[i] = make_uint4(acc.x ^ (uint32_t)i, acc.y, acc.z, acc.w);
            }
        }
    }
    if (WQ == 0 && (acc.x & acc.y & acc.z & acc.w) == 0xFFFFFFFFu) sink[threadIdx.x] = acc.x;
}

}  // namespace

// Streams `units` units through a persistent grid of `blocks` workgroups of
// 256 threads; with `unrolled` set, the tile-pair mixes at head_dim 128 use
// the compile-time kernels (others fall back to the loop kernel).  src holds units * rq words, dst units * wq words, sink 256
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
    if (unrolled && rq == 4096 && wq == 864) {
        hipLaunchKernelGGL((stream_mix_fixed<4096, 864>), dim3((unsigned)blocks), dim3(256), 0, st, s4, d4, units, k4);
        return (int)hipGetLastError();
    }
    if (unrolled && rq == 864 && wq == 4096) {
        hipLaunchKernelGGL((stream_mix_fixed<864, 4096>), dim3((unsigned)blocks), dim3(256), 0, st, s4, d4, units, k4);
        return (int)hipGetLastError();
    }
    if (unrolled && rq == 864 && wq == 0) {
        hipLaunchKernelGGL((stream_mix_fixed<864, 0>), dim3((unsigned)blocks), dim3(256), 0, st, s4, d4, units, k4);
        return (int)hipGetLastError();
    }
    if (unrolled && rq == 4096 && wq == 0) {
        hipLaunchKernelGGL((stream_mix_fixed<4096, 0>), dim3((unsigned)blocks), dim3(256), 0, st, s4, d4, units, k4);
        return (int)hipGetLastError();
    }
    hipLaunchKernelGGL(stream_mix_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4*>(src),
                       static_cast<uint4*>(dst), units, rq, wq, static_cast<uint32_t*>(sink));
    return (int)hipGetLastError();
}
