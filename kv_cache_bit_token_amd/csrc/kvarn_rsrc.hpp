// kvarn_rsrc.hpp -- raw buffer descriptors for the attention kernels, gfx950.
//
// A descriptor covers one wave-uniform byte range (base and size in scalar
// registers); loads through it take a per-lane byte offset and a scalar
// offset.  Only the per-lane offset (plus the instruction's immediate) is
// checked against the range: a lane whose offset lies at or past the end
// reads zero without touching memory, while the scalar offset is added
// unchecked.  So a kernel may move the scalar offset only inside a range it
// knows is whole (a full tile); where rows can run past the end, the row
// offset goes into the per-lane part or the descriptor's base moves.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvarn {

// Word 3 of a raw buffer descriptor on gfx9-family parts (32-bit data
// format, no swizzle): byte offsets are checked against num_records.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// Cache-policy bits of a buffer access (gfx940-family encoding): NT marks
// data that is streamed through once, so it is not kept in the caches.
constexpr int kPolicyNT = 2;

template <int POL = 0>
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POL));
}
template <int POL = 0>
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, POL));
}
template <int POL = 0>
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, POL));
}

}  // namespace kvarn
