// kvarn_device.hpp -- device helpers shared by the gfx950 kernels.
//
// Register tile layout used by every kernel
// -----------------------------------------
// One workgroup owns one 128-token tile of K or V with D = 64, 128 or 256
// (padded) channels and 2*D threads.  Each lane holds TPL = 4 tokens x CPL =
// 16 channels in 64 VGPRs:
//     lane = tb * R + cb,   R = D / 16 lanes per token row-group,
//     tokens 4*tb .. 4*tb+3,  tb in [0, 32)
//     channel block cb (16 channels) of the row-group, cb in [0, R)
// Row-group reductions (over channels) stay inside R <= 16 lanes of one DPP
// row; column reductions (over tokens) go through LDS.
//
// Walsh-Hadamard transform along channels
// ---------------------------------------
// The rotation is the natural-order (Sylvester) Hadamard matrix, which
// factors as H_D = H_R (over channel blocks) (x) H_16 (inside a block).  The
// 16 in-lane channels take four ordinary butterfly stages.  The log2(R)
// cross-lane stages pair lanes with DPP patterns that exist on gfx9:
// quad_perm xor 1, quad_perm xor 2, row_half_mirror (xor 7 within 8 lanes)
// and row_ror:8 (xor 8 within 16 lanes).  Each cross-lane stage is one
// multiply-add per value, y = self + sign * partner, with sign = -1 on the
// lane that plays the "upper" half of the pair.  Over GF(2) the masks
// {1,2,7,8} form a basis M; with phi = M^-1, stage k's upper lanes are
// those with phi_k(lane) = 1.  The network then computes, on lane i, the
// Hadamard output of block nu(i) = (phi^T phi) i, up to the sign
// (-1)^<f, nu(i)> with f = xor of all masks.  Loading natural channel block
// i ^ f into lane i cancels that sign exactly, so:
//     lane cb loads input block  cb ^ kF   (natural channel order)
//     lane cb holds output block kNu[cb]   (Sylvester channel order)
// The same network is its own inverse up to the 1/D scale (the scaled
// Hadamard matrix is symmetric and involutory), so dequantisation uses the
// identical load/store relabelling.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvarn {

constexpr int TILE = 128;
constexpr int TPL = 4;   // tokens per lane
constexpr int CPL = 16;  // channels per lane

// DPP controls (gfx9 encoding)
constexpr int DPP_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_HMIR = 0x141;  // row_half_mirror: lane i <-> 7 - i within 8
constexpr int DPP_ROR8 = 0x128;  // row_ror:8: lane i <-> i ^ 8 within 16

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// ---- lane network constants, R = lanes per row-group ----------------------
template <int R> struct Net;
template <> struct Net<4> {
    static constexpr int kF = 3;
    __device__ static int nu(int i) { return i; }
    // upper-lane flag of each stage (xor1, xor2)
    __device__ static int up0(int i) { return i & 1; }
    __device__ static int up1(int i) { return (i >> 1) & 1; }
};
template <> struct Net<8> {
    static constexpr int kF = 4;
    __device__ static int nu(int i) {
        int b0 = i & 1, b1 = (i >> 1) & 1, b2 = (i >> 2) & 1;
        return (b0 ^ b2) | ((b1 ^ b2) << 1) | ((b0 ^ b1 ^ b2) << 2);
    }
    __device__ static int up0(int i) { return (i ^ (i >> 2)) & 1; }         // xor1
    __device__ static int up1(int i) { return ((i >> 1) ^ (i >> 2)) & 1; }  // xor2
    __device__ static int up2(int i) { return (i >> 2) & 1; }               // half mirror
};
template <> struct Net<16> {
    static constexpr int kF = 12;
    __device__ static int nu(int i) { return Net<8>::nu(i & 7) | (i & 8); }
    __device__ static int up0(int i) { return Net<8>::up0(i & 7); }
    __device__ static int up1(int i) { return Net<8>::up1(i & 7); }
    __device__ static int up2(int i) { return Net<8>::up2(i & 7); }
    __device__ static int up3(int i) { return (i >> 3) & 1; }               // ror 8
};

__device__ __forceinline__ float sign_of(int upper) { return upper ? -1.0f : 1.0f; }

// Ordinary butterflies over the 16 in-lane channels of every token, from
// the stage of span H0 on (H0 = 2 when the loads already did the first).
template <int H0 = 1>
__device__ __forceinline__ void fwht_inlane(float (&x)[TPL][CPL]) {
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
#pragma unroll
        for (int h = H0; h < CPL; h <<= 1) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                if ((c & h) == 0) {
                    float a = x[i][c], b = x[i][c + h];
                    x[i][c] = a + b;
                    x[i][c + h] = a - b;
                }
            }
        }
    }
}

template <int CTRL>
__device__ __forceinline__ void xstage(float (&x)[TPL][CPL], float sg) {
#pragma unroll
    for (int i = 0; i < TPL; ++i)
#pragma unroll
        for (int c = 0; c < CPL; ++c) x[i][c] = __builtin_fmaf(dpp<CTRL>(x[i][c]), sg, x[i][c]);
}

// One cross-lane stage as single instructions: v_fmac_f32 with a DPP source
// computes x += sign * x(partner lane) in place.  The compiler does not form
// this DPP multiply-add from the builtins, so it is written out; the leading
// s_nop 1 gives the two wait states a DPP read needs after a VALU write of
// the same VGPR (inside a block every instruction reads a different VGPR,
// written by the previous stage).
#define KVARN_FMAC_DPP_BLOCK(CTRL)                                                              \
    asm volatile("s_nop 1\n"                                                                   \
                 "v_fmac_f32_dpp %0, %0, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"            \
                 "v_fmac_f32_dpp %1, %1, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"            \
                 "v_fmac_f32_dpp %2, %2, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"            \
                 "v_fmac_f32_dpp %3, %3, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"            \
                 "v_fmac_f32_dpp %4, %4, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"            \
                 "v_fmac_f32_dpp %5, %5, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"            \
                 "v_fmac_f32_dpp %6, %6, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"            \
                 "v_fmac_f32_dpp %7, %7, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"            \
                 "v_fmac_f32_dpp %8, %8, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"            \
                 "v_fmac_f32_dpp %9, %9, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"            \
                 "v_fmac_f32_dpp %10, %10, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"          \
                 "v_fmac_f32_dpp %11, %11, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"          \
                 "v_fmac_f32_dpp %12, %12, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"          \
                 "v_fmac_f32_dpp %13, %13, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"          \
                 "v_fmac_f32_dpp %14, %14, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"          \
                 "v_fmac_f32_dpp %15, %15, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"          \
                 : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]),     \
                   "+v"(r[6]), "+v"(r[7]), "+v"(r[8]), "+v"(r[9]), "+v"(r[10]), "+v"(r[11]),   \
                   "+v"(r[12]), "+v"(r[13]), "+v"(r[14]), "+v"(r[15])                           \
                 : "v"(sg))

template <int CTRL>
__device__ __forceinline__ void xstage_fmac(float (&r)[CPL], float sg) {
    if constexpr (CTRL == DPP_XOR1) KVARN_FMAC_DPP_BLOCK("quad_perm:[1,0,3,2]");
    else if constexpr (CTRL == DPP_XOR2) KVARN_FMAC_DPP_BLOCK("quad_perm:[2,3,0,1]");
    else if constexpr (CTRL == DPP_HMIR) KVARN_FMAC_DPP_BLOCK("row_half_mirror");
    else KVARN_FMAC_DPP_BLOCK("row_ror:8");
}

// Cross-lane stages; cb = lane position in its row-group.
template <int R>
__device__ __forceinline__ void fwht_crosslane(float (&x)[TPL][CPL], int cb) {
    using N = Net<R>;
    const float s0 = sign_of(N::up0(cb)), s1 = sign_of(N::up1(cb));
#pragma unroll
    for (int i = 0; i < TPL; ++i) xstage_fmac<DPP_XOR1>(x[i], s0);
#pragma unroll
    for (int i = 0; i < TPL; ++i) xstage_fmac<DPP_XOR2>(x[i], s1);
    if constexpr (R >= 8) {
        const float s2 = sign_of(N::up2(cb));
#pragma unroll
        for (int i = 0; i < TPL; ++i) xstage_fmac<DPP_HMIR>(x[i], s2);
    }
    if constexpr (R >= 16) {
        const float s3 = sign_of(N::up3(cb));
#pragma unroll
        for (int i = 0; i < TPL; ++i) xstage_fmac<DPP_ROR8>(x[i], s3);
    }
}

// All-reduce across the R lanes of a row-group (every lane gets the result;
// each pairwise step is commutative, so all lanes hold identical bits).
template <int R>
__device__ __forceinline__ float rg_sum(float v) {
    v += dpp<DPP_XOR1>(v);
    v += dpp<DPP_XOR2>(v);
    if constexpr (R >= 8) v += dpp<DPP_HMIR>(v);
    if constexpr (R >= 16) v += dpp<DPP_ROR8>(v);
    return v;
}
template <int R>
__device__ __forceinline__ float rg_min(float v) {
    v = fminf(v, dpp<DPP_XOR1>(v));
    v = fminf(v, dpp<DPP_XOR2>(v));
    if constexpr (R >= 8) v = fminf(v, dpp<DPP_HMIR>(v));
    if constexpr (R >= 16) v = fminf(v, dpp<DPP_ROR8>(v));
    return v;
}
template <int R>
__device__ __forceinline__ float rg_max(float v) {
    v = fmaxf(v, dpp<DPP_XOR1>(v));
    v = fmaxf(v, dpp<DPP_XOR2>(v));
    if constexpr (R >= 8) v = fmaxf(v, dpp<DPP_HMIR>(v));
    if constexpr (R >= 16) v = fmaxf(v, dpp<DPP_ROR8>(v));
    return v;
}

// First butterfly straight from a packed pair of fp16 values (lo, hi):
// s = lo + hi, d = lo - hi, each with one fp32 rounding of the exact result
// (the mixed-precision multiply-add widens both halves exactly), the same
// values as widening first and adding in fp32.
__device__ __forceinline__ void h2_butterfly(uint32_t w, float& s, float& d) {
    asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(s) : "v"(w));
    asm("v_fma_mix_f32 %0, -%1, 1.0, %1 op_sel:[1,0,0] op_sel_hi:[1,0,1]" : "=v"(d) : "v"(w));
}

// Min / max across the R lanes of a row-group for four values at once, one
// DPP instruction per value and stage (the s_nop gives the DPP read its two
// wait states after the VALU write of the same VGPRs).  Inputs are results
// of arithmetic, never signalling NaNs, so the plain min/max is exact.
#define KVARN_DPP4(OP, CTRL)                                              \
    asm volatile("s_nop 1\n"                                             \
                 OP "_dpp %0, %0, %0 " CTRL " row_mask:0xf bank_mask:0xf\n" \
                 OP "_dpp %1, %1, %1 " CTRL " row_mask:0xf bank_mask:0xf\n" \
                 OP "_dpp %2, %2, %2 " CTRL " row_mask:0xf bank_mask:0xf\n" \
                 OP "_dpp %3, %3, %3 " CTRL " row_mask:0xf bank_mask:0xf\n" \
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]))

template <int R, bool MAX>
__device__ __forceinline__ void rg_minmax4(float (&v)[4]) {
    if constexpr (MAX) {
        KVARN_DPP4("v_max_f32", "quad_perm:[1,0,3,2]");
        KVARN_DPP4("v_max_f32", "quad_perm:[2,3,0,1]");
        if constexpr (R >= 8) KVARN_DPP4("v_max_f32", "row_half_mirror");
        if constexpr (R >= 16) KVARN_DPP4("v_max_f32", "row_ror:8");
    } else {
        KVARN_DPP4("v_min_f32", "quad_perm:[1,0,3,2]");
        KVARN_DPP4("v_min_f32", "quad_perm:[2,3,0,1]");
        if constexpr (R >= 8) KVARN_DPP4("v_min_f32", "row_half_mirror");
        if constexpr (R >= 16) KVARN_DPP4("v_min_f32", "row_ror:8");
    }
}

// Three-way min / max of values that are results of arithmetic (never
// signalling NaNs): written out so that no canonicalising operation is
// inserted for operands that come from LDS.
__device__ __forceinline__ float min3f(float a, float b, float c) {
    float r;
    asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Flat-group test of the normalisation in fp32: a spread below 2^-16 of the
// group mean cannot be told apart from a constant group.
__device__ __forceinline__ bool is_flat(float sd, float mean) {
    return sd <= 1.52587890625e-05f * fabsf(mean);
}

__device__ __forceinline__ uint16_t f2h_bits(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}
__device__ __forceinline__ float h2f_bits(uint16_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// value of lane L (wave-uniform result)
__device__ __forceinline__ float lane_f(float v, int L) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), L));
}

// Orders the LDS accesses of one wavefront: what its lanes wrote before is
// visible to its lanes after (no workgroup barrier).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D> constexpr int padded_ok() { return D == 64 || D == 128 || D == 256; }

}  // namespace kvarn
