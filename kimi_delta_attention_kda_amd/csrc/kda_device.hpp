// kda_device.hpp -- small device helpers shared by the KDA kernels (gfx950).
//
// Pages cited by title and section:
//   [SGL-PR]  "SGLang PR #26586 (KDA packed decode)" -- gate, beta and
//             L2-norm formulas of the fused decode kernel snippet.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

constexpr float kLog2e = 1.4426950408889634f;

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16);
}

// float -> bf16 bit pattern, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Two floats -> packed bf16 pair (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 v;
    v[0] = static_cast<__bf16>(a);
    v[1] = static_cast<__bf16>(b);
    return __builtin_bit_cast(uint32_t, v);
}

// softplus(x) = log(1 + e^x), switching to x above a threshold of 20, where
// the two differ by less than e^-20 relative.  [SGL-PR] uses a threshold whose
// value the page does not print; 20 is the usual choice.
__device__ __forceinline__ float softplus_f(float x) {
    return x > 20.0f ? x : log1pf(expf(x));
}

__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + expf(-x)); }

// e^{-A softplus(z)}, the per-channel decay of the decode gate, written as
// 2^{-A log2(1 + 2^{z log2 e})} so that it costs two hardware transcendentals
// (v_exp_f32, v_log_f32) and no branch; above z = 20 softplus(z) is taken as z
// as in softplus_f.  For z far below zero 1 + e^z rounds to 1 and the decay
// to 1, an absolute error below 2^-24 A in the exponent.
__device__ __forceinline__ float gate_decay(float z, float A) {
    const float l2 = z > 20.0f ? z * kLog2e : __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(z * kLog2e));
    return __builtin_amdgcn_exp2f(-A * l2);
}

// DPP move of x from another lane (CTRL = dpp_ctrl; lanes whose source is
// outside the 16-lane row read 0).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF,
                                                                 false));
}

// Sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15), in VALU: quad
// butterflies, then the mirrored half row, then the mirrored row.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp_f<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp_f<0x141>(x);   // row_half_mirror
    x += dpp_f<0x140>(x);   // row_mirror
    return x;
}

}  // namespace kda
