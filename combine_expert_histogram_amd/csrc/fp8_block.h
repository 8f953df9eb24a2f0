// Device helpers shared by the kernels that quantise to fp8 e4m3 with one
// fp32 scale per 128-element block (the landed tokens' rows, and stage2's
// silu(gate) * up rows): a block is held by 8 adjacent lanes, 16 values each.
//
// Bit-exactness: the definition is e4m3(x / s), s = amax / 448, with IEEE
// divisions.  encode_block16 computes w = x * (1/s) (both roundings to
// nearest) and encodes w with the hardware conversion (v_cvt_pk_fp8_f32: OCP
// e4m3, round to nearest even; every |w| here is below the 464 rounding
// boundary, so no saturation case arises), unless w lies within 8 fp32 ulps
// of an e4m3 rounding tie, or in the e4m3 subnormal range (|w| < 2^-6,
// nonzero): such elements (rare; the lane takes one divergent branch) redo the
// IEEE division x / s.  Bound: 1/s and the product each carry <= 2^-24
// relative error, so |w - x/s| <= 2 ulp(x/s), and the correctly rounded
// quotient is within 0.5 ulp of x/s, so outside the window both round to the
// same code.
#pragma once

#include "common.h"

namespace moe {

constexpr uint32_t kE4m3MinNormalBits = 0x3C800000u;   // 2^-6, smallest e4m3 normal

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// max of the 8 lanes l..l|7 (aligned groups of 8): quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], then row_half_mirror joins the two quads.
__device__ __forceinline__ uint32_t group8_max(uint32_t v) {
    v = max(v, dpp<0xB1>(v));
    v = max(v, dpp<0x4E>(v));
    v = max(v, dpp<0x141>(v));
    return v;
}

// True when w might round differently from the IEEE quotient: within 8 ulps
// of an e4m3 rounding tie in the normal range, or a nonzero e4m3 subnormal.
__device__ __forceinline__ bool needs_exact(float w) {
    const uint32_t ab = __float_as_uint(w) & 0x7FFFFFFFu;
    const bool tie = ((ab & 0xFFFFFu) - 0x7FFF8u) < 16u;
    const bool sub = (ab - 1u) < (kE4m3MinNormalBits - 1u);
    return tie | sub;
}

// four e4m3 codes of (a, b, c, d), hardware round to nearest even
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
    return (uint32_t)v;
}

// Codes of this lane's 16 values of a block whose |max| over all its 128
// values is amax (the same in the block's 8 lanes): out[i] holds the codes of
// x[4i .. 4i+3], byte j = x[4i+j].  Returns the block's scale s = amax / 448
// (0 for an all-zero block, whose codes are 0).
__device__ __forceinline__ float encode_block16(const float (&xv)[16], float amax, uint32_t (&out)[4]) {
    const float s = amax / 448.0f;
    const float r = 1.0f / s;
    const bool zero = amax == 0.0f;
    // a scale too small for 1/s to be finite takes the exact division throughout
    const bool all_exact = !(r <= 3.0e38f);
    float w[16];
    bool slow = all_exact;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        w[i] = __fmul_rn(xv[i], r);
        slow |= needs_exact(w[i]);
    }
    if (slow) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (all_exact || needs_exact(w[i])) w[i] = xv[i] / s;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        out[i] = zero ? 0u : cvt4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
    return zero ? 0.0f : s;
}

// MX (e8m0) group exponent: E = ceil(log2(t)), t = amax / 448 (IEEE fp32
// division), read off t's bits (an exact power of two keeps its exponent,
// anything above it rounds up), clamped to [-127, 127]; an all-zero group
// (amax == 0) gives -127.  For finite amax, E <= 120, so 2^-E is a normal float.
__device__ __forceinline__ int mx_exponent(float amax) {
    if (!(amax > 0.0f)) return -127;
    const uint32_t b = __float_as_uint(amax / 448.0f);
    const int ex = (int)((b >> 23) & 0xFF);
    const uint32_t man = b & 0x7FFFFFu;
    int E;
    if (ex == 0) E = man > 0x400000u ? -126 : -127;     // subnormal t: (2^-127, 2^-126) or below
    else E = ex - 127 + (man != 0 ? 1 : 0);
    return max(-127, min(127, E));
}

// 2^-E as a float (E in [-127, 120])
__device__ __forceinline__ float exp2_neg(int E) { return __uint_as_float((uint32_t)(127 - E) << 23); }

}  // namespace moe
