// Device helpers shared by the kernels that quantise to fp8 e4m3 with one
// fp32 scale per 128-element block (the landed tokens' rows, and stage2's
// silu(gate) * up rows): a block is held by 8 adjacent lanes, 16 values each.
//
// Bit-exactness: the definition is e4m3(fl32(x / s)), s = fl32(amax / 448),
// IEEE divisions, round to nearest even.  Neither division is done on the
// fast path:
//  * s: s0 = amax * c with c = fl(1/448); the residual amax - 448 * s0 is exact
//    in fp32 (one fma), and s = fma(residual, c, s0) is the correctly rounded
//    quotient.  Checked exhaustively against the IEEE quotient for every fp32
//    mantissa of a binade (and exactly, in rational arithmetic, for every
//    bf16 amax); the result scales by powers of two, so it holds for every
//    amax >= 2^-100, where no intermediate is subnormal.  Smaller, infinite
//    and NaN maxima take the IEEE divisions.
//  * fl32(x / s) is computed as fl32(fl64(x * R)), R ~ 1/s in fp64: r = v_rcp_f32
//    with one fp32 Newton step (relative error about 2^-23), then two fp64
//    Newton steps, leaving |R s - 1| below about 2^-52, so fl64(x * R) is within
//    2^-51 (relative) of x / s.  That is close enough, for any fp32 x, where
//    the quotient is a normal fp32 number: a rounding midpoint M there has a
//    25-bit odd significand m1 and s a 24-bit one m2, so x = M s would make m1
//    divide x's significand, which is impossible, and near equality x - M s is
//    a nonzero multiple of the last bit of M s (x's exponent must be at least
//    22 above it for the magnitudes to match), so |x/s - M| >= 2^-49 |M|.  x / s
//    and its fp64 approximation therefore lie on the same side of every such
//    midpoint and round to the same fp32 value.  Quotients below 2^-126 may
//    differ from the IEEE one in their last place, but every magnitude below
//    2^-10 encodes to a zero of x's sign, so the codes agree.  The hardware
//    conversion (v_cvt_pk_fp8_f32: OCP e4m3, round to nearest even, subnormal
//    results included) then gives the code.  |fl32(x / s)| <= 448 (1 + 2^-22),
//    far under the 464 rounding boundary, so no saturation case arises.
//    Inputs with few significant bits (bf16 activations) put x / s within
//    2^-19 of an e4m3 midpoint for about one element in 200, so a cheaper
//    fp32 bracket with an IEEE fallback would take the fallback in nine passes
//    of ten.
#pragma once

#include "common.h"

namespace moe {

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

// four e4m3 codes of (a, b, c, d), hardware round to nearest even
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
    return (uint32_t)v;
}

// s = amax / 448 rounded to nearest even, for amax >= 2^-100 (see above)
__device__ __forceinline__ float div448(float amax) {
    constexpr float c = 0x1.24924ap-9f;                  // fl(1/448)
    const float s0 = __fmul_rn(amax, c);
    const float rem = fmaf(-s0, 448.0f, amax);           // exact
    return fmaf(rem, c, s0);
}

// Codes of this lane's 16 values of a block whose |max| over all its 128
// values is amax (the same in the block's 8 lanes; a magnitude, never -0):
// out[i] holds the codes of x[4i .. 4i+3], byte j = x[4i+j].  Returns the
// block's scale s = amax / 448 (+0 for an all-zero block, whose codes are 0).
__device__ __forceinline__ float encode_block16(const float (&xv)[16], float amax, uint32_t (&out)[4]) {
    // maxima below 2^-100 (rare: the workloads never produce them), zero,
    // infinity and NaN take the IEEE divisions
    if (__builtin_expect(!(amax >= 0x1p-100f && amax <= 0x1.fffffep127f), 0)) {
        const float s = amax / 448.0f;
        const bool zero = amax == 0.0f;                 // codes 0 (x / 0 would give NaN)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[i] = zero ? 0u : cvt4(xv[4 * i] / s, xv[4 * i + 1] / s, xv[4 * i + 2] / s, xv[4 * i + 3] / s);
        return s;
    }
    const float s = div448(amax);
    const float r0 = __builtin_amdgcn_rcpf(s);
    const float r = fmaf(r0, fmaf(-s, r0, 1.0f), r0);
    const double sd = (double)s;
    double R = (double)r;
    R = fma(R, fma(-sd, R, 1.0), R);
    R = fma(R, fma(-sd, R, 1.0), R);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        out[i] = cvt4((float)((double)xv[4 * i] * R), (float)((double)xv[4 * i + 1] * R),
                      (float)((double)xv[4 * i + 2] * R), (float)((double)xv[4 * i + 3] * R));
    return s;
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
