// Device helpers shared by the kernels that quantise to fp8 e4m3 with one
// fp32 scale per 128-element block (the landed tokens' rows, and stage2's
// silu(gate) * up rows): a block is held by 8 adjacent lanes, 16 values each.
//
// Bit-exactness: the definition is e4m3(x / s), s = amax / 448, with IEEE
// divisions.  Neither division is done on the fast path:
//  * s: s0 = amax * c with c = fl(1/448); the residual amax - 448 * s0 is exact
//    in fp32 (one fma), and s = fma(residual, c, s0) is the correctly rounded
//    quotient.  Checked exhaustively against the IEEE quotient for every fp32
//    mantissa of a binade (and exactly, in rational arithmetic, for every
//    bf16 amax); the result scales by powers of two, so it holds for every
//    amax >= 2^-100, where no intermediate is subnormal.  Smaller maxima take
//    the IEEE division.
//  * x / s is bracketed instead: r = 1/s to within a few 2^-24 (v_rcp_f32 and
//    one Newton step), r_hi = r * (1 + 2^-20) and r_lo = r * (1 - 2^-20)
//    satisfy r_lo <= 1/s <= r_hi, so x * r_lo <= x / s <= x * r_hi for x >= 0
//    (reversed for x < 0), and rounding to fp32 keeps that order.  The
//    hardware conversion (v_cvt_pk_fp8_f32: OCP e4m3, round to nearest even,
//    subnormal results included) is monotone, so when the codes of x * r_lo
//    and x * r_hi agree, the code of the IEEE quotient is the same one.  They
//    differ only when a rounding boundary of e4m3 lies in the 2^-19-wide
//    bracket (about one element in 5 * 10^4); a lane holding such an element
//    redoes its 16 values with the IEEE division.  Every |x * r_hi| is below
//    448 * (1 + 2^-19), far under the 464 rounding boundary, so no saturation
//    case arises.
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
// values is amax (the same in the block's 8 lanes): out[i] holds the codes of
// x[4i .. 4i+3], byte j = x[4i+j].  Returns the block's scale s = amax / 448
// (0 for an all-zero block, whose codes are 0).
__device__ __forceinline__ float encode_block16(const float (&xv)[16], float amax, uint32_t (&out)[4]) {
    const bool zero = amax == 0.0f;
    // maxima below 2^-100 (rare: the workloads never produce them) take the IEEE
    // divisions throughout
    const bool tiny = !(amax >= 0x1p-100f);
    float s;
    if (__builtin_expect(tiny, 0)) s = amax / 448.0f;
    else s = div448(amax);
    const float r0 = __builtin_amdgcn_rcpf(s);
    const float r = fmaf(r0, fmaf(-s, r0, 1.0f), r0);
    const float r_hi = __fmul_rn(r, 1.0f + 0x1p-20f), r_lo = __fmul_rn(r, 1.0f - 0x1p-20f);
    bool slow = tiny;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t hi = cvt4(__fmul_rn(xv[4 * i], r_hi), __fmul_rn(xv[4 * i + 1], r_hi),
                                 __fmul_rn(xv[4 * i + 2], r_hi), __fmul_rn(xv[4 * i + 3], r_hi));
        const uint32_t lo = cvt4(__fmul_rn(xv[4 * i], r_lo), __fmul_rn(xv[4 * i + 1], r_lo),
                                 __fmul_rn(xv[4 * i + 2], r_lo), __fmul_rn(xv[4 * i + 3], r_lo));
        slow |= hi != lo;
        out[i] = hi;
    }
    if (slow && !zero) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[i] = cvt4(xv[4 * i] / s, xv[4 * i + 1] / s, xv[4 * i + 2] / s, xv[4 * i + 3] / s);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = zero ? 0u : out[i];
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
