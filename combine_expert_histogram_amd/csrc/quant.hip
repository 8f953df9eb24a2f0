// Step 2: quant + dispatch - each landed token's bf16 row is read once and
// quantised once into its compact slot as fp8 e4m3 with one fp32 scale per
// 128-element block ("poc(cco): MegaMoE stage1 dispatch over SDMA", commit
// "each token read and quantised once"; "How it works now": every lane stores
// one contiguous 16 B, 1 KiB per wavefront store instruction).
//
// Mapping: one wavefront per slot row; a pass covers 1024 hidden elements =
// 8 blocks of 128; lane l takes 16 consecutive elements (two 16 B loads) of
// block l/8, so a block is 8 adjacent lanes and its |max| is three DPP steps.
// Because slot rows are dense and row-major, lane l's 16 codes land in bytes
// [16l, 16l+16) of the pass: the wavefront's store is one contiguous 1 KiB
// without an LDS round trip (the pages needed an LDS swizzle for that because
// their send buffer interleaved payload and scales).
//
// Bit-exactness: the definition is e4m3(x / s) with an IEEE division.  The
// kernel computes w = x * (1/s) (both roundings to nearest) and uses it
// whenever w is not within a few fp32 ulps of an e4m3 rounding tie: then x/s
// and w round to the same code.  The rare near-tie elements redo the IEEE
// division.  Bound: 1/s and the product each carry <= 2^-24 relative error,
// so |w - x/s| <= 2 ulp(x/s); the correctly rounded quotient is within 0.5 ulp
// of x/s; the test window is +-8 ulp (normal range) or 2^-16 of the 2^-9 code
// spacing (subnormal range, where the error is < 2^-19 of it).
#include "common.h"

namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / MOE_WAVE;
constexpr uint32_t kMinNormalBits = 0x3C800000u;   // 2^-6, smallest e4m3 normal

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// |max| of the 8 lanes l..l|7 (aligned groups of 8): quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], then row_half_mirror joins the two quads.
__device__ __forceinline__ uint32_t group8_max(uint32_t v) {
    v = max(v, dpp<0xB1>(v));
    v = max(v, dpp<0x4E>(v));
    v = max(v, dpp<0x141>(v));
    return v;
}

// OCP e4m3 code of a finite fp32 value, round to nearest even, saturate at 448.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const uint32_t b = __float_as_uint(v);
    const uint32_t ab = b & 0x7FFFFFFFu;
    const uint32_t sgn = (b >> 24) & 0x80u;
    // normal range: drop 20 mantissa bits with round-to-nearest-even, rebias 127 -> 7
    const uint32_t rb = ab + 0x7FFFFu + ((ab >> 20) & 1u);
    const uint32_t cn = min((rb >> 20) - (120u << 3), 0x7Eu);
    // subnormal range: multiples of 2^-9 (a count of 8 is the smallest normal)
    const uint32_t cs = (uint32_t)rintf(__uint_as_float(ab) * 512.0f);
    return (ab >= kMinNormalBits ? cn : cs) | sgn;
}

// True when v is close enough to an e4m3 rounding tie that an approximate
// quotient might round differently from the IEEE quotient.
__device__ __forceinline__ bool near_tie(float v) {
    const uint32_t ab = __float_as_uint(v) & 0x7FFFFFFFu;
    const bool nn = ((ab & 0xFFFFFu) - 0x7FFF8u) < 16u;
    const float t = __uint_as_float(ab) * 512.0f;
    const bool ns = fabsf(t - floorf(t) - 0.5f) < 1.52587890625e-05f;   // 2^-16
    return ab >= kMinNormalBits ? nn : ns;
}

__device__ __forceinline__ uint32_t quant_pair(uint32_t word, float r, float s, bool exact) {
    float x0 = moe::bf16_lo(word), x1 = moe::bf16_hi(word);
    float w0 = __fmul_rn(x0, r), w1 = __fmul_rn(x1, r);
    if (exact || near_tie(w0)) w0 = x0 / s;
    if (exact || near_tie(w1)) w1 = x1 / s;
    return e4m3_code(w0) | (e4m3_code(w1) << 8);
}

__global__ void __launch_bounds__(kBlock)
quant_dispatch_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ slot_tok,
                      const int32_t* __restrict__ totals, int64_t T, int H,
                      uint8_t* __restrict__ q, float* __restrict__ q_scale) {
    const int64_t U = min((int64_t)totals[1], T);     // slots_cap = T
    const int lane = threadIdx.x % MOE_WAVE;
    const int sub = lane & 7;                    // 16-element piece within a block
    const int nblk = H / 128;
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    for (int64_t u = (int64_t)blockIdx.x * kWaves + threadIdx.x / MOE_WAVE; u < U; u += nwaves) {
        const int g = slot_tok[u];
        if ((uint64_t)g >= (uint64_t)T) continue;           // cannot come from the layout
        const moe::u32x4* src = reinterpret_cast<const moe::u32x4*>(x + (int64_t)g * H);
        moe::u32x4* dst = reinterpret_cast<moe::u32x4*>(q + u * H);
        float* sdst = q_scale + u * nblk;
#pragma unroll 2
        for (int cb = 0; cb < nblk; cb += 8) {
            const int blk = cb + (lane >> 3);
            const bool act = blk < nblk;
            moe::u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = v0;
            if (act) {
                v0 = __builtin_nontemporal_load(src + blk * 16 + sub * 2);
                v1 = __builtin_nontemporal_load(src + blk * 16 + sub * 2 + 1);
            }
            const uint32_t wv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            uint32_t m = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) m = max(m, max(wv[i] & 0x7FFFu, (wv[i] >> 16) & 0x7FFFu));
            m = group8_max(m);
            const float amax = __uint_as_float(m << 16);
            const float s = amax / 448.0f;
            const float r = 1.0f / s;
            // a zero block stores zeros; a scale too small for 1/s to be finite
            // takes the exact division for every element
            const bool zero = m == 0;
            const bool exact = !(r <= 3.0e38f);
            uint32_t out[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = quant_pair(wv[2 * i], r, s, exact);
                const uint32_t hi = quant_pair(wv[2 * i + 1], r, s, exact);
                out[i] = zero ? 0u : (lo | (hi << 16));
            }
            if (act) {
                dst[blk * 8 + sub] = moe::u32x4{out[0], out[1], out[2], out[3]};
                if (sub == 0) sdst[blk] = zero ? 0.0f : s;
            }
        }
    }
}

}  // namespace

extern "C" moe_status moe_quant_dispatch(const moe_dims* dims, const uint16_t* x_bf16,
                                         const int32_t* slot_tok, const int32_t* totals,
                                         uint8_t* q_e4m3, float* q_scale, void* hip_stream) {
    moe::Dims d;
    moe_status st = moe::load_dims(dims, &d, true);
    if (st != MOE_OK) return st;
    if (d.T == 0) return MOE_OK;
    if (!x_bf16 || !slot_tok || !totals || !q_e4m3 || !q_scale) return MOE_ERR_INVALID_ARG;
    if (d.T * d.H >= ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
    const int64_t waves = d.T;                                   // one per slot (slots_cap = T)
    const int grid = (int)std::min<int64_t>((waves + kWaves - 1) / kWaves, 16384);
    hipLaunchKernelGGL(quant_dispatch_kernel, dim3(grid), dim3(kBlock), 0,
                       reinterpret_cast<hipStream_t>(hip_stream), x_bf16, slot_tok, totals, d.T,
                       (int)d.H, q_e4m3, q_scale);
    return moe::launch_status();
}
