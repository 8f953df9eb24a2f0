// Step 2: quant + dispatch - each landed token's bf16 row is read once and
// quantised once into its compact slot as fp8 e4m3 with one fp32 scale per
// 128-element block ("poc(cco): MegaMoE stage1 dispatch over SDMA", commit
// "each token read and quantised once"; "How it works now": every lane stores
// one contiguous 16 B, 1 KiB per wavefront store instruction).
//
// Mapping: one wavefront per quarter slot row (four work items per row, so the
// last round of work items is not left mostly empty); a pass covers 1024
// hidden elements = 8 blocks of 128; lane l takes 16 consecutive elements (two
// 16 B loads) of block l/8, so a block is 8 adjacent lanes and its |max| is
// three DPP steps.  The loads run two passes ahead of the arithmetic.  The
// activation rows are read with ordinary loads and the codes
// written with non-temporal stores (measured best of the four combinations).
// Because slot rows are dense and row-major, lane l's 16 codes land in bytes
// [16l, 16l+16) of the pass: the wavefront's store is one contiguous 1 KiB
// without an LDS round trip (the pages needed an LDS swizzle for that because
// their send buffer interleaved payload and scales).
//
// Bit-exactness of the fp32-scale codes at multiply cost: fp8_block.h.
#include "fp8_block.h"

namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / MOE_WAVE;
// pieces per slot row (whole 8-block passes; at H = 7168: 2, 2, 2 and 1
// passes), and passes of loads in flight ahead of the arithmetic.  Four pieces
// with both passes' loads issued up front measured fastest (45.2 against 47.9
// us cold, and 38.9 against 38.1 warm, for two pieces with one pass ahead;
// whole rows or deeper prefetch cost registers and occupancy and ran slower)
constexpr int kSplit = 4;
constexpr int kAhead = 2;
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

using moe::cvt4;
using moe::dpp;
using moe::group8_max;

__global__ void __launch_bounds__(kBlock)
quant_dispatch_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ slot_tok,
                      const int32_t* __restrict__ totals, int64_t T, int H,
                      uint8_t* __restrict__ q, float* __restrict__ q_scale) {
    MOE_TRACE_T0(tr0);
    const int64_t U = min((int64_t)totals[1], T);     // slots_cap = T
    const int lane = threadIdx.x % MOE_WAVE;
    const int sub = lane & 7;                    // 16-element piece within a block
    const int nblk = H / 128;
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    // work item = one of kSplit pieces of a slot row (pieces of whole 8-block passes)
    const int per = ((nblk + 8 * kSplit - 1) / (8 * kSplit)) * 8;
    for (int64_t it = (int64_t)blockIdx.x * kWaves + threadIdx.x / MOE_WAVE; it < U * kSplit; it += nwaves) {
        const int64_t u = it / kSplit;
        const int b0 = (int)(it - u * kSplit) * per;
        const int b1 = min(nblk, b0 + per);
        if (b0 >= b1) continue;
        const int g = slot_tok[u];
        if ((uint64_t)g >= (uint64_t)T) continue;           // cannot come from the layout
        const moe::u32x4* src = reinterpret_cast<const moe::u32x4*>(x + (int64_t)g * H);
        moe::u32x4* dst = reinterpret_cast<moe::u32x4*>(q + u * H);
        float* sdst = q_scale + u * nblk;
        // a pass's two loads per lane (addresses past the row's last block re-read
        // that block)
        auto load = [&](int cb, moe::u32x4& a, moe::u32x4& b) __attribute__((always_inline)) {
            const int blk = min(cb + (lane >> 3), b1 - 1);
            a = src[blk * 16 + sub * 2];
            b = src[blk * 16 + sub * 2 + 1];
        };
        // the loads of kAhead passes are in flight before the arithmetic (a work item
        // of two passes has all its loads issued up front)
        moe::u32x4 na[kAhead], nb[kAhead];
#pragma unroll
        for (int d = 0; d < kAhead; ++d)
            if (b0 + 8 * d < b1) load(b0 + 8 * d, na[d], nb[d]);
        for (int cb = b0; cb < b1; cb += 8) {
            const int blk = cb + (lane >> 3);
            const bool act = blk < b1;
            const moe::u32x4 v0 = na[0], v1 = nb[0];
#pragma unroll
            for (int d = 0; d + 1 < kAhead; ++d) {
                na[d] = na[d + 1];
                nb[d] = nb[d + 1];
            }
            if (cb + 8 * kAhead < b1) load(cb + 8 * kAhead, na[kAhead - 1], nb[kAhead - 1]);
            const uint32_t wv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            // |max| of the 16 bf16 values (packed 16-bit integer max of the magnitudes)
            u16x2 m2 = {0, 0};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t a = wv[i] & 0x7FFF7FFFu;
                m2 = __builtin_elementwise_max(m2, *reinterpret_cast<const u16x2*>(&a));
            }
            uint32_t m = max((uint32_t)m2.x, (uint32_t)m2.y);
            m = group8_max(m);
            float xv[16];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                xv[2 * i] = moe::bf16_lo(wv[i]);
                xv[2 * i + 1] = moe::bf16_hi(wv[i]);
            }
            uint32_t out[4];
            const float s = moe::encode_block16(xv, __uint_as_float(m << 16), out);
            if (act) {
                __builtin_nontemporal_store(moe::u32x4{out[0], out[1], out[2], out[3]}, dst + blk * 8 + sub);
                if (sub == 0) sdst[blk] = s;
            }
        }
    }
    if (threadIdx.x % MOE_WAVE == 0) MOE_TRACE_PUT(moe::kTrQuant, blockIdx.x * kWaves + threadIdx.x / MOE_WAVE, threadIdx.x / MOE_WAVE, 0, tr0);
}

// MX-style variant ("Where we stand": e8m0 block scales; commit
// "ready-first / quant-lds-store": packed four per dword): groups of 32
// elements, a group being one lane pair of the mapping above.  Per group:
// E = moe::mx_exponent(amax) (ceil(log2(amax / 448)), clamped; an all-zero
// group: -127); payload = e4m3(x * 2^-E), the scaling
// exact, so the hardware conversion's round to nearest even is the only
// rounding and no magnitude exceeds 448 (an all-zero group: zero bytes);
// code = E + 127, the four codes of a 128-element block packed into one dword
// (group g of the block in byte g).

__global__ void __launch_bounds__(kBlock)
quant_dispatch_mx_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ slot_tok,
                         const int32_t* __restrict__ totals, int64_t T, int H,
                         uint8_t* __restrict__ q, uint32_t* __restrict__ q_scale) {
    MOE_TRACE_T0(tr0);
    const int64_t U = min((int64_t)totals[1], T);
    const int lane = threadIdx.x % MOE_WAVE;
    const int sub = lane & 7;
    const int nblk = H / 128;
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    const int per = ((nblk + 8 * kSplit - 1) / (8 * kSplit)) * 8;
    for (int64_t it = (int64_t)blockIdx.x * kWaves + threadIdx.x / MOE_WAVE; it < U * kSplit; it += nwaves) {
        const int64_t u = it / kSplit;
        const int b0 = (int)(it - u * kSplit) * per;
        const int b1 = min(nblk, b0 + per);
        if (b0 >= b1) continue;
        const int g = slot_tok[u];
        if ((uint64_t)g >= (uint64_t)T) continue;
        const moe::u32x4* src = reinterpret_cast<const moe::u32x4*>(x + (int64_t)g * H);
        moe::u32x4* dst = reinterpret_cast<moe::u32x4*>(q + u * H);
        uint32_t* sdst = q_scale + u * nblk;
        auto load = [&](int cb, moe::u32x4& a, moe::u32x4& b) __attribute__((always_inline)) {
            const int blk = min(cb + (lane >> 3), b1 - 1);
            a = src[blk * 16 + sub * 2];
            b = src[blk * 16 + sub * 2 + 1];
        };
        // the loads of kAhead passes are in flight before the arithmetic (a work item
        // of two passes has all its loads issued up front)
        moe::u32x4 na[kAhead], nb[kAhead];
#pragma unroll
        for (int d = 0; d < kAhead; ++d)
            if (b0 + 8 * d < b1) load(b0 + 8 * d, na[d], nb[d]);
        for (int cb = b0; cb < b1; cb += 8) {
            const int blk = cb + (lane >> 3);
            const bool act = blk < b1;
            const moe::u32x4 v0 = na[0], v1 = nb[0];
#pragma unroll
            for (int d = 0; d + 1 < kAhead; ++d) {
                na[d] = na[d + 1];
                nb[d] = nb[d + 1];
            }
            if (cb + 8 * kAhead < b1) load(cb + 8 * kAhead, na[kAhead - 1], nb[kAhead - 1]);
            const uint32_t wv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            u16x2 m2 = {0, 0};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t a = wv[i] & 0x7FFF7FFFu;
                m2 = __builtin_elementwise_max(m2, *reinterpret_cast<const u16x2*>(&a));
            }
            uint32_t m = max((uint32_t)m2.x, (uint32_t)m2.y);
            m = max(m, dpp<0xB1>(m));                     // the lane pair = one group of 32
            const int E = moe::mx_exponent(__uint_as_float(m << 16));
            const float p2 = moe::exp2_neg(E);
            // an all-zero group (negative zeros included) stores zero bytes
            const bool zero = m == 0;
            uint32_t out[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                out[i] = zero ? 0u
                              : cvt4(moe::bf16_lo(wv[2 * i]) * p2, moe::bf16_hi(wv[2 * i]) * p2,
                                     moe::bf16_lo(wv[2 * i + 1]) * p2, moe::bf16_hi(wv[2 * i + 1]) * p2);
            // codes of the block's groups 0..3 sit in lanes sub = 0, 2, 4, 6
            const uint32_t code = (uint32_t)(E + 127);
            const int base = lane & ~7;
            const uint32_t packed = (uint32_t)__shfl((int)code, base, MOE_WAVE) |
                                    ((uint32_t)__shfl((int)code, base + 2, MOE_WAVE) << 8) |
                                    ((uint32_t)__shfl((int)code, base + 4, MOE_WAVE) << 16) |
                                    ((uint32_t)__shfl((int)code, base + 6, MOE_WAVE) << 24);
            if (act) {
                __builtin_nontemporal_store(moe::u32x4{out[0], out[1], out[2], out[3]}, dst + blk * 8 + sub);
                if (sub == 0) sdst[blk] = packed;
            }
        }
    }
    if (threadIdx.x % MOE_WAVE == 0) MOE_TRACE_PUT(moe::kTrQuantMx, blockIdx.x * kWaves + threadIdx.x / MOE_WAVE, threadIdx.x / MOE_WAVE, 0, tr0);
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
    const int64_t waves = d.T * kSplit;                          // one per row piece (slots_cap = T)
    const int grid = (int)std::min<int64_t>((waves + kWaves - 1) / kWaves, 16384);
    hipLaunchKernelGGL(quant_dispatch_kernel, dim3(grid), dim3(kBlock), 0,
                       reinterpret_cast<hipStream_t>(hip_stream), x_bf16, slot_tok, totals, d.T,
                       (int)d.H, q_e4m3, q_scale);
    return moe::launch_status();
}

extern "C" moe_status moe_quant_dispatch_mx(const moe_dims* dims, const uint16_t* x_bf16,
                                            const int32_t* slot_tok, const int32_t* totals,
                                            uint8_t* q_e4m3, uint32_t* q_scale, void* hip_stream) {
    moe::Dims d;
    moe_status st = moe::load_dims(dims, &d, true);
    if (st != MOE_OK) return st;
    if (d.T == 0) return MOE_OK;
    if (!x_bf16 || !slot_tok || !totals || !q_e4m3 || !q_scale) return MOE_ERR_INVALID_ARG;
    if (d.T * d.H >= ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
    const int64_t waves = d.T * kSplit;
    const int grid = (int)std::min<int64_t>((waves + kWaves - 1) / kWaves, 16384);
    hipLaunchKernelGGL(quant_dispatch_mx_kernel, dim3(grid), dim3(kBlock), 0,
                       reinterpret_cast<hipStream_t>(hip_stream), x_bf16, slot_tok, totals, d.T,
                       (int)d.H, q_e4m3, q_scale);
    return moe::launch_status();
}
