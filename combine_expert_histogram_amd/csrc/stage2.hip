// Stage2 activation: h = silu(gate) * up on each expert-major row of GEMM1's
// output ([R, 2I] bf16: gate columns [0, I), up columns [I, 2I)), quantised
// straight to fp8 e4m3 with one fp32 scale per 128 elements of h (GEMM1's
// activation rule), the A operand of the down-projection GEMM2
// ("poc(cco): MegaMoE stage1 dispatch over SDMA", "What": stage1's output
// feeds stage2 + combine).
//
// Mapping: a work item is one pass over 1024 elements of h (8 blocks of 128)
// of one row, one wavefront per item; lane l takes 16 consecutive elements of
// block l/8: two 16 B loads of gate and two of up (each wavefront load a
// contiguous 1 KiB of the row), silu * up in fp32 (exp and reciprocal from
// the hardware's approximations: h is not bit-reproducible on the host and
// its codes are checked to tolerance), the block |max| over the block's 8
// lanes by DPP, the block's codes and scale by encode_block16 (exact given
// h), and one contiguous 16 B code store per lane.  HBM bound: per row it
// reads 4I bytes and writes I + I/32.  The GEMM1 rows are read with ordinary
// loads (they may still be in the last-level cache right after GEMM1; 1-2 %
// faster than non-temporal loads there and after a cache flush) and the codes
// written with non-temporal stores.
//
// MX variant (the pages' e8m0 format, "Where we stand"; packed four per dword,
// commit "ready-first / quant-lds-store"): a group of 32 elements of h is one
// lane pair, its |max| one DPP exchange, E = mx_exponent(|max|), payload
// e4m3(h * 2^-E) (exact scaling), the block's four codes packed by lane
// shuffles into one dword per 128 elements.
#include "fp8_block.h"

namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / MOE_WAVE;

__device__ __forceinline__ float silu_mul(float g, float u) {
    // silu(g) = g / (1 + e^-g); e^-g overflows to +inf for g < -88, giving -0
    const float e = __expf(-g);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

template <bool MX>
__global__ void __launch_bounds__(kBlock)
silu_mul_quant_kernel(const uint16_t* __restrict__ y1, const int32_t* __restrict__ totals, int64_t rows_cap,
                      int I, uint8_t* __restrict__ q, void* __restrict__ q_scale_v) {
    MOE_TRACE_T0(tr0);
    const int64_t R = min((int64_t)totals[0], rows_cap);
    const int lane = threadIdx.x % MOE_WAVE;
    const int sub = lane & 7;
    const int nblk = I / 128;
    const int passes = (nblk + 7) / 8;
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    for (int64_t it = (int64_t)blockIdx.x * kWaves + threadIdx.x / MOE_WAVE; it < R * passes; it += nwaves) {
        const int64_t r = it / passes;
        const int blk = (int)(it - r * passes) * 8 + (lane >> 3);
        const bool act = blk < nblk;
        const int b = act ? blk : nblk - 1;                 // idle lanes re-read the last block
        const moe::u32x4* gp = reinterpret_cast<const moe::u32x4*>(y1 + r * 2 * I + b * 128 + sub * 16);
        const moe::u32x4* up = reinterpret_cast<const moe::u32x4*>(y1 + r * 2 * I + I + b * 128 + sub * 16);
        const moe::u32x4 g0 = *gp, g1 = *(gp + 1);
        const moe::u32x4 u0 = *up, u1 = *(up + 1);
        const uint32_t gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        const uint32_t uw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
        float h[16];
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            h[2 * i] = silu_mul(moe::bf16_lo(gw[i]), moe::bf16_lo(uw[i]));
            h[2 * i + 1] = silu_mul(moe::bf16_hi(gw[i]), moe::bf16_hi(uw[i]));
            m = max(m, __float_as_uint(h[2 * i]) & 0x7FFFFFFFu);
            m = max(m, __float_as_uint(h[2 * i + 1]) & 0x7FFFFFFFu);
        }
        uint32_t out[4];
        moe::u32x4* dst = reinterpret_cast<moe::u32x4*>(q + r * I + b * 128 + sub * 16);
        if constexpr (MX) {
            m = max(m, moe::dpp<0xB1>(m));                  // the lane pair = one group of 32
            const int E = moe::mx_exponent(__uint_as_float(m));
            const float p2 = moe::exp2_neg(E);
            const bool zero = m == 0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                out[i] = zero ? 0u : moe::cvt4(h[4 * i] * p2, h[4 * i + 1] * p2, h[4 * i + 2] * p2, h[4 * i + 3] * p2);
            // codes of the block's groups 0..3 sit in lanes sub = 0, 2, 4, 6
            const int code = E + 127;
            const int base = lane & ~7;
            const uint32_t packed = (uint32_t)__shfl(code, base, MOE_WAVE) |
                                    ((uint32_t)__shfl(code, base + 2, MOE_WAVE) << 8) |
                                    ((uint32_t)__shfl(code, base + 4, MOE_WAVE) << 16) |
                                    ((uint32_t)__shfl(code, base + 6, MOE_WAVE) << 24);
            if (act) {
                __builtin_nontemporal_store(moe::u32x4{out[0], out[1], out[2], out[3]}, dst);
                if (sub == 0) static_cast<uint32_t*>(q_scale_v)[r * nblk + b] = packed;
            }
        } else {
            m = moe::group8_max(m);
            const float s = moe::encode_block16(h, __uint_as_float(m), out);
            if (act) {
                __builtin_nontemporal_store(moe::u32x4{out[0], out[1], out[2], out[3]}, dst);
                if (sub == 0) static_cast<float*>(q_scale_v)[r * nblk + b] = s;
            }
        }
    }
    if (threadIdx.x % MOE_WAVE == 0) MOE_TRACE_PUT(moe::kTrAct, blockIdx.x * kWaves + threadIdx.x / MOE_WAVE, threadIdx.x / MOE_WAVE, 0, tr0);
}

template <bool MX>
moe_status run_silu_mul_quant(const moe_dims* dims, int32_t inter, const uint16_t* y1_bf16, const int32_t* totals,
                              uint8_t* h_e4m3, void* h_scale, void* hip_stream) {
    moe::Dims d;
    moe_status st = moe::load_dims(dims, &d, false);
    if (st != MOE_OK) return st;
    if (inter < 128 || inter % 128 != 0) return MOE_ERR_INVALID_ARG;
    if (d.T == 0) return MOE_OK;
    if (!y1_bf16 || !totals || !h_e4m3 || !h_scale) return MOE_ERR_INVALID_ARG;
    const int64_t rows_cap = d.T * d.k;
    if (rows_cap * 2 * inter >= ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
    const int64_t items = rows_cap * ((inter / 128 + 7) / 8);
    const int grid = (int)std::min<int64_t>((items + kWaves - 1) / kWaves, 16384);
    hipLaunchKernelGGL(silu_mul_quant_kernel<MX>, dim3(grid), dim3(kBlock), 0,
                       reinterpret_cast<hipStream_t>(hip_stream), y1_bf16, totals, rows_cap, (int)inter,
                       h_e4m3, h_scale);
    return moe::launch_status();
}

}  // namespace

extern "C" moe_status moe_silu_mul_quant(const moe_dims* dims, int32_t inter, const uint16_t* y1_bf16,
                                         const int32_t* totals, uint8_t* h_e4m3, float* h_scale,
                                         void* hip_stream) {
    return run_silu_mul_quant<false>(dims, inter, y1_bf16, totals, h_e4m3, h_scale, hip_stream);
}

extern "C" moe_status moe_silu_mul_quant_mx(const moe_dims* dims, int32_t inter, const uint16_t* y1_bf16,
                                            const int32_t* totals, uint8_t* h_e4m3, uint32_t* h_scale,
                                            void* hip_stream) {
    return run_silu_mul_quant<true>(dims, inter, y1_bf16, totals, h_e4m3, h_scale, hip_stream);
}
