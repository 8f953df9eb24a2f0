// Step 4: combine - top-k weighted gather-sum of expert output rows back to
// token order (TilePipe "Communication Kernels": push combine to the token
// owners; "poc(cco): MegaMoE stage1 dispatch over SDMA", "What": stage2 +
// combine produce the layer output from the expert-major tables).
//
//   out[g, c] = bf16( sum_{j < k, assign_row[g*k+j] valid} w[g,j] * y[row, c] )
//
// fp32 accumulation in ascending j (fused multiply-add).  The step is a pure
// HBM stream: every expert row is read once (assign_row is a bijection onto
// the rows) and every output row written once.  A thread owns 8 columns
// (one 16 B load per contribution, one 16 B store); all k loads of a thread
// are issued before the first FMA so that 8 x 16 B per lane are in flight.
#include "common.h"

namespace {

constexpr int kThreads = 128;

template <int K>
__global__ void __launch_bounds__(kThreads)
combine_kernel(const uint16_t* __restrict__ y, int64_t y_rows, const int32_t* __restrict__ assign_row,
               const float* __restrict__ topk_w, uint16_t* __restrict__ out, int width, int k,
               int col_blocks) {
    MOE_TRACE_T0(tr0);
    const int64_t g = blockIdx.x / col_blocks;
    const int cb = blockIdx.x - (int)(g * col_blocks);
    const int c8 = cb * kThreads + threadIdx.x;         // group of 8 columns
    if (c8 * 8 >= width) return;
    const int32_t* ar = assign_row + g * k;
    const float* wt = topk_w + g * k;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    constexpr int KC = K > 0 ? K : 8;                   // contributions per round
    for (int j0 = 0; j0 < k; j0 += KC) {
        moe::u32x4 v[KC];
        float wj[KC];
        bool ok[KC];
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            const int jj = j0 + j;
            const int r = jj < k ? ar[jj] : -1;
            ok[j] = r >= 0 && (int64_t)r < y_rows;
            wj[j] = ok[j] ? wt[jj] : 0.0f;
            v[j] = ok[j] ? __builtin_nontemporal_load(
                               reinterpret_cast<const moe::u32x4*>(y + (int64_t)r * width) + c8)
                         : moe::u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            if (!ok[j]) continue;                       // absent rows add nothing
            const uint32_t wv[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = fmaf(wj[j], moe::bf16_lo(wv[i]), acc[2 * i]);
                acc[2 * i + 1] = fmaf(wj[j], moe::bf16_hi(wv[i]), acc[2 * i + 1]);
            }
        }
    }
    moe::u32x4 o;
    o.x = moe::pack_bf16x2(acc[0], acc[1]);
    o.y = moe::pack_bf16x2(acc[2], acc[3]);
    o.z = moe::pack_bf16x2(acc[4], acc[5]);
    o.w = moe::pack_bf16x2(acc[6], acc[7]);
    __builtin_nontemporal_store(o, reinterpret_cast<moe::u32x4*>(out + g * width) + c8);
    if (threadIdx.x == 0) MOE_TRACE_PUT(moe::kTrCombine, blockIdx.x, 0, 0, tr0);
}

}  // namespace

extern "C" moe_status moe_combine(const moe_dims* dims, int32_t width, const uint16_t* y_bf16,
                                  int64_t y_rows, const int32_t* assign_row, const float* topk_w,
                                  uint16_t* out_bf16, void* hip_stream) {
    moe::Dims d;
    moe_status st = moe::load_dims(dims, &d, false);
    if (st != MOE_OK) return st;
    if (width < 8 || width % 8 != 0 || y_rows < 0) return MOE_ERR_INVALID_ARG;
    if (d.T == 0) return MOE_OK;
    if (!assign_row || !topk_w || !out_bf16 || (y_rows > 0 && !y_bf16)) return MOE_ERR_INVALID_ARG;
    const int col_blocks = (width / 8 + kThreads - 1) / kThreads;
    const int64_t grid = d.T * col_blocks;
    if (grid > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
#define MOE_COMBINE_LAUNCH(KK)                                                                  \
    hipLaunchKernelGGL(combine_kernel<KK>, dim3((unsigned)grid), dim3(kThreads), 0, stream, y_bf16, \
                       y_rows, assign_row, topk_w, out_bf16, (int)width, (int)d.k, col_blocks)
    switch (d.k) {
        case 1: MOE_COMBINE_LAUNCH(1); break;
        case 2: MOE_COMBINE_LAUNCH(2); break;
        case 4: MOE_COMBINE_LAUNCH(4); break;
        case 6: MOE_COMBINE_LAUNCH(6); break;
        case 8: MOE_COMBINE_LAUNCH(8); break;
        default: MOE_COMBINE_LAUNCH(0); break;
    }
#undef MOE_COMBINE_LAUNCH
    return moe::launch_status();
}
