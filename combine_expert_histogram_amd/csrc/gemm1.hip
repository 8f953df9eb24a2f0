// Step 3: grouped GEMM1 over the local experts, A rows read in place through
// the rowmap ("poc(cco): MegaMoE stage1 dispatch over SDMA", "What": GEMM1
// reads its A rows in place through a rowmap; commit 1: fp8 rows and block
// scales through the rowmap; "Where we stand": block-scaled fp8 tiles, one
// expert per tile, the compute-bound loop of stage1).
//
// y[r, c] = sum_kb (sum_{h in kb} qA[r,h] * qW[c,h]) * sA[r,kb] * sW[c/128,kb]
//
// The scales are fp32 (not powers of two), so they cannot ride in the MFMA's
// e8m0 block scales: each 128-wide K block is one fp8 MFMA with a zero
// accumulator per 16x16 sub-tile (v_mfma_f32_16x16x128_f8f6f4 covers exactly
// K = 128), and its fp32 result is folded into the running sum with one FMA
// by sA[row] * sW (precomputed per row and K block in LDS).
//
// Tiles: 128 rows of one expert x 128 columns; 4 wavefronts in 2 x 2, each
// 64 x 64 = 4 x 4 MFMA sub-tiles.  A (gathered rows) and B (weight rows,
// K-contiguous) stage through LDS with an XOR swizzle of the 16 B chunk index
// by row, so the MFMA operand reads (16 rows x 32 B per quarter-wave) spread
// over the banks.  The grid is persistent; each workgroup derives the tile
// table (experts x column tiles x row tiles) from expert_offsets on the
// device, so no host read-back is needed.
#include "common.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int kMaxL = 1024;

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 4); }

__global__ void __launch_bounds__(kThreads)
grouped_gemm1_kernel(const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
                     const int32_t* __restrict__ row_slot, const int32_t* __restrict__ expert_offsets,
                     const uint8_t* __restrict__ w, const float* __restrict__ w_scale,
                     uint16_t* __restrict__ y, int L, int N, int H, int64_t T, int64_t rows_cap) {
    __shared__ __align__(16) uint8_t As[BM * BK];
    __shared__ __align__(16) uint8_t Bs[BN * BK];
    __shared__ __align__(16) float fs[BM];
    __shared__ int slot_s[BM];
    __shared__ int tstart[kMaxL + 1];     // first tile of each expert
    __shared__ int eoff[kMaxL + 1];

    const int tid = threadIdx.x;
    const int lane = tid % MOE_WAVE;
    const int wave = tid / MOE_WAVE;
    const int wm = wave >> 1, wn = wave & 1;
    const int NT = N / BN;
    const int KB = H / BK;

    // tile table: experts in order, each expert's tiles column-tile-major
    for (int i = tid; i <= L; i += kThreads) {
        int64_t o = expert_offsets[i];
        eoff[i] = (int)(o < 0 ? 0 : (o > rows_cap ? rows_cap : o));
    }
    __syncthreads();
    if (wave == 0) {
        int carry = 0;
        for (int base = 0; base < L; base += MOE_WAVE) {
            const int e = base + lane;
            int mt = 0;
            if (e < L) {
                const int cnt = eoff[e + 1] - eoff[e];
                mt = cnt > 0 ? (cnt + BM - 1) / BM : 0;
            }
            const int incl = moe::wave_inclusive_scan(mt * NT);
            if (e < L) tstart[e] = carry + incl - mt * NT;
            carry += __shfl(incl, MOE_WAVE - 1, MOE_WAVE);
        }
        if (lane == 0) tstart[L] = carry;
    }
    __syncthreads();
    const int total = tstart[L];

    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        // expert of this tile: last e with tstart[e] <= tile
        int lo = 0, hi = L - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tstart[mid] <= tile) lo = mid; else hi = mid - 1;
        }
        const int e = lo;
        const int cnt = eoff[e + 1] - eoff[e];
        const int mt = (cnt + BM - 1) / BM;
        const int local = tile - tstart[e];
        const int nt = local / mt;
        const int mtile = local - nt * mt;
        const int r0 = eoff[e] + mtile * BM;
        const int nvalid = min(BM, eoff[e + 1] - r0);
        const int n0 = nt * BN;

        for (int i = tid; i < BM; i += kThreads) {
            int s = -1;
            if (i < nvalid) {
                s = row_slot[r0 + i];
                if ((uint64_t)s >= (uint64_t)T) s = -1;
            }
            slot_s[i] = s;
        }
        __syncthreads();

        v4f acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

        const uint8_t* wexp = w + ((int64_t)e * N + n0) * H;
        const float* wsc = w_scale + ((int64_t)e * (N / 128) + n0 / 128) * KB;

        for (int kb = 0; kb < KB; ++kb) {
            // stage A rows (gathered through the rowmap) and B rows
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = (tid >> 3) + 32 * i;
                const int ch = tid & 7;
                const int s = slot_s[row];
                moe::u32x4 va = moe::u32x4{0u, 0u, 0u, 0u};
                if (s >= 0)
                    va = *reinterpret_cast<const moe::u32x4*>(q + (int64_t)s * H + kb * BK + ch * 16);
                *reinterpret_cast<moe::u32x4*>(As + swz(row, ch)) = va;
                const moe::u32x4 vb =
                    *reinterpret_cast<const moe::u32x4*>(wexp + (int64_t)row * H + kb * BK + ch * 16);
                *reinterpret_cast<moe::u32x4*>(Bs + swz(row, ch)) = vb;
            }
            if (tid < BM) {
                const int s = slot_s[tid];
                fs[tid] = s >= 0 ? q_scale[(int64_t)s * KB + kb] * wsc[kb] : 0.0f;
            }
            __syncthreads();

            v8i bf[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = wn * 64 + j * 16 + (lane & 15);
                const int c0 = (lane >> 4) * 2;
                const moe::u32x4 b0 = *reinterpret_cast<const moe::u32x4*>(Bs + swz(col, c0));
                const moe::u32x4 b1 = *reinterpret_cast<const moe::u32x4*>(Bs + swz(col, c0 + 1));
                bf[j] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                            (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wm * 64 + i * 16 + (lane & 15);
                const int c0 = (lane >> 4) * 2;
                const moe::u32x4 a0 = *reinterpret_cast<const moe::u32x4*>(As + swz(row, c0));
                const moe::u32x4 a1 = *reinterpret_cast<const moe::u32x4*>(As + swz(row, c0 + 1));
                const v8i af = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                                   (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                const v4f f = *reinterpret_cast<const v4f*>(fs + wm * 64 + i * 16 + 4 * (lane >> 4));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        af, bf[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[i][j][v] = fmaf(p[v], f[v], acc[i][j][v]);
                }
            }
            __syncthreads();
        }

        // epilogue: bf16 (RNE), valid rows only
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = wm * 64 + i * 16 + 4 * (lane >> 4) + v;
                if (row < nvalid) {
                    uint16_t* yrow = y + (int64_t)(r0 + row) * N + n0 + wn * 64 + (lane & 15);
#pragma unroll
                    for (int j = 0; j < 4; ++j) yrow[j * 16] = (uint16_t)moe::f32_to_bf16_rne(acc[i][j][v]);
                }
            }
        __syncthreads();
    }
}

}  // namespace

extern "C" moe_status moe_grouped_gemm1_workspace(const moe_dims* dims, int32_t n, size_t* bytes) {
    moe::Dims d;
    moe_status st = moe::load_dims(dims, &d, true);
    if (st != MOE_OK) return st;
    if (!bytes || n < 128 || n % 128 != 0) return MOE_ERR_INVALID_ARG;
    *bytes = 0;
    return MOE_OK;
}

extern "C" moe_status moe_grouped_gemm1(const moe_dims* dims, int32_t n, const uint8_t* q_e4m3,
                                        const float* q_scale, const int32_t* row_slot,
                                        const int32_t* expert_offsets, const int32_t* totals,
                                        const uint8_t* w_e4m3, const float* w_scale, uint16_t* y_bf16,
                                        void* ws, size_t ws_bytes, void* hip_stream) {
    (void)ws;
    (void)ws_bytes;
    (void)totals;
    moe::Dims d;
    moe_status st = moe::load_dims(dims, &d, true);
    if (st != MOE_OK) return st;
    if (n < 128 || n % 128 != 0) return MOE_ERR_INVALID_ARG;
    if (d.L > kMaxL) return MOE_ERR_UNSUPPORTED;
    if (d.T == 0) return MOE_OK;
    if (!q_e4m3 || !q_scale || !row_slot || !expert_offsets || !w_e4m3 || !w_scale || !y_bf16)
        return MOE_ERR_INVALID_ARG;
    const int64_t rows_cap = d.T * d.k;
    if (rows_cap * n >= ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
    // upper bound of the tile count: sum over experts of ceil(rows/BM)
    const int64_t max_tiles = ((rows_cap + BM - 1) / BM + d.L) * (n / BN);
    const int grid = (int)std::min<int64_t>(max_tiles, 512);
    hipLaunchKernelGGL(grouped_gemm1_kernel, dim3(grid), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(hip_stream), q_e4m3, q_scale, row_slot,
                       expert_offsets, w_e4m3, w_scale, y_bf16, (int)d.L, (int)n, (int)d.H, d.T,
                       rows_cap);
    return moe::launch_status();
}
