// Measurement aids, not part of the hot path's C ABI (built as a separate
// library, libmoe_ceiling.so, loaded only by the benchmark):
//  * a kernel that does nothing but fp8 MFMAs, so the benchmark can report the
//    MFMA rate this chip sustains in the same run next to the grouped GEMM1's;
//  * read/write streams: output word i is the xor of word i of each of two
//    (four, or eight) planes of the source (non-temporal loads and stores, 8 loads in
//    flight per lane, one pass of small workgroups), so the benchmark can
//    report what this chip sustains on a mix of two bytes read per byte
//    written, the quant's mix, and of eight, the combine's (in a sweep over
//    launch shapes many one-pass workgroups ran fastest: 6.1 TB/s for 1.9 GB
//    read + 235 MB written against 5.5 TB/s with 8 workgroups a CU each
//    streaming a contiguous chunk; ordinary loads ran slower);
//  * a read stream: one pass of 16 B loads over a buffer, each workgroup
//    reading one contiguous chunk (8 loads in flight per lane), folded into one
//    word per thread, so the benchmark can report the HBM read rate this chip
//    sustains (the hot path's HBM-bound kernels mostly read: the combine reads
//    9 bytes for each one it writes).  Contiguous chunks measured faster than a
//    grid-stride sweep (about 6.9-7.0 against 5.8-6.1 TB/s over 2 GiB) and
//    non-temporal loads faster than ordinary ones; the ordinary-load form
//    leaves the buffer's lines in the caches, which makes it a cache flush that
//    leaves nothing dirty behind (a write flush makes the next kernel pay for
//    writing the flush's lines back).
//
// Each wavefront keeps 16 independent 16x16x128 fp8 MFMA accumulators and
// runs `iters` rounds of 16 MFMAs (the operands vary with the lane and the
// accumulators carry from round to round, so nothing can be hoisted); 8
// wavefronts per workgroup, one workgroup per CU.  The scaled variant passes
// per-lane e8m0 block scales (codes 126 .. 129) as the MX GEMM1 does.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <bool SCALED>
__global__ void __launch_bounds__(512) mfma_loop_kernel(int iters, float* out) {
    const int lane = threadIdx.x;
    const int sa = SCALED ? 126 + (lane & 3) : 0, sb = SCALED ? 126 + ((lane >> 2) & 3) : 0;
    const v8i a = {lane, lane * 3, 0x38383838, 0x30303030, lane ^ 0x55, 11, 13, lane * 5};
    const v8i b = {lane * 7, 0x38383838, 2, 3, 0x28282828, 5, lane, 7};
    v4f acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 16; ++k)
            acc[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[k], 0, 0, 0, sa, 0, sb);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const u32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT>
__global__ void __launch_bounds__(256) read_stream_kernel(const u32x4* __restrict__ p, int64_t n16, int64_t chunk,
                                                          uint32_t* __restrict__ out) {
    constexpr int U = 8;
    const int64_t beg = (int64_t)blockIdx.x * chunk;
    const int64_t end = min(n16, beg + chunk);
    uint32_t acc = 0;
    int64_t i = beg + threadIdx.x;
    for (; i + (U - 1) * 256 < end; i += U * 256) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = ld16<NT>(p + i + u * 256);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < end; i += 256) {
        const u32x4 a = ld16<NT>(p + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// one pass per workgroup: U output words a lane (RATIO loads each), U * 256
// consecutive words a workgroup
template <int RATIO, int U>
__global__ void __launch_bounds__(256) rw_stream_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        int64_t n_out16) {
    const int64_t i0 = (int64_t)blockIdx.x * (U * 256) + threadIdx.x;
    u32x4 a[U][RATIO];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < RATIO; ++r)
            if (i0 + u * 256 < n_out16) a[u][r] = __builtin_nontemporal_load(src + r * n_out16 + i0 + u * 256);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (i0 + u * 256 >= n_out16) continue;
        u32x4 v = a[u][0];
#pragma unroll
        for (int r = 1; r < RATIO; ++r) v ^= a[u][r];
        __builtin_nontemporal_store(v, dst + i0 + u * 256);
    }
}

}  // namespace

// Writes out_bytes (a multiple of 16) to the device buffer `dst`, 16 B word i
// the xor of word i of each of the `ratio` (2, 4 or 8) consecutive
// out_bytes-sized planes of `src` (ratio * out_bytes), on `hip_stream`: one
// pass of 256-thread workgroups, 4 (ratio 2), 2 (ratio 4) or 1 (ratio 8)
// output words a lane, so 8 loads a lane are in flight.  Ratio 4 is stage2's
// act mix (four bytes read per byte written).  Returns 0, or -1 for bad
// arguments / a launch error.
extern "C" int moe_ceiling_rw_stream(const void* src, void* dst, int64_t out_bytes, int ratio, void* hip_stream) {
    if (!src || !dst || out_bytes <= 0 || out_bytes % 16 != 0 || (ratio != 2 && ratio != 4 && ratio != 8)) return -1;
    const int64_t n16 = out_bytes / 16;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    if (ratio == 2)
        hipLaunchKernelGGL((rw_stream_kernel<2, 4>), dim3((unsigned)((n16 + 1023) / 1024)), dim3(256), 0, st,
                           static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
    else if (ratio == 4)
        hipLaunchKernelGGL((rw_stream_kernel<4, 2>), dim3((unsigned)((n16 + 511) / 512)), dim3(256), 0, st,
                           static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
    else
        hipLaunchKernelGGL((rw_stream_kernel<8, 1>), dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, st,
                           static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Reads `bytes` (a multiple of 16) from the device buffer `buf` once with grid
// workgroups of 256 threads on `hip_stream`, workgroup i reading the i-th of
// grid equal contiguous chunks; non-temporal loads unless `temporal` is
// nonzero.  `out` holds grid * 256 words.  Returns 0, or -1 for bad arguments /
// a launch error.
extern "C" int moe_ceiling_read_stream(const void* buf, int64_t bytes, int grid, int temporal, uint32_t* out,
                                       void* hip_stream) {
    if (!buf || !out || grid <= 0 || bytes <= 0 || bytes % 16 != 0) return -1;
    const int64_t n16 = bytes / 16;
    const int64_t chunk = (n16 + grid - 1) / grid;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    if (temporal)
        hipLaunchKernelGGL(read_stream_kernel<false>, dim3(grid), dim3(256), 0, st, static_cast<const u32x4*>(buf),
                           n16, chunk, out);
    else
        hipLaunchKernelGGL(read_stream_kernel<true>, dim3(grid), dim3(256), 0, st, static_cast<const u32x4*>(buf),
                           n16, chunk, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Launches grid workgroups of 512 threads on `hip_stream`; `out` holds
// grid * 512 floats.  FLOP per launch = grid * 8 * iters * 16 * 65536.
// Returns 0, or -1 for bad arguments / a launch error.
extern "C" int moe_ceiling_mfma_fp8(int grid, int iters, float* out, void* hip_stream) {
    if (grid <= 0 || iters <= 0 || !out) return -1;
    hipLaunchKernelGGL(mfma_loop_kernel<false>, dim3(grid), dim3(512), 0,
                       reinterpret_cast<hipStream_t>(hip_stream), iters, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// The same with nonzero per-lane e8m0 scales (the MX GEMM1's instruction form).
extern "C" int moe_ceiling_mfma_fp8_scaled(int grid, int iters, float* out, void* hip_stream) {
    if (grid <= 0 || iters <= 0 || !out) return -1;
    hipLaunchKernelGGL(mfma_loop_kernel<true>, dim3(grid), dim3(512), 0,
                       reinterpret_cast<hipStream_t>(hip_stream), iters, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
