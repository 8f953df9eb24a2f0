// Measurement aids, not part of the hot path's C ABI (built as a separate
// library, libmoe_ceiling.so, loaded only by the benchmark):
//  * a kernel that does nothing but fp8 MFMAs, so the benchmark can report the
//    MFMA rate this chip sustains in the same run next to the grouped GEMM1's;
//  * a two-to-one read/write stream: each output word is the xor of two
//    consecutive 16 B words of the source (non-temporal loads and stores, 4
//    pairs in flight per lane, each workgroup one contiguous chunk), so the
//    benchmark can report what this chip sustains on a mix of two bytes read
//    per byte written, the quant's mix (measured: ≈5.2 TB/s cold for 160 MB
//    read + 80 MB written, against ≈7 TB/s for reads alone; ordinary stores or
//    fewer workgroups ran slower);
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

__global__ void __launch_bounds__(256) rw_stream_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        int64_t n_out16, int64_t chunk) {
    constexpr int U = 4;
    const int64_t beg = (int64_t)blockIdx.x * chunk;
    const int64_t end = min(n_out16, beg + chunk);
    int64_t i = beg + threadIdx.x;
    for (; i + (U - 1) * 256 < end; i += U * 256) {
        u32x4 a[U], b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            a[u] = __builtin_nontemporal_load(src + 2 * (i + u * 256));
            b[u] = __builtin_nontemporal_load(src + 2 * (i + u * 256) + 1);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) __builtin_nontemporal_store(a[u] ^ b[u], dst + i + u * 256);
    }
    for (; i < end; i += 256) __builtin_nontemporal_store(src[2 * i] ^ src[2 * i + 1], dst + i);
}

}  // namespace

// Writes out_bytes (a multiple of 16) to the device buffer `dst`, each 16 B word
// the xor of two consecutive words of `src` (2 * out_bytes), with grid
// workgroups of 256 threads on `hip_stream`, workgroup i handling the i-th of
// grid equal contiguous chunks.  Returns 0, or -1 for bad arguments / a launch
// error.
extern "C" int moe_ceiling_rw_stream(const void* src, void* dst, int64_t out_bytes, int grid, void* hip_stream) {
    if (!src || !dst || grid <= 0 || out_bytes <= 0 || out_bytes % 16 != 0) return -1;
    const int64_t n16 = out_bytes / 16;
    const int64_t chunk = (n16 + grid - 1) / grid;
    hipLaunchKernelGGL(rw_stream_kernel, dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(hip_stream),
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16, chunk);
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
