// Internal helpers shared by the HIP kernels and the C ABI wrappers.
// CDNA4 (gfx950): 64-lane wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "moe_hotpath.h"
#include "trace.h"

#define MOE_WAVE 64

namespace moe {

// Native 16-byte vector (ext_vector_type, usable with the nontemporal builtins).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- host side
struct Dims {
    int64_t S, Ts, T, k, E, e0, L, H;
};

// Validates the dims fields every call shares.  H is only checked when a step
// uses it (need_hidden).
inline moe_status load_dims(const moe_dims* d, Dims* out, bool need_hidden) {
    if (!d || !out) return MOE_ERR_INVALID_ARG;
    if (d->num_sources < 1 || d->tokens_per_source < 0) return MOE_ERR_INVALID_ARG;
    if (d->num_experts < 1 || d->top_k < 1 || d->top_k > d->num_experts) return MOE_ERR_INVALID_ARG;
    if (d->expert_begin < 0 || d->num_local_experts < 1) return MOE_ERR_INVALID_ARG;
    if ((int64_t)d->expert_begin + d->num_local_experts > d->num_experts) return MOE_ERR_INVALID_ARG;
    if (need_hidden && (d->hidden < 128 || d->hidden % 128 != 0)) return MOE_ERR_INVALID_ARG;
    Dims r;
    r.S = d->num_sources;
    r.Ts = d->tokens_per_source;
    r.T = r.S * r.Ts;
    r.k = d->top_k;
    r.E = d->num_experts;
    r.e0 = d->expert_begin;
    r.L = d->num_local_experts;
    r.H = d->hidden;
    // int32 indices everywhere: T*k rows and slot*H bytes must fit.
    if (r.T * r.k >= (int64_t)INT32_MAX) return MOE_ERR_UNSUPPORTED;
    *out = r;
    return MOE_OK;
}

inline moe_status launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// ---------------------------------------------------------------- device side
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = __lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Wave-wide inclusive prefix sum of an int (64 lanes, shuffle based).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int l = __lane_id();
#pragma unroll
    for (int off = 1; off < MOE_WAVE; off <<= 1) {
        int t = __shfl_up(v, off, MOE_WAVE);
        if (l >= off) v += t;
    }
    return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int off = MOE_WAVE / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, MOE_WAVE);
    return v;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
// two fp32 values rounded to nearest-even bf16 and packed (lo in bits 0..15):
// one v_cvt_pk_bf16_f32 (NaNs stay NaNs)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

}  // namespace moe
