// Clock-stamp trace of the kernels' workgroups, wavefronts and GEMM tiles, a
// measurement aid compiled in only when the library is built with
// MOE_TRACE=1 (libmoe_hotpath_trace.so, `python -m
// combine_expert_histogram_amd.build --trace`).  In the product build every
// macro below expands to nothing and the kernels are unchanged.
//
// A record is {begin, end, kernel, block, item, aux}: both stamps read
// s_memrealtime (a constant 100 MHz counter common to the whole chip), kernel
// is a TraceKernel id, block the workgroup, item and aux what the kernel
// stores there (the wavefront; a GEMM tile's id and its position in the
// workgroup's tile sequence).  Records go to a device buffer the caller
// attaches with moe_trace_attach (traced build only; not part of the hot
// path's C ABI): a 16-byte header {records per kernel id, 0, 0, 0}, then one
// region of that many records per kernel id (16 ids).  A unit writes its own
// slot of its kernel's region (the workgroup, workgroup x 4 + wavefront, or
// the tile id): one plain store, no atomics, so the stamps do not serialise
// the kernel (an append counter did: 32K quant wavefronts queued on one
// address for over a millisecond).  Slots past the region are dropped; the
// attach call zeroes the buffer, so unwritten slots read as kernel 0.  One
// call at a time is meant to be traced: a second call of the same kernel
// overwrites the first one's slots.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_hotpath.h"

#ifndef MOE_TRACE
#define MOE_TRACE 0
#endif

namespace moe {

enum TraceKernel : uint32_t {
    kTrLayoutCount = 1,   // per workgroup
    kTrLayoutPlace = 2,   // per workgroup
    kTrQuant = 3,         // per wavefront (item = wavefront of the workgroup)
    kTrQuantMx = 4,       // per wavefront
    kTrGemmPrep = 5,      // per workgroup (block 0 plans the tiles)
    kTrGemmLoader = 6,    // per workgroup: the first loader wavefront, start to last load
    kTrGemmCompute = 7,   // per workgroup: compute wavefront 0, start to last store
    kTrGemmTile = 8,      // per tile (item = tile id, aux = position in the sequence)
    kTrCombine = 9,       // per workgroup
    kTrAct = 10,          // per wavefront (stage2 act)
};

struct TraceRec {
    uint64_t t0, t1;
    uint32_t kernel, block, item, aux;
};
static_assert(sizeof(TraceRec) == 32, "record layout");

}  // namespace moe

#if MOE_TRACE

namespace moe {

struct TraceHdr {
    uint32_t region, pad0, pad1, pad2;
};
constexpr uint32_t kTraceKernels = 16;

// The attached buffer, as seen by this source file's kernels (the library's
// source files are separate device code objects, each with its own copy, all
// set by moe_trace_attach through the registry below).
static __device__ TraceHdr* g_trace_buf;

__device__ __forceinline__ uint64_t trace_now() { return __builtin_amdgcn_s_memrealtime(); }

// Writes {t0, now, kernel, blockIdx.x, item, aux} into slot `slot` of the
// kernel's region; called by one lane.
__device__ __forceinline__ void trace_put(uint32_t kernel, uint32_t slot, uint32_t item, uint32_t aux, uint64_t t0) {
    TraceHdr* h = g_trace_buf;
    if (!h || kernel >= kTraceKernels || slot >= h->region) return;
    const uint64_t t1 = trace_now();
    reinterpret_cast<TraceRec*>(h + 1)[(uint64_t)kernel * h->region + slot] =
        TraceRec{t0, t1, kernel, blockIdx.x, item, aux};
}

// host side: every source file registers a setter of its copy of the pointer
typedef int (*TraceSetter)(void* device_buf);
int trace_register(TraceSetter f);   // api.hip

static int trace_set_this_file(void* p) {
    return hipMemcpyToSymbol(HIP_SYMBOL(g_trace_buf), &p, sizeof(p)) == hipSuccess ? 0 : -1;
}
static const int g_trace_registered = trace_register(&trace_set_this_file);

}  // namespace moe

#define MOE_TRACE_T0(name) const uint64_t name = ::moe::trace_now()
#define MOE_TRACE_PUT(kernel, slot, item, aux, t0) ::moe::trace_put((kernel), (slot), (item), (aux), (t0))

extern "C" {
// Attaches a device buffer of `bytes` (16-byte header, then 16 regions of
// (bytes - 16) / 512 records of 32 bytes; zeroed and the header written here,
// synchronously) that every kernel of the library writes its records to from
// now on.  Returns MOE_ERR_INVALID_ARG for a null buffer or one too small for a
// record per region, MOE_ERR_HIP if a copy fails.
moe_status moe_trace_attach(void* device_buf, uint64_t bytes);
// Detaches the buffer: kernels launched afterwards record nothing.
moe_status moe_trace_detach(void);
}

#else

#define MOE_TRACE_T0(name) \
    do {                   \
    } while (0)
#define MOE_TRACE_PUT(kernel, slot, item, aux, t0) \
    do {                                           \
    } while (0)

#endif
