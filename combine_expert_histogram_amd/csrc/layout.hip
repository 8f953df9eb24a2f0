// Step 1: layout - stable counting sort of routed assignments into
// expert-major rows, plus the compact landed-token slot list.
//
// What is computed follows "poc(cco): MegaMoE stage1 dispatch over SDMA"
// (commit "recv_layout": the receiver counts the routes per expert and writes
// the rowmap / srcmap tables) and "EPDispatchKernel"
// (wait_for_arrivals_and_compute_offsets: per-local-expert offsets; the rows of
// one expert are one contiguous range).  Rows of an expert are in ascending
// (token, k-slot) order, so the result is unique and the tables are
// bit-reproducible run to run.
//
// Three launches (no grid-wide barrier: a grid barrier needs co-residency, and
// on gfx950 cross-workgroup release/acquire costs whole-L2 write-back /
// invalidate, "cut the whole-L2 cache operations" commit of the same PR):
//   count   - one wavefront per chunk of CT tokens: per-chunk expert histogram
//             (LDS atomics; order does not matter for counts) and the chunk's
//             landed-token count.
//   scan    - one 1024-thread workgroup: exclusive scan of the histogram in
//             expert-major order -> each chunk's first row per expert, the
//             expert offsets, and each chunk's first slot.
//   scatter - one wavefront per chunk again: ranks every local assignment
//             among the equal-expert assignments before it in the chunk.  A
//             pass takes 64 consecutive assignments; lanes with the same expert
//             find each other through a per-expert 64-bit lane mask in LDS
//             (ds_or), so a pass costs a fixed handful of LDS round trips
//             whatever the number of distinct experts in it.
#include "common.h"

namespace {

using moe::Dims;

constexpr int kBlock = 256;                       // 4 wavefronts, one chunk each
constexpr int kWaves = kBlock / MOE_WAVE;
constexpr int kScanThreads = 1024;
constexpr int kScanPerThread = 8;
constexpr int64_t kHistTarget = 32768;            // histogram entries the scan aims for
constexpr int kMaxLocalExperts = 1024;

struct Plan {
    int64_t CT = 16;   // tokens per chunk
    int64_t NC = 0;    // chunks
    // workspace offsets in int32 units
    int64_t off_hist = 0, off_base = 0, off_landed = 0, off_slot = 0, total_ints = 0;
};

Plan make_plan(const Dims& d) {
    Plan p;
    p.CT = 16;
    auto nchunks = [&](int64_t ct) { return (d.T + ct - 1) / ct; };
    while (nchunks(p.CT) * d.L > kHistTarget && p.CT < 512) p.CT *= 2;
    p.NC = nchunks(p.CT);
    auto al = [](int64_t v) { return (v + 63) & ~int64_t(63); };   // 256-byte alignment
    p.off_hist = 0;
    p.off_base = al(p.off_hist + d.L * p.NC);
    p.off_landed = al(p.off_base + d.L * p.NC);
    p.off_slot = al(p.off_landed + p.NC);
    p.total_ints = al(p.off_slot + p.NC);
    return p;
}

size_t count_lds(const Dims& d, const Plan& p) { return kWaves * (d.L * 4 + p.CT); }
size_t scatter_lds(const Dims& d, const Plan& p) {
    return kWaves * (d.L * 8 + d.L * 4 + p.CT * 4 + p.CT);
}

// ------------------------------------------------------------------ count
__global__ void __launch_bounds__(kBlock)
layout_count_kernel(const int32_t* __restrict__ ids, int64_t T, int k, int e0, int L,
                    int CT, int NC, int32_t* __restrict__ hist, int32_t* __restrict__ landed) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int wave = threadIdx.x / MOE_WAVE;
    const int lane = threadIdx.x % MOE_WAVE;
    const int c = blockIdx.x * kWaves + wave;
    int* cnt = reinterpret_cast<int*>(smem) + wave * L;
    unsigned char* flag = smem + kWaves * L * 4 + wave * CT;

    for (int i = lane; i < L; i += MOE_WAVE) cnt[i] = 0;
    for (int i = lane; i < CT; i += MOE_WAVE) flag[i] = 0;
    __syncthreads();

    const int64_t t0 = (int64_t)c * CT;
    const int64_t t1 = c < NC ? min(T, t0 + CT) : t0;
    for (int64_t a = t0 * k + lane; a < t1 * k; a += MOE_WAVE) {
        const int le = ids[a] - e0;
        if ((unsigned)le < (unsigned)L) {
            atomicAdd(&cnt[le], 1);
            flag[a / k - t0] = 1;
        }
    }
    __syncthreads();

    if (c < NC) {
        int nl = 0;
        for (int64_t t = t0 + lane; t < t1; t += MOE_WAVE) nl += flag[t - t0];
        nl = moe::wave_sum(nl);
        for (int i = lane; i < L; i += MOE_WAVE) hist[(int64_t)i * NC + c] = cnt[i];
        if (lane == 0) landed[c] = nl;
    }
}

// ------------------------------------------------------------------ scan
// Block-wide exclusive scan over n ints in tiles of 1024*8; out(idx, prefix)
// is called for every index.  Returns the total.
template <class Out>
__device__ int block_exclusive_scan(const int32_t* __restrict__ in, int64_t n, Out out) {
    __shared__ int wsum[kScanThreads / MOE_WAVE];
    const int tid = threadIdx.x;
    const int wave = tid / MOE_WAVE, lane = tid % MOE_WAVE;
    int carry = 0;
    for (int64_t tile = 0; tile < n; tile += (int64_t)kScanThreads * kScanPerThread) {
        int v[kScanPerThread];
        int s = 0;
#pragma unroll
        for (int i = 0; i < kScanPerThread; ++i) {
            const int64_t idx = tile + (int64_t)tid * kScanPerThread + i;
            v[i] = idx < n ? in[idx] : 0;
            s += v[i];
        }
        const int incl = moe::wave_inclusive_scan(s);
        if (lane == MOE_WAVE - 1) wsum[wave] = incl;
        __syncthreads();
        if (wave == 0) {
            int x = lane < kScanThreads / MOE_WAVE ? wsum[lane] : 0;
            x = moe::wave_inclusive_scan(x);
            if (lane < kScanThreads / MOE_WAVE) wsum[lane] = x;
        }
        __syncthreads();
        int ex = carry + incl - s + (wave ? wsum[wave - 1] : 0);
        const int tile_total = wsum[kScanThreads / MOE_WAVE - 1];
#pragma unroll
        for (int i = 0; i < kScanPerThread; ++i) {
            const int64_t idx = tile + (int64_t)tid * kScanPerThread + i;
            if (idx < n) out(idx, ex);
            ex += v[i];
        }
        carry += tile_total;
        __syncthreads();
    }
    return carry;
}

__global__ void __launch_bounds__(kScanThreads)
layout_scan_kernel(const int32_t* __restrict__ hist, const int32_t* __restrict__ landed,
                   int L, int NC, int S, int64_t Ts, int32_t* __restrict__ base,
                   int32_t* __restrict__ slot_base, int32_t* __restrict__ expert_counts,
                   int32_t* __restrict__ expert_offsets, int32_t* __restrict__ src_slot_offsets,
                   int32_t* __restrict__ totals) {
    __shared__ int offs[kMaxLocalExperts + 1];
    for (int i = threadIdx.x; i <= L; i += kScanThreads) offs[i] = 0;
    __syncthreads();

    const int64_t nh = (int64_t)L * NC;
    const int R = block_exclusive_scan(hist, nh, [&](int64_t idx, int ex) {
        const int le = (int)(idx / NC);
        const int c = (int)(idx - (int64_t)le * NC);
        base[(int64_t)c * L + le] = ex;
        if (c == 0) offs[le] = ex;
    });
    const int U = block_exclusive_scan(landed, NC, [&](int64_t idx, int ex) { slot_base[idx] = ex; });
    __syncthreads();
    if (NC == 0) {
        for (int i = threadIdx.x; i < L; i += kScanThreads) offs[i] = 0;
        __syncthreads();
    }
    if (threadIdx.x == 0) offs[L] = R;
    __syncthreads();
    for (int i = threadIdx.x; i < L; i += kScanThreads) {
        expert_offsets[i] = offs[i];
        expert_counts[i] = offs[i + 1] - offs[i];
    }
    if (threadIdx.x == 0) {
        expert_offsets[L] = R;
        totals[0] = R;
        totals[1] = U;
    }
    // Sources whose first token is past the end (the last entry, or every
    // entry when Ts == 0) start at U; the scatter writes the others.
    for (int s = threadIdx.x; s <= S; s += kScanThreads)
        if ((int64_t)s * Ts >= (int64_t)S * Ts) src_slot_offsets[s] = U;
}

// ------------------------------------------------------------------ scatter
__global__ void __launch_bounds__(kBlock)
layout_scatter_kernel(const int32_t* __restrict__ ids, int64_t T, int k, int e0, int L,
                      int CT, int NC, int64_t Ts, const int32_t* __restrict__ base,
                      const int32_t* __restrict__ slot_base, int32_t* __restrict__ row_slot,
                      int32_t* __restrict__ row_assign, int32_t* __restrict__ assign_row,
                      int32_t* __restrict__ tok_slot, int32_t* __restrict__ slot_tok,
                      int32_t* __restrict__ src_slot_offsets) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int wave = threadIdx.x / MOE_WAVE;
    const int lane = threadIdx.x % MOE_WAVE;
    const int c = blockIdx.x * kWaves + wave;
    uint64_t* mask = reinterpret_cast<uint64_t*>(smem) + wave * L;
    int* cnt = reinterpret_cast<int*>(smem + kWaves * L * 8) + wave * L;
    int* tslot = reinterpret_cast<int*>(smem + kWaves * L * 12) + wave * CT;
    unsigned char* flag = smem + kWaves * (L * 12 + CT * 4) + wave * CT;

    const int64_t t0 = (int64_t)c * CT;
    const int64_t t1 = c < NC ? min(T, t0 + CT) : t0;
    for (int i = lane; i < L; i += MOE_WAVE) {
        mask[i] = 0;
        cnt[i] = c < NC ? base[(int64_t)c * L + i] : 0;
    }
    for (int i = lane; i < CT; i += MOE_WAVE) flag[i] = 0;
    __syncthreads();

    // landed flags
    for (int64_t a = t0 * k + lane; a < t1 * k; a += MOE_WAVE) {
        const int le = ids[a] - e0;
        if ((unsigned)le < (unsigned)L) flag[a / k - t0] = 1;
    }
    __syncthreads();

    // slots: landed tokens numbered in ascending token order
    int running = c < NC ? slot_base[c] : 0;
    for (int64_t tb = t0; tb < t1; tb += MOE_WAVE) {
        const int64_t t = tb + lane;
        const bool in = t < t1;
        const bool f = in && flag[t - t0];
        const uint64_t bal = __ballot(f);
        const int slot = running + __popcll(bal & moe::lanemask_lt());
        if (in) {
            if (f) {
                tok_slot[t] = slot;
                if (slot < T) slot_tok[slot] = (int32_t)t;     // slots_cap = T
                tslot[t - t0] = slot;
            } else {
                tok_slot[t] = -1;
            }
            if (Ts > 0 && t % Ts == 0) src_slot_offsets[t / Ts] = slot;
        }
        running += __popcll(bal);
    }
    __syncthreads();

    // rows: stable rank of each local assignment within its expert
    for (int64_t ab = t0 * k; ab < t1 * k; ab += MOE_WAVE) {
        const int64_t a = ab + lane;
        const bool valid = a < t1 * k;
        const int le = valid ? ids[a] - e0 : -1;
        const bool loc = valid && (unsigned)le < (unsigned)L;
        if (loc) atomicOr(reinterpret_cast<unsigned long long*>(&mask[le]), 1ull << lane);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
        const uint64_t m = loc ? mask[le] : 0ull;
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
        const int rank = __popcll(m & moe::lanemask_lt());
        const int leader = loc ? (__ffsll((unsigned long long)m) - 1) : lane;
        int b = 0;
        if (loc && leader == lane) {
            b = cnt[le];
            cnt[le] = b + __popcll(m);
            mask[le] = 0ull;
        }
        b = __shfl(b, leader, MOE_WAVE);
        if (loc) {
            const int row = b + rank;
            if ((int64_t)row < T * k) {                        // rows_cap = T*k
                row_assign[row] = (int32_t)a;
                row_slot[row] = tslot[a / k - t0];
            }
            assign_row[a] = row;
        } else if (valid) {
            assign_row[a] = -1;
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
}

}  // namespace

extern "C" moe_status moe_capacity(const moe_dims* dims, int64_t* rows_cap, int64_t* slots_cap) {
    Dims d;
    moe_status st = moe::load_dims(dims, &d, false);
    if (st != MOE_OK) return st;
    if (!rows_cap || !slots_cap) return MOE_ERR_INVALID_ARG;
    *rows_cap = d.T * d.k;
    *slots_cap = d.T;
    return MOE_OK;
}

extern "C" moe_status moe_route_layout_workspace(const moe_dims* dims, size_t* bytes) {
    Dims d;
    moe_status st = moe::load_dims(dims, &d, false);
    if (st != MOE_OK) return st;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    if (d.L > kMaxLocalExperts) return MOE_ERR_UNSUPPORTED;
    *bytes = (size_t)make_plan(d).total_ints * 4;
    return MOE_OK;
}

extern "C" moe_status moe_route_layout(const moe_dims* dims, const int32_t* topk_ids,
                                       int32_t* expert_counts, int32_t* expert_offsets,
                                       int32_t* row_slot, int32_t* row_assign, int32_t* assign_row,
                                       int32_t* tok_slot, int32_t* slot_tok,
                                       int32_t* src_slot_offsets, int32_t* totals, void* ws,
                                       size_t ws_bytes, void* hip_stream) {
    Dims d;
    moe_status st = moe::load_dims(dims, &d, false);
    if (st != MOE_OK) return st;
    if (d.L > kMaxLocalExperts) return MOE_ERR_UNSUPPORTED;
    if (!expert_counts || !expert_offsets || !src_slot_offsets || !totals) return MOE_ERR_INVALID_ARG;
    if (d.T > 0 && (!topk_ids || !row_slot || !row_assign || !assign_row || !tok_slot || !slot_tok))
        return MOE_ERR_INVALID_ARG;
    const Plan p = make_plan(d);
    if (!ws || ws_bytes < (size_t)p.total_ints * 4) return MOE_ERR_WORKSPACE;
    hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
    int32_t* w = reinterpret_cast<int32_t*>(ws);
    int32_t* hist = w + p.off_hist;
    int32_t* base = w + p.off_base;
    int32_t* landed = w + p.off_landed;
    int32_t* slot_base = w + p.off_slot;
    const int grid = (int)((p.NC + kWaves - 1) / kWaves);

    if (grid > 0) {
        hipLaunchKernelGGL(layout_count_kernel, dim3(grid), dim3(kBlock), count_lds(d, p), stream,
                           topk_ids, d.T, (int)d.k, (int)d.e0, (int)d.L, (int)p.CT, (int)p.NC,
                           hist, landed);
        if ((st = moe::launch_status()) != MOE_OK) return st;
    }
    hipLaunchKernelGGL(layout_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, hist, landed,
                       (int)d.L, (int)p.NC, (int)d.S, d.Ts, base, slot_base, expert_counts,
                       expert_offsets, src_slot_offsets, totals);
    if ((st = moe::launch_status()) != MOE_OK) return st;
    if (grid > 0) {
        hipLaunchKernelGGL(layout_scatter_kernel, dim3(grid), dim3(kBlock), scatter_lds(d, p), stream,
                           topk_ids, d.T, (int)d.k, (int)d.e0, (int)d.L, (int)p.CT, (int)p.NC, d.Ts,
                           base, slot_base, row_slot, row_assign, assign_row, tok_slot, slot_tok,
                           src_slot_offsets);
        if ((st = moe::launch_status()) != MOE_OK) return st;
    }
    return MOE_OK;
}
