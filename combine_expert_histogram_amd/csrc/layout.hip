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
// Two launches, no grid-wide barrier (a grid barrier needs co-residency, and
// on gfx950 a cross-workgroup release/acquire writes back / invalidates the
// whole L2, "cut the whole-L2 cache operations" commit of the same PR):
//   count - one workgroup per chunk of CB tokens: the chunk's per-expert
//           histogram (LDS atomics; order does not matter for counts) and its
//           landed-token count, written expert-major to the workspace.
//   place - one workgroup per chunk again.  It reads the whole histogram
//           (at most ~32K ints) to get, per expert, the rows of
//           all earlier chunks and the expert totals, so no separate scan
//           launch is needed; then each of its four wavefronts ranks the local
//           assignments of its quarter of the chunk.  A pass takes 64
//           consecutive assignments; lanes with the same expert find each
//           other by OR-ing their lane bit into a per-expert 64-bit mask in
//           LDS (ds_or_b64), so a pass costs a fixed handful of LDS round trips
//           whatever the number of distinct experts in it.
#include "common.h"

#include <mutex>

namespace {

using moe::Dims;

constexpr int kBlock = 256;                       // 4 wavefronts
constexpr int kWaves = kBlock / MOE_WAVE;
constexpr int64_t kHistTarget = 32768;            // histogram entries aimed for
constexpr int kMaxLocalExperts = 1024;
constexpr int kHistBatch = 16;                    // histogram loads a thread keeps in flight
constexpr int kIdPasses = 4;                      // routing-id passes a wavefront holds in registers
constexpr int kCountBatch = 8;                    // routing ids a count thread loads before its atomics

struct Plan {
    int64_t CB = 64;   // tokens per chunk (one workgroup)
    int64_t NC = 0;    // chunks
    int64_t NCp = 0;   // histogram row stride: NC rounded up to 4 (16 B rows)
    int64_t off_hist = 0, off_landed = 0, total_ints = 0;   // workspace, int32 units
};

Plan make_plan(const Dims& d) {
    Plan p;
    const int64_t cap = d.L > 512 ? 512 : 2048;   // keeps the place kernel under 64 KB LDS
    auto nchunks = [&](int64_t cb) { return (d.T + cb - 1) / cb; };
    while (nchunks(p.CB) * d.L > kHistTarget && p.CB < cap) p.CB *= 2;
    p.NC = nchunks(p.CB);
    p.NCp = (p.NC + 3) & ~int64_t(3);
    auto al = [](int64_t v) { return (v + 63) & ~int64_t(63); };   // 256-byte alignment
    p.off_hist = 0;
    p.off_landed = al(d.L * p.NCp);
    p.total_ints = al(p.off_landed + p.NC);
    return p;
}

size_t count_lds(const Dims& d, const Plan& p) { return d.L * 4 + p.CB + 64; }

// place kernel LDS: mask[4][L] u64 | wcnt[4][L] | A[L] | Tt[L] | offs[L+1] | misc[16] |
//                   tslot[CB] | flag[CB]
struct PlaceLds {
    size_t mask, wcnt, A, Tt, offs, misc, tslot, flag, total;
};
__host__ __device__ PlaceLds place_lds(int64_t L, int64_t CB) {
    PlaceLds o;
    o.mask = 0;
    o.wcnt = o.mask + kWaves * L * 8;
    o.A = o.wcnt + kWaves * L * 4;
    o.Tt = o.A + L * 4;
    o.offs = o.Tt + L * 4;
    o.misc = o.offs + (L + 1) * 4;
    o.tslot = (o.misc + 16 * 4 + 15) & ~size_t(15);
    o.flag = o.tslot + CB * 4;
    o.total = o.flag + CB;
    return o;
}

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// ------------------------------------------------------------------ count
__global__ void __launch_bounds__(kBlock)
layout_count_kernel(const int32_t* __restrict__ ids, int64_t T, int k, int e0, int L, int CB,
                    int NCp, int32_t* __restrict__ hist, int32_t* __restrict__ landed) {
    MOE_TRACE_T0(tr0);
    extern __shared__ __align__(16) unsigned char smem[];
    int* cnt = reinterpret_cast<int*>(smem);
    int* red = cnt + L;                                   // 16 ints
    unsigned char* flag = reinterpret_cast<unsigned char*>(red + 16);
    const int tid = threadIdx.x;
    const int c = blockIdx.x;
    for (int i = tid; i < L; i += kBlock) cnt[i] = 0;
    for (int i = tid; i < CB; i += kBlock) flag[i] = 0;
    __syncthreads();

    const int64_t t0 = (int64_t)c * CB;
    const int64_t t1 = min(T, t0 + CB);
    // a thread's ids are loaded kCountBatch at a time before their atomics, so
    // the batch costs one memory round trip
    const int64_t b0 = t0 * k, b1 = t1 * k;
    for (int64_t base = b0; base < b1; base += (int64_t)kBlock * kCountBatch) {
        int v[kCountBatch];
#pragma unroll
        for (int u = 0; u < kCountBatch; ++u) {
            const int64_t a = base + u * kBlock + tid;
            v[u] = a < b1 ? ids[a] : 0;
        }
#pragma unroll
        for (int u = 0; u < kCountBatch; ++u) {
            const int64_t a = base + u * kBlock + tid;
            const int le = v[u] - e0;
            if (a < b1 && (unsigned)le < (unsigned)L) {
                atomicAdd(&cnt[le], 1);
                flag[(int)(a / k - t0)] = 1;
            }
        }
    }
    __syncthreads();
    int nl = 0;
    for (int i = tid; i < (int)(t1 - t0); i += kBlock) nl += flag[i];
    nl = moe::wave_sum(nl);
    if (tid % MOE_WAVE == 0) red[tid / MOE_WAVE] = nl;
    for (int i = tid; i < L; i += kBlock) hist[(int64_t)i * NCp + c] = cnt[i];
    __syncthreads();
    if (tid == 0) landed[c] = red[0] + red[1] + red[2] + red[3];
    if (tid == 0) MOE_TRACE_PUT(moe::kTrLayoutCount, blockIdx.x, 0, 0, tr0);
}

// ------------------------------------------------------------------ place
__global__ void __launch_bounds__(kBlock)
layout_place_kernel(const int32_t* __restrict__ ids, int64_t T, int k, int e0, int L, int CB,
                    int NC, int NCp, int S, int64_t Ts, const int32_t* __restrict__ hist,
                    const int32_t* __restrict__ landed, int32_t* __restrict__ expert_counts,
                    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ row_slot,
                    int32_t* __restrict__ row_assign, int32_t* __restrict__ assign_row,
                    int32_t* __restrict__ tok_slot, int32_t* __restrict__ slot_tok,
                    int32_t* __restrict__ src_slot_offsets, int32_t* __restrict__ totals) {
    MOE_TRACE_T0(tr0);
    extern __shared__ __align__(16) unsigned char smem[];
    const PlaceLds lo = place_lds(L, CB);
    const int tid = threadIdx.x;
    const int wave = tid / MOE_WAVE;
    const int lane = tid % MOE_WAVE;
    const int c = blockIdx.x;                              // may be >= NC when T == 0
    uint64_t* mask = reinterpret_cast<uint64_t*>(smem + lo.mask) + wave * L;
    int* wcnt_all = reinterpret_cast<int*>(smem + lo.wcnt);
    int* wcnt = wcnt_all + wave * L;
    int* A = reinterpret_cast<int*>(smem + lo.A);          // rows of this expert in chunks < c
    int* Tt = reinterpret_cast<int*>(smem + lo.Tt);        // expert totals
    int* offs = reinterpret_cast<int*>(smem + lo.offs);
    int* misc = reinterpret_cast<int*>(smem + lo.misc);    // [0] slots before c, [1] U, [4..8) wave landed
    int* tslot = reinterpret_cast<int*>(smem + lo.tslot);
    unsigned char* flag = smem + lo.flag;

    for (int i = tid; i < L; i += kBlock) {
        A[i] = 0;
        Tt[i] = 0;
    }
    for (int i = tid; i < kWaves * L; i += kBlock) {
        wcnt_all[i] = 0;
        reinterpret_cast<uint64_t*>(smem + lo.mask)[i] = 0ull;
    }
    for (int i = tid; i < CB; i += kBlock) flag[i] = 0;
    if (tid < 16) misc[tid] = 0;

    // this chunk's tokens; wave `wave` owns tokens [tw0, tw1), i.e. assignments
    // [a0, a1), taken 64 at a time (pass p: assignment a0 + 64 p + lane)
    const int64_t t0 = (int64_t)c * CB;
    const int64_t t1 = c < NC ? min(T, t0 + CB) : t0;
    const int CW = CB / kWaves;
    const int64_t tw0 = min(t1, t0 + (int64_t)wave * CW);
    const int64_t tw1 = min(t1, tw0 + CW);
    const int64_t a0 = tw0 * k, a1 = tw1 * k;
    const int npass = (int)((a1 - a0 + MOE_WAVE - 1) / MOE_WAVE);
    // the first kIdPasses passes' routing ids, loaded now so that their memory
    // round trip overlaps the histogram reads (phases 2 and 5 use them; later
    // passes read ids again there)
    int idr[kIdPasses];
#pragma unroll
    for (int p = 0; p < kIdPasses; ++p) {
        const int64_t a = a0 + p * MOE_WAVE + lane;
        idr[p] = a < a1 ? ids[a] : 0;
    }
    __syncthreads();

    // (1) prefix information from the histogram: the rows of all earlier chunks
    // (A) and the expert's total (Tt).  The histogram was written by the count
    // launch, on every XCD, so these reads miss this XCD's L2; each costs a full
    // memory round trip.  An expert's row (NCp / 4 int4) is therefore split over
    // tpe consecutive lanes that issue their loads together (a thread's loads in
    // batches of kHistBatch), and the lanes' sums are joined by shuffles: with
    // L = 32 every load of the phase is in flight at once instead of eight
    // dependent batches per expert.
    {
        const int Q = NCp / 4;
        int tpe = 1;                                       // lanes per expert: a power of two <= 64
        while (tpe < MOE_WAVE && tpe * 2 * L <= kBlock && tpe < Q) tpe *= 2;
        const int sub = tid & (tpe - 1);
        for (int le0 = 0; le0 < L; le0 += kBlock / tpe) {  // same trip count in every thread
            const int le = le0 + tid / tpe;
            int sa = 0, st = 0;
            if (le < L) {
                const int4* row = reinterpret_cast<const int4*>(hist + (int64_t)le * NCp);
                for (int q0 = sub; q0 < Q; q0 += kHistBatch * tpe) {
                    int4 v[kHistBatch];
#pragma unroll
                    for (int u = 0; u < kHistBatch; ++u) {
                        const int qq = q0 + u * tpe;
                        v[u] = qq < Q ? row[qq] : int4{0, 0, 0, 0};
                    }
#pragma unroll
                    for (int u = 0; u < kHistBatch; ++u) {
                        const int cc = (q0 + u * tpe) * 4;
                        const int e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                        for (int z = 0; z < 4; ++z) {
                            const int val = cc + z < NC ? e[z] : 0;     // stride padding is not written
                            st += val;
                            if (cc + z < c) sa += val;
                        }
                    }
                }
            }
            for (int off = tpe / 2; off > 0; off >>= 1) {
                sa += __shfl_xor(sa, off, MOE_WAVE);
                st += __shfl_xor(st, off, MOE_WAVE);
            }
            if (le < L && sub == 0) {
                A[le] = sa;
                Tt[le] = st;
            }
        }
        int lb = 0, lt = 0;
        for (int j = tid; j < NC; j += kBlock) {
            const int v = landed[j];
            lt += v;
            if (j < c) lb += v;
        }
        lb = moe::wave_sum(lb);
        lt = moe::wave_sum(lt);
        if (lane == 0) {
            if (lb) atomicAdd(&misc[0], lb);
            if (lt) atomicAdd(&misc[1], lt);
        }
    }

    // (2) this wave's per-expert counts and the chunk's landed flags
    auto count_one = [&](int64_t a, int id) __attribute__((always_inline)) {
        const int le = id - e0;
        if (a < a1 && (unsigned)le < (unsigned)L) {
            atomicAdd(&wcnt[le], 1);
            flag[(int)(a / k - t0)] = 1;
        }
    };
#pragma unroll
    for (int p = 0; p < kIdPasses; ++p)
        if (p < npass) count_one(a0 + p * MOE_WAVE + lane, idr[p]);
    for (int p = kIdPasses; p < npass; ++p) {
        const int64_t a = a0 + p * MOE_WAVE + lane;
        count_one(a, a < a1 ? ids[a] : 0);
    }
    __syncthreads();

    // (3) expert offsets; per-wave first row of each expert; slot bases
    if (wave == 0) {
        int carry = 0;
        for (int b = 0; b < L; b += MOE_WAVE) {
            const int e = b + lane;
            const int v = e < L ? Tt[e] : 0;
            const int incl = moe::wave_inclusive_scan(v);
            if (e < L) offs[e] = carry + incl - v;
            carry += __shfl(incl, MOE_WAVE - 1, MOE_WAVE);
        }
        if (lane == 0) offs[L] = carry;
    } else if (wave == 1) {
        for (int w = 0; w < kWaves; ++w) {
            const int64_t a0 = min(t1, t0 + (int64_t)w * CW), a1 = min(t1, a0 + CW);
            int cntw = 0;
            for (int64_t t = a0 + lane; t < a1; t += MOE_WAVE) cntw += flag[(int)(t - t0)];
            cntw = moe::wave_sum(cntw);
            if (lane == 0) misc[4 + w] = cntw;
        }
    }
    __syncthreads();
    for (int le = tid; le < L; le += kBlock) {
        int run = offs[le] + A[le];
        for (int w = 0; w < kWaves; ++w) {
            const int v = wcnt_all[w * L + le];
            wcnt_all[w * L + le] = run;
            run += v;
        }
    }
    const int R = offs[L];
    const int U = misc[1];
    if (c == 0) {
        for (int le = tid; le < L; le += kBlock) {
            expert_offsets[le] = offs[le];
            expert_counts[le] = Tt[le];
        }
        if (tid == 0) {
            expert_offsets[L] = R;
            totals[0] = R;
            totals[1] = U;
        }
        for (int s = tid; s <= S; s += kBlock)
            if ((int64_t)s * Ts >= T) src_slot_offsets[s] = U;   // sources starting at the end
    }
    __syncthreads();

    // (4) slots of this wave's tokens, ascending token order
    int running = misc[0];
    for (int w = 0; w < wave; ++w) running += misc[4 + w];
    for (int64_t tb = tw0; tb < tw1; tb += MOE_WAVE) {
        const int64_t t = tb + lane;
        const bool in = t < tw1;
        const bool f = in && flag[(int)(t - t0)];
        const uint64_t bal = __ballot(f);
        const int slot = running + __popcll(bal & moe::lanemask_lt());
        if (in) {
            if (f) {
                tok_slot[t] = slot;
                if (slot < T) slot_tok[slot] = (int32_t)t;     // slots_cap = T
                tslot[(int)(t - t0)] = slot;
            } else {
                tok_slot[t] = -1;
            }
            if (Ts > 0 && t % Ts == 0) src_slot_offsets[t / Ts] = slot;
        }
        running += __popcll(bal);
    }
    wave_sync_lds();

    // (5) rows: stable rank of each local assignment within its expert
    auto place_one = [&](int64_t a, int id) __attribute__((always_inline)) {
        const bool valid = a < a1;
        const int le = valid ? id - e0 : -1;
        const bool loc = valid && (unsigned)le < (unsigned)L;
        if (loc) atomicOr(reinterpret_cast<unsigned long long*>(&mask[le]), 1ull << lane);
        wave_sync_lds();
        const uint64_t m = loc ? mask[le] : 0ull;
        wave_sync_lds();
        const int rank = __popcll(m & moe::lanemask_lt());
        const int leader = loc ? (__ffsll((unsigned long long)m) - 1) : lane;
        int b = 0;
        if (loc && leader == lane) {
            b = wcnt[le];
            wcnt[le] = b + __popcll(m);
            mask[le] = 0ull;
        }
        b = __shfl(b, leader, MOE_WAVE);
        if (loc) {
            const int row = b + rank;
            if ((int64_t)row < T * k) {                        // rows_cap = T*k
                row_assign[row] = (int32_t)a;
                row_slot[row] = tslot[(int)(a / k - t0)];
            }
            assign_row[a] = row;
        } else if (valid) {
            assign_row[a] = -1;
        }
        wave_sync_lds();
    };
#pragma unroll
    for (int p = 0; p < kIdPasses; ++p)
        if (p < npass) place_one(a0 + p * MOE_WAVE + lane, idr[p]);
    for (int p = kIdPasses; p < npass; ++p) {
        const int64_t a = a0 + p * MOE_WAVE + lane;
        place_one(a, a < a1 ? ids[a] : 0);
    }
    if (tid == 0) MOE_TRACE_PUT(moe::kTrLayoutPlace, blockIdx.x, 0, 0, tr0);
}

// Validates the layout call's arguments and sizes its plan; no HIP call.
moe_status check_layout(const moe_dims* dims, const int32_t* topk_ids, int32_t* expert_counts,
                        int32_t* expert_offsets, int32_t* row_slot, int32_t* row_assign, int32_t* assign_row,
                        int32_t* tok_slot, int32_t* slot_tok, int32_t* src_slot_offsets, int32_t* totals,
                        Dims* d, Plan* p) {
    moe_status st = moe::load_dims(dims, d, false);
    if (st != MOE_OK) return st;
    if (d->L > kMaxLocalExperts) return MOE_ERR_UNSUPPORTED;
    if (!expert_counts || !expert_offsets || !src_slot_offsets || !totals) return MOE_ERR_INVALID_ARG;
    if (d->T > 0 && (!topk_ids || !row_slot || !row_assign || !assign_row || !tok_slot || !slot_tok))
        return MOE_ERR_INVALID_ARG;
    *p = make_plan(*d);
    if (p->NCp * d->L >= INT32_MAX) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// The two launches on `stream`, with the histogram and landed counts in ws.
moe_status launch_layout(const Dims& d, const Plan& p, const int32_t* topk_ids, int32_t* expert_counts,
                         int32_t* expert_offsets, int32_t* row_slot, int32_t* row_assign, int32_t* assign_row,
                         int32_t* tok_slot, int32_t* slot_tok, int32_t* src_slot_offsets, int32_t* totals,
                         int32_t* ws, hipStream_t stream) {
    moe_status st;
    int32_t* hist = ws + p.off_hist;
    int32_t* landed = ws + p.off_landed;
    if (p.NC > 0) {
        hipLaunchKernelGGL(layout_count_kernel, dim3((unsigned)p.NC), dim3(kBlock), count_lds(d, p),
                           stream, topk_ids, d.T, (int)d.k, (int)d.e0, (int)d.L, (int)p.CB, (int)p.NCp,
                           hist, landed);
        if ((st = moe::launch_status()) != MOE_OK) return st;
    }
    // at least one workgroup, so that T == 0 still writes the counts and totals
    const unsigned grid = (unsigned)std::max<int64_t>(p.NC, 1);
    hipLaunchKernelGGL(layout_place_kernel, dim3(grid), dim3(kBlock), place_lds(d.L, p.CB).total,
                       stream, topk_ids, d.T, (int)d.k, (int)d.e0, (int)d.L, (int)p.CB, (int)p.NC,
                       (int)p.NCp, (int)d.S, d.Ts, hist, landed, expert_counts, expert_offsets, row_slot,
                       row_assign, assign_row, tok_slot, slot_tok, src_slot_offsets, totals);
    return moe::launch_status();
}

// ------------------------------------------------ allocation-free variant
// The layout's workspace (the per-chunk histogram and landed counts) in a
// static device array instead of a caller-provided buffer, for callers that
// cannot allocate.  Every GPU the library runs on holds its own copy of the
// array until the process ends.  It needs no clearing between calls: the count
// launch writes every histogram entry and landed count that the place launch
// reads (the histogram's row padding is never read).
constexpr int64_t kScratchInts = 65536;                   // 256 KiB
static __device__ __align__(256) int32_t scratch[kScratchInts];

// Device address of `scratch` on each device, looked up once per device with
// that device current.  In host code `scratch` names a host-side stand-in, so
// kernels only ever receive these addresses.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices] = {};

moe_status scratch_address(int32_t** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
        g_scratch_addr[dev] = p;
    }
    *out = static_cast<int32_t*>(g_scratch_addr[dev]);
    return MOE_OK;
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
    Plan p;
    moe_status st = check_layout(dims, topk_ids, expert_counts, expert_offsets, row_slot, row_assign, assign_row,
                                 tok_slot, slot_tok, src_slot_offsets, totals, &d, &p);
    if (st != MOE_OK) return st;
    if (!ws || ws_bytes < (size_t)p.total_ints * 4) return MOE_ERR_WORKSPACE;
    return launch_layout(d, p, topk_ids, expert_counts, expert_offsets, row_slot, row_assign, assign_row, tok_slot,
                         slot_tok, src_slot_offsets, totals, reinterpret_cast<int32_t*>(ws),
                         reinterpret_cast<hipStream_t>(hip_stream));
}

extern "C" moe_status moe_route_layout_noalloc(const moe_dims* dims, const int32_t* topk_ids,
                                               int32_t* expert_counts, int32_t* expert_offsets,
                                               int32_t* row_slot, int32_t* row_assign, int32_t* assign_row,
                                               int32_t* tok_slot, int32_t* slot_tok,
                                               int32_t* src_slot_offsets, int32_t* totals, void* hip_stream) {
    Dims d;
    Plan p;
    moe_status st = check_layout(dims, topk_ids, expert_counts, expert_offsets, row_slot, row_assign, assign_row,
                                 tok_slot, slot_tok, src_slot_offsets, totals, &d, &p);
    if (st != MOE_OK) return st;
    if (p.total_ints > kScratchInts) return MOE_ERR_WORKSPACE;   // the static array is too small
    int32_t* ws = nullptr;
    if ((st = scratch_address(&ws)) != MOE_OK) return st;
    return launch_layout(d, p, topk_ids, expert_counts, expert_offsets, row_slot, row_assign, assign_row, tok_slot,
                         slot_tok, src_slot_offsets, totals, ws, reinterpret_cast<hipStream_t>(hip_stream));
}
