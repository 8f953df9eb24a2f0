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
// K = 128), folded into the fp32 running sum by one FMA with sA[row] * sW.
// The MFMA computes the transposed sub-tile (weight rows as its A operand), so
// a lane holds 4 consecutive output columns of one row: one row scale per lane
// and sub-tile row, and 8 contiguous output bytes per lane in the epilogue.
//
// Tile: BM rows of one expert x 256 columns, eight wavefronts (two per SIMD)
// in a WM x WN grid, each owning 64 x (256/WN) = 4 x NJ sub-tiles.  Two
// shapes are built: 128 x 256 with a 3-stage K ring, and 256 x 256 with a
// 2-stage ring (fewer operand bytes per MAC; the 160 KB LDS holds two of its
// 66 KB stages).
//
// Operand staging: K blocks stream through the LDS ring, filled by
// global_load_lds_dwordx4 (memory straight to LDS, no staging registers); a
// stage is waited for with an explicit vmcnt.  Each lane of a direct-to-LDS
// load lands at base + 16 * lane; the swizzle of the 16 B chunks inside a
// 128 B row (chunk c of row r sits in slot c ^ (r & 7) ^ ((r >> 3) & 1)) is made
// by choosing which global chunk each lane fetches: 16 consecutive rows read
// at one chunk then hit 16 distinct 16 B bank groups of a 256 B window (and 8
// distinct ones of a 128 B window).
//
// Overlap: the operand loads are bounded by the number of L2 requests a CU can
// keep in flight, so a wavefront that issued all of a stage's loads at once
// would stall at the issue until the queue drains, with its MFMAs waiting
// behind.  The loads of the next stage are therefore spread between the MFMA
// groups of the current K step.
//
// The ring stages are distinct LDS objects and the K loop is unrolled by the
// stage count, so each step reads one stage and fills another by name: the
// compiler can then prove that the operand reads do not alias the loads in
// flight into the other stages and keeps only the explicit waits.
//
// Row scales: the rows of a tile are gathered, so their scales would cost one
// scattered 4 B request per row and K block.  A pre-pass writes the scales
// into a K-block-major table indexed by expert-major row (the caller's
// workspace), and a stage reads its row scales as one contiguous piece per
// wavefront.
//
// Scheduling: one persistent workgroup per CU walks the tile table (experts
// in order; per expert, column tiles outer and row tiles inner, so the row
// tiles that share a weight slab are adjacent) derived on the device from
// expert_offsets.  Consecutive tile ids go to workgroups of the same XCD
// (workgroup b runs on XCD b % 8), so the row tiles sharing a weight slab
// meet in that XCD's L2.  A wavefront whose 64 rows all lie past the expert's
// last row skips its MFMAs, so a final partial row tile costs accordingly less.
#include "common.h"

#include <type_traits>

#ifndef MOE_GEMM1_SPAN
#define MOE_GEMM1_SPAN 64
#endif
// cache-policy bits of the operand loads (0: default)
#ifndef MOE_GEMM1_AUXA
#define MOE_GEMM1_AUXA 0
#endif
#ifndef MOE_GEMM1_AUXB
#define MOE_GEMM1_AUXB 0
#endif
#ifndef MOE_GEMM1_KROT_M
#define MOE_GEMM1_KROT_M 0
#endif
#ifndef MOE_GEMM1_KROT_N
#define MOE_GEMM1_KROT_N 0
#endif

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
using moe::u32x4;

constexpr int BN = 256, BK = 128;
constexpr int kMaxL = 1024;
constexpr int kXcds = 8;
constexpr int kMinBM = 128;   // tile descriptors are sized for the smallest row tile

template <int BM_, int WM_, int WN_, int NSTAGE_, int LAG_>
struct Cfg {
    static constexpr int BM = BM_, WM = WM_, WN = WN_, NSTAGE = NSTAGE_;
    static constexpr int LAG = LAG_;   // column groups between an MFMA and the fold of its product
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = kWaves * MOE_WAVE;
    static constexpr int RW = BM / WM, CW = BN / WN;              // rows / columns of a wavefront
    static constexpr int MI = RW / 16, NJ = CW / 16;
    // the next stage's loads are spread over the first SPAN column groups of a step
    static constexpr int SPAN = MOE_GEMM1_SPAN < 1 ? 1 : (MOE_GEMM1_SPAN > NJ ? NJ : MOE_GEMM1_SPAN);
    static constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
    static constexpr int S_ROWS = BM / kWaves;                     // row scales loaded per wavefront
    static constexpr int S_BYTES = kWaves * 256;                   // one 256 B slot per wavefront
    static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
    static constexpr int A_LOADS = A_BYTES / (16 * 64 * kWaves);   // per wavefront per stage
    static constexpr int B_LOADS = B_BYTES / (16 * 64 * kWaves);
    static constexpr int STAGE_LOADS = A_LOADS + B_LOADS + 1;
    static_assert(RW % 16 == 0 && CW % 16 == 0, "wavefront tiles are whole 16 x 16 sub-tiles");
    static_assert(A_BYTES % (1024 * kWaves) == 0 && B_BYTES % (1024 * kWaves) == 0 && A_LOADS >= 1 &&
                      B_LOADS >= 1, "every wavefront issues the same whole number of 1 KB loads");
    static_assert(kThreads <= 1024 && BM >= kMinBM, "workgroup size, descriptor capacity");
    static_assert(CW <= 128 && 128 % CW == 0, "a wavefront's columns share one weight scale");
    static_assert(S_ROWS >= 1 && S_ROWS <= 64 && BM % kWaves == 0, "row scales split over wavefronts");
    static_assert(STAGE_LOADS < 64, "vmcnt holds 6 bits");
    static_assert(NSTAGE == 2 || NSTAGE == 3, "two or three ring stages");
    static_assert(LAG >= -1 && LAG <= 1, "products folded at once, in their own group or the next");
    static_assert(NSTAGE * STAGE + BM * 4 <= 160 * 1024, "LDS budget");
};

#define GPTR(p) ((const void __attribute__((address_space(1)))*)(p))
#define LPTR(p) ((void __attribute__((address_space(3)))*)(p))

// s_waitcnt immediate waiting until at most n vector-memory ops are outstanding
// (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14)
constexpr int wait_vm(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14); }

__device__ __forceinline__ void cbarrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <class C>
__global__ void __launch_bounds__(C::kThreads, 1)
grouped_gemm1_kernel(const uint8_t* __restrict__ q, const float* __restrict__ row_scale,
                     const int4* __restrict__ tiles, const int32_t* __restrict__ row_slot,
                     const uint8_t* __restrict__ w, const float* __restrict__ w_scale,
                     uint16_t* __restrict__ y, int N, int H, int64_t T, int64_t scale_ld) {
    constexpr int BM = C::BM, kThreads = C::kThreads, MI = C::MI, NJ = C::NJ;
    constexpr int A_BYTES = C::A_BYTES, B_BYTES = C::B_BYTES, STAGE = C::STAGE;
    constexpr int A_LOADS = C::A_LOADS, B_LOADS = C::B_LOADS, NLOADS = C::STAGE_LOADS;
    constexpr int RW = C::RW, CW = C::CW, WN = C::WN;
    // With S stages, the loads of K block kb+S-1 are issued during step kb; at
    // the top of step kb the ops outstanding are, in issue order, those of the
    // stages kb .. kb+S-2, so "at most (S-2) stages outstanding" means stage kb
    // has landed (loads complete in order).
    constexpr int kWaitSteady = wait_vm((C::NSTAGE - 2) * NLOADS);
    constexpr int kWaitAll = wait_vm(0);

    __shared__ __align__(16) uint8_t stage0[STAGE];
    __shared__ __align__(16) uint8_t stage1[STAGE];
    __shared__ __align__(16) uint8_t stage2[C::NSTAGE == 3 ? STAGE : 16];
    __shared__ int slot_s[BM];

    const int tid = threadIdx.x;
    const int lane = tid % MOE_WAVE;
    const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);
    const int wm = wave / WN, wn = wave % WN;
    const int KB = H / BK;
    const int NB = N / 128;
    const int total = tiles[0].x;
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int my = (b % kXcds) * (G / kXcds) + b / kXcds;   // G is a multiple of 8

    // Direct-to-LDS load gi (of the workgroup) fills LDS chunks gi*64 + l = row
    // gi*8 + l/8, slot l%8, which holds global chunk (l%8) ^ (l/8) ^ (gi & 1).
    const int lrow = lane >> 3;
    const int gchunk = (lane & 7) ^ lrow;

    for (int it = 0;; ++it) {
        const int tile = it * G + my;
        if (tile >= total) break;
        const int4 td = tiles[1 + tile];
        const int e = td.x, nt = td.y, r0 = td.z;
        const int nvalid = td.w & 511, mtile = td.w >> 9;
        const int n0 = nt * BN;
        const int ncols = min(BN, N - n0);            // 256, or 128 for a final half tile
        const bool active = wm * RW < nvalid && wn * CW < ncols;   // wavefront has output
        // K rotation: this tile walks the K blocks starting at kb0 (wrapping), so the
        // tiles that share an operand slab reach each K block at different times and
        // only the first of them waits for the slab's miss in L2
        const int kb0 = (mtile * MOE_GEMM1_KROT_M + nt * MOE_GEMM1_KROT_N) % KB;
        auto phys = [&](int kb) __attribute__((always_inline)) { const int p = kb + kb0; return p >= KB ? p - KB : p; };

        if (tid < BM) {
            int s0 = row_slot[r0];
            if ((uint64_t)s0 >= (uint64_t)T) s0 = 0;
            int s = s0;                       // rows past the expert reuse row 0's slot
            if (tid < nvalid) {
                s = row_slot[r0 + tid];
                if ((uint64_t)s >= (uint64_t)T) s = s0;
            }
            slot_s[tid] = s;
        }
        __syncthreads();

        uint32_t a_off[A_LOADS];
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            const int r = (wave * A_LOADS + i) * 8 + lrow;
            a_off[i] = (uint32_t)slot_s[r] * (uint32_t)H + (gchunk ^ ((wave * A_LOADS + i) & 1)) * 16;
        }
        const uint8_t* wexp = w + ((int64_t)e * N + n0) * H;
        const uint32_t b_lane0 = (uint32_t)lrow * (uint32_t)H + gchunk * 16;
        const uint32_t b_lane1 = (uint32_t)lrow * (uint32_t)H + (gchunk ^ 1) * 16;
        const float* wsc = w_scale + ((int64_t)e * NB + min((n0 + wn * CW) / 128, NB - 1)) * KB;
        // uniform base + per-lane 32-bit offset, so each load takes the scalar-base form
        const float* srow = row_scale + r0 + wave * C::S_ROWS;
        const uint32_t s_lane = (uint32_t)min(lane, C::S_ROWS - 1) * 4u;

        // the idx-th load of stage `kb` into LDS `base` (idx is a compile-time
        // constant after unrolling)
        auto issue_one = [&](int idx, int kb, uint8_t* base) __attribute__((always_inline)) {
            kb = phys(kb);
            if (idx < A_LOADS) {
                const int i = idx;
                __builtin_amdgcn_global_load_lds(GPTR((q + kb * BK) + a_off[i]),
                                                 LPTR(base + (wave * A_LOADS + i) * 1024), 16, 0, MOE_GEMM1_AUXA);
            } else if (idx < A_LOADS + B_LOADS) {
                const int i = idx - A_LOADS;
                // rows past a half tile re-read the first half (their columns are not stored)
                int rb = (wave * B_LOADS + i) * 8;
                if (rb >= ncols) rb -= ncols;
                __builtin_amdgcn_global_load_lds(
                    GPTR((wexp + kb * BK + (uint32_t)rb * (uint32_t)H) + (((wave * B_LOADS + i) & 1) ? b_lane1 : b_lane0)),
                    LPTR(base + A_BYTES + (wave * B_LOADS + i) * 1024), 16, 0, MOE_GEMM1_AUXB);
            } else {
                // row scales of K block kb: wavefront w loads rows [r0 + w*S_ROWS, +S_ROWS)
                // into the first S_ROWS floats of its 256 B slot; its other lanes repeat
                // the last row (same line, no extra request)
                __builtin_amdgcn_global_load_lds(GPTR(reinterpret_cast<const uint8_t*>(srow + kb * scale_ld) + s_lane),
                                                 LPTR(base + A_BYTES + B_BYTES + wave * 256), 4, 0, 0);
            }
        };
        auto issue_all = [&](int kb, uint8_t* base) __attribute__((always_inline)) {
#pragma unroll
            for (int d = 0; d < NLOADS; ++d) issue_one(d, kb, base);
        };

        v4f acc[MI][NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

        // One K step: compute from `cur`; when `fill` is set, the loads of K block
        // kb_fill into `nxt` are spread between the MFMA groups (load d after
        // column group j = d * NJ / NLOADS).
        auto step = [&](int kb, const uint8_t* cur, bool fill, int kb_fill, uint8_t* nxt) __attribute__((always_inline)) {
            const float sw = wsc[phys(kb)];
            const uint8_t* As = cur;
            const uint8_t* Bs = As + A_BYTES;
            const float* Ss = reinterpret_cast<const float*>(Bs + B_BYTES);   // per-wavefront scale slots
            v8i af[MI];
            float f[MI];
            if (active) {
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    const int row = wm * RW + i * 16 + (lane & 15);
                    const int c0 = (lane >> 4) * 2;
                    const int sw_r = (row & 7) ^ ((row >> 3) & 1);
                    const u32x4 a0 = *reinterpret_cast<const u32x4*>(As + row * BK + ((c0 ^ sw_r) << 4));
                    const u32x4 a1 = *reinterpret_cast<const u32x4*>(As + row * BK + (((c0 + 1) ^ sw_r) << 4));
                    af[i] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                    f[i] = Ss[(row / C::S_ROWS) * 64 + row % C::S_ROWS] * sw;
                }
            }
            // B fragment of column group j, read from LDS
            auto read_b = [&](int j) __attribute__((always_inline)) {
                const int col = wn * CW + j * 16 + (lane & 15);
                const int c0 = (lane >> 4) * 2;
                const int sw_c = (col & 7) ^ ((col >> 3) & 1);
                const u32x4 b0 = *reinterpret_cast<const u32x4*>(Bs + col * BK + ((c0 ^ sw_c) << 4));
                const u32x4 b1 = *reinterpret_cast<const u32x4*>(Bs + col * BK + (((c0 + 1) ^ sw_c) << 4));
                return v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
            };
            // The products of a column group's MFMAs are folded into the running sums
            // after all of the group's MFMAs are issued (LAG 0) or one group later
            // (LAG 1), so a wavefront does not wait on each MFMA's own result.
            v4f pp[MI];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                if (C::LAG < 0 && active) {
                    // fold each product at once (four registers of products; the other
                    // wavefronts of the SIMD cover the MFMA latency)
                    const v8i bf = read_b(j);
#pragma unroll
                    for (int i = 0; i < MI; ++i) {
                        const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            bf, af[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[i][j][v] = fmaf(p[v], f[i], acc[i][j][v]);
                    }
                } else if (active) {
                    const v8i bf = read_b(j);
                    v4f pc[MI];
#pragma unroll
                    for (int i = 0; i < MI; ++i)
                        // transposed sub-tile: lane l holds row (l & 15), columns 4*(l >> 4) + v
                        pc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            bf, af[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                    if constexpr (C::LAG == 0) {
#pragma unroll
                        for (int i = 0; i < MI; ++i)
#pragma unroll
                            for (int v = 0; v < 4; ++v) acc[i][j][v] = fmaf(pc[i][v], f[i], acc[i][j][v]);
                    } else {
                        if (j > 0) {
#pragma unroll
                            for (int i = 0; i < MI; ++i)
#pragma unroll
                                for (int v = 0; v < 4; ++v)
                                    acc[i][j - 1][v] = fmaf(pp[i][v], f[i], acc[i][j - 1][v]);
                        }
#pragma unroll
                        for (int i = 0; i < MI; ++i) pp[i] = pc[i];
                    }
                }
                if (fill) {
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int d = 0; d < NLOADS; ++d)
                        if (d * C::SPAN / NLOADS == j) issue_one(d, kb_fill, nxt);
                }
                // column groups stay in order: no operand reads hoisted across them
                if (C::kWaves > 8) __builtin_amdgcn_sched_barrier(0);
                else if (fill) __builtin_amdgcn_sched_barrier(0);
            }
            if (C::LAG == 1 && active) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[i][NJ - 1][v] = fmaf(pp[i][v], f[i], acc[i][NJ - 1][v]);
            }
        };

        if constexpr (C::NSTAGE == 3) {
            // stage 1 is always filled (with K block 0 again when there is one K
            // block) so that the steady loop starts from the same memory-op count
            // on every path
            issue_all(0, stage0);
            issue_all(KB > 1 ? 1 : 0, stage1);
            int kb = 0;
            // steady state: every step refills the stage two ahead, unconditionally,
            // so the compiler sees the same memory ops on every path
            for (; kb + 4 < KB; kb += 3) {
                __builtin_amdgcn_s_waitcnt(kWaitSteady); cbarrier(); step(kb, stage0, true, kb + 2, stage2);
                __builtin_amdgcn_s_waitcnt(kWaitSteady); cbarrier(); step(kb + 1, stage1, true, kb + 3, stage0);
                __builtin_amdgcn_s_waitcnt(kWaitSteady); cbarrier(); step(kb + 2, stage2, true, kb + 4, stage1);
            }
            // tail (at most 4 K blocks; kb is a multiple of 3 here)
            auto tail = [&](int k, const uint8_t* cur, uint8_t* nxt2) __attribute__((always_inline)) {
                if (k >= KB) return;
                if (k + 1 < KB) __builtin_amdgcn_s_waitcnt(kWaitSteady);
                else __builtin_amdgcn_s_waitcnt(kWaitAll);
                cbarrier();
                step(k, cur, k + 2 < KB, k + 2, nxt2);
            };
            tail(kb, stage0, stage2);
            tail(kb + 1, stage1, stage0);
            tail(kb + 2, stage2, stage1);
            tail(kb + 3, stage0, stage2);
        } else {
            issue_all(0, stage0);
            int kb = 0;
            for (; kb + 2 < KB; kb += 2) {
                __builtin_amdgcn_s_waitcnt(kWaitAll); cbarrier(); step(kb, stage0, true, kb + 1, stage1);
                __builtin_amdgcn_s_waitcnt(kWaitAll); cbarrier(); step(kb + 1, stage1, true, kb + 2, stage0);
            }
            // tail (one or two K blocks; kb is even here)
            __builtin_amdgcn_s_waitcnt(kWaitAll);
            cbarrier();
            step(kb, stage0, kb + 1 < KB, kb + 1, stage1);
            if (kb + 1 < KB) {
                __builtin_amdgcn_s_waitcnt(kWaitAll);
                cbarrier();
                step(kb + 1, stage1, false, 0, stage0);
            }
        }

        __builtin_amdgcn_s_waitcnt(kWaitAll);
        // epilogue: bf16 (RNE), valid rows and columns only; 4 consecutive columns
        // (8 bytes) per lane and sub-tile
        if (active) {
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int row = wm * RW + i * 16 + (lane & 15);
                if (row < nvalid) {
                    uint16_t* yrow = y + (int64_t)(r0 + row) * N + n0 + wn * CW + 4 * (lane >> 4);
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        const uint32_t lo = moe::f32_to_bf16_rne(acc[i][j][0]) | (moe::f32_to_bf16_rne(acc[i][j][1]) << 16);
                        const uint32_t hi = moe::f32_to_bf16_rne(acc[i][j][2]) | (moe::f32_to_bf16_rne(acc[i][j][3]) << 16);
                        *reinterpret_cast<uint2*>(yrow + j * 16) = make_uint2(lo, hi);
                    }
                }
            }
        }
        __syncthreads();
    }
}

// Pre-pass, one launch:
//  * row-scale table: out[kb * scale_ld + r] = q_scale[row_slot[r], kb] for the
//    R expert-major rows (R = expert_offsets[L]).  One thread per row reads its
//    slot's contiguous scales; for a fixed kb, consecutive threads write
//    consecutive floats.  A row id outside [0, T) gets scale 0 (a zero row).
//  * tile descriptors (the last workgroup): per local expert ceil(count / BM)
//    row tiles times NT column tiles, experts in order, column tiles outer and
//    row tiles inner; tiles[0].x = number of tiles, tiles[1 + t] =
//    {expert, column tile, first row, valid rows | row tile << 9}.
template <int BM>
__global__ void __launch_bounds__(256)
gemm1_prep_kernel(const float* __restrict__ q_scale, const int32_t* __restrict__ row_slot,
                  const int32_t* __restrict__ expert_offsets, int L, int KB, int NT, int64_t T,
                  int64_t rows_cap, int64_t scale_ld, float* __restrict__ out, int4* __restrict__ tiles,
                  int64_t tiles_cap) {
    if (blockIdx.x == gridDim.x - 1) {
        __shared__ int eoff[kMaxL + 1];
        __shared__ int tstart[kMaxL + 1];
        __shared__ int wsum[256 / MOE_WAVE];
        const int tid = threadIdx.x, lane = tid % MOE_WAVE, wv = tid / MOE_WAVE;
        for (int i = tid; i <= L; i += 256) {
            const int64_t o = expert_offsets[i];
            eoff[i] = (int)(o < 0 ? 0 : (o > rows_cap ? rows_cap : o));
        }
        __syncthreads();
        // tstart = exclusive prefix of the per-expert tile counts (4 experts per thread)
        int cnt4[4], run = 0;
        for (int u = 0; u < 4; ++u) {
            const int e = tid * 4 + u;
            int mt = 0;
            if (e < L) {
                const int c = eoff[e + 1] - eoff[e];
                mt = c > 0 ? (c + BM - 1) / BM : 0;
            }
            cnt4[u] = mt * NT;
            run += cnt4[u];
        }
        const int incl = moe::wave_inclusive_scan(run);
        if (lane == MOE_WAVE - 1) wsum[wv] = incl;
        __syncthreads();
        int base = incl - run;
        for (int i = 0; i < wv; ++i) base += wsum[i];
        for (int u = 0; u < 4; ++u) {
            const int e = tid * 4 + u;
            if (e < L) tstart[e] = base;
            base += cnt4[u];
        }
        if (tid == 255) tstart[L] = base;   // every expert index lies below 4 * 256
        __syncthreads();
        // offsets from the layout give at most rows_cap / BM + L row tiles; the clamp
        // only keeps malformed offsets inside the descriptor array
        const int total = (int)min((int64_t)tstart[L], tiles_cap);
        for (int t = tid; t < total; t += 256) {
            int lo = 0, hi = L - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (tstart[mid] <= t) lo = mid; else hi = mid - 1;
            }
            const int e = lo;
            const int mt = (eoff[e + 1] - eoff[e] + BM - 1) / BM;
            const int local = t - tstart[e];
            const int nt = local / mt, mtile = local - nt * mt;
            const int r0 = eoff[e] + mtile * BM;
            const int nvalid = min(BM, eoff[e + 1] - r0);
            tiles[1 + t] = int4{e, nt, r0, nvalid | (mtile << 9)};
        }
        if (tid == 0) tiles[0] = int4{total, 0, 0, 0};
        return;
    }
    int64_t R = expert_offsets[L];
    R = R < 0 ? 0 : (R > rows_cap ? rows_cap : R);
    const int64_t nthr = (int64_t)(gridDim.x - 1) * 256;
    for (int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x; r < R; r += nthr) {
        const int s = row_slot[r];
        const bool ok = (uint64_t)s < (uint64_t)T;
        const float* src = q_scale + (int64_t)(ok ? s : 0) * KB;
        for (int kb = 0; kb < KB; ++kb) out[kb * scale_ld + r] = ok ? src[kb] : 0.0f;
    }
}

// Rows of the table: every row a tile can name (rows_cap plus one tile of the
// largest row count), rounded up to 64 floats.
constexpr int kMaxBM = 256;
int64_t scale_ld_of(int64_t rows_cap) { return ((rows_cap + kMaxBM) + 63) & ~int64_t(63); }

int cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

#ifndef MOE_GEMM1_CFG
#define MOE_GEMM1_CFG 0
#endif
#ifndef MOE_GEMM1_LAG
#define MOE_GEMM1_LAG 0
#endif
//                  BM  WM WN stages
using Tile256w8  = Cfg<256, 4, 2, 2, MOE_GEMM1_LAG>;
using Tile128w8  = Cfg<128, 2, 4, 3, MOE_GEMM1_LAG>;
using Tile256w16 = Cfg<256, 4, 4, 2, MOE_GEMM1_LAG>;
using Tile128w16 = Cfg<128, 4, 4, 3, MOE_GEMM1_LAG>;
using TileCfg = std::conditional_t<
    MOE_GEMM1_CFG == 0, Tile256w8,
    std::conditional_t<MOE_GEMM1_CFG == 1, Tile128w8,
                       std::conditional_t<MOE_GEMM1_CFG == 2, Tile256w16, Tile128w16>>>;
static_assert(TileCfg::BM <= kMaxBM, "scale table padding covers one tile");

// Workspace: the row-scale table, then the tile descriptors (16 B each).
struct WsLayout {
    int64_t scale_ld, table_bytes, tiles_cap, bytes;
};
WsLayout ws_layout(const moe::Dims& d, int n) {
    WsLayout l;
    const int64_t rows_cap = d.T * d.k;
    l.scale_ld = scale_ld_of(rows_cap);
    l.table_bytes = ((d.H / BK) * l.scale_ld * 4 + 255) & ~int64_t(255);
    l.tiles_cap = (rows_cap / kMinBM + d.L) * ((n + BN - 1) / BN);
    l.bytes = l.table_bytes + (1 + l.tiles_cap) * 16;
    return l;
}

}  // namespace

extern "C" moe_status moe_grouped_gemm1_workspace(const moe_dims* dims, int32_t n, size_t* bytes) {
    moe::Dims d;
    moe_status st = moe::load_dims(dims, &d, true);
    if (st != MOE_OK) return st;
    if (!bytes || n < 128 || n % 128 != 0) return MOE_ERR_INVALID_ARG;
    *bytes = (size_t)ws_layout(d, n).bytes;
    return MOE_OK;
}

extern "C" moe_status moe_grouped_gemm1(const moe_dims* dims, int32_t n, const uint8_t* q_e4m3,
                                        const float* q_scale, const int32_t* row_slot,
                                        const int32_t* expert_offsets, const int32_t* totals,
                                        const uint8_t* w_e4m3, const float* w_scale, uint16_t* y_bf16,
                                        void* ws, size_t ws_bytes, void* hip_stream) {
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
    // 32-bit offsets inside the kernel: slot rows of q, rows of one expert's weight;
    // row tile ids in 22 bits of a descriptor
    if (d.T * d.H >= ((int64_t)1 << 32) || (int64_t)n * d.H >= ((int64_t)1 << 31) ||
        rows_cap * n >= ((int64_t)1 << 40) || rows_cap / kMinBM >= ((int64_t)1 << 22))
        return MOE_ERR_UNSUPPORTED;
    const int64_t KB = d.H / BK;
    const WsLayout wl = ws_layout(d, n);
    if (!ws || ws_bytes < (size_t)wl.bytes) return MOE_ERR_WORKSPACE;
    if (KB * wl.scale_ld >= ((int64_t)1 << 31) || wl.tiles_cap >= ((int64_t)1 << 31) - 1)
        return MOE_ERR_UNSUPPORTED;
    int cus = cu_count();
    if (cus <= 0) return MOE_ERR_HIP;
    hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
    float* row_scale = reinterpret_cast<float*>(ws);
    int4* tiles = reinterpret_cast<int4*>(static_cast<uint8_t*>(ws) + wl.table_bytes);
    const int NT = (int)((n + BN - 1) / BN);
    // gather workgroups plus the planning workgroup (the last one)
    const int pgrid = (int)std::min<int64_t>((rows_cap + 255) / 256, 2048) + 1;
    hipLaunchKernelGGL((gemm1_prep_kernel<TileCfg::BM>), dim3(pgrid), dim3(256), 0, stream, q_scale, row_slot,
                       expert_offsets, (int)d.L, (int)KB, NT, d.T, rows_cap, wl.scale_ld, row_scale, tiles,
                       wl.tiles_cap);
    if ((st = moe::launch_status()) != MOE_OK) return st;
    const int grid = ((cus + kXcds - 1) / kXcds) * kXcds;
    hipLaunchKernelGGL((grouped_gemm1_kernel<TileCfg>), dim3(grid), dim3(TileCfg::kThreads), 0, stream,
                       q_e4m3, row_scale, tiles, row_slot, w_e4m3, w_scale, y_bf16, (int)n, (int)d.H, d.T,
                       wl.scale_ld);
    return moe::launch_status();
}
