// Step 3: grouped GEMM1 over the local experts, A rows read in place through
// the rowmap ("poc(cco): MegaMoE stage1 dispatch over SDMA", "What": GEMM1
// reads its A rows in place through a rowmap; commit 1: fp8 rows and block
// scales through the rowmap; "Where we stand": block-scaled fp8 tiles, one
// expert per tile, the compute-bound loop of stage1).  The same kernel, by
// template flags, is the MX variant (e8m0 group scales in the MFMA's
// block-scale operands, MX) and stage2's GEMM2 (A rows read directly, DIRECT).
//
// y[r, c] = sum_kb (sum_{h in kb} qA[r,h] * qW[c,h]) * sA[r,kb] * sW[c/128,kb]
//
// The scales are fp32 (not powers of two), so they cannot ride in the MFMA's
// e8m0 block scales: each 128-wide K block is one fp8 MFMA with a zero
// accumulator per 16x16 sub-tile (v_mfma_f32_16x16x128_f8f6f4 covers exactly
// K = 128), folded into the fp32 running sum by one FMA with sA[row] * sW.
// The MFMA computes the transposed sub-tile (weight rows as its A operand), so
// a lane holds 4 consecutive output columns of one row: one row scale per lane
// and sub-tile row; the epilogue regroups the bf16 outputs through LDS into
// whole 128 B rows before storing them.
//
// Tile: 128 rows of one expert x 256 columns.  Workgroup of 12 wavefronts
// (three per SIMD): 2 x 4 compute wavefronts of 64 x 64 outputs each, and 4
// loader wavefronts.
//
// Why loaders: the operand stream is bounded by the L2 requests a CU can keep
// in flight (about 70 lines) and by their latency (L2 misses to HBM take
// several times as long as hits), so the loads alone take about as long as
// the MFMAs alone.  A wavefront whose next instruction is a load that the full queue
// cannot accept stalls, and the MFMAs behind it in its instruction stream
// stall with it; when every wavefront both loads and computes, load time and
// MFMA time add up instead of overlapping.  The compute wavefronts here never
// issue a load (only LDS reads), so their MFMAs run while the loaders block.
//
// Operand staging: K blocks stream through a 3-stage LDS ring filled with
// global_load_lds_dwordx4 (memory straight to LDS, no staging registers).  The
// loaders walk this workgroup's tiles back to back, so the ring runs across
// tile boundaries and the next tile's first K blocks load during the current
// tile's last steps and epilogue.  One workgroup barrier per K step g: before
// it the loaders have waited (explicit vmcnt) for stage g; after it the compute
// wavefronts read stage g while the loaders refill the stage that step g-1
// read.  The compute wavefronts take barrier g inside step g-1, as soon as
// every fragment of step g-1 is in their registers, and issue step g-1's last
// column group of MFMAs after it, between their first reads of stage g (except
// across a tile boundary).  Each lane of a direct-to-LDS load lands at base + 16 * lane; the
// swizzle of the 16 B chunks inside a 128 B row (chunk c of row r sits in slot
// c ^ (r & 7) ^ ((r >> 3) & 1)) is made by choosing which global chunk each
// lane fetches: 16 consecutive rows read at one chunk then hit 16 distinct
// 16 B bank groups of a 256 B window (and 8 distinct ones of a 128 B window).
//
// Row scales: the rows of a tile are gathered, so their scales would cost one
// scattered 4 B request per row and K block.  A pre-pass writes the scales
// into a K-block-major table indexed by expert-major row (the caller's
// workspace), and each loader brings 64 rows' scales per stage as one
// contiguous 256 B piece.  The weights' scales of the stage's K block ride in
// the same ring, so a step's operands and scales all come from LDS and the
// compute wavefronts read them in the order of first use (column group 0 and
// row group 0 first, the scales last: the fold that needs them comes one
// column group later).
//
// Scheduling: one persistent workgroup per CU walks its slots of a tile table
// that the pre-pass derives from expert_offsets.  In the natural order (experts
// in order; per expert, column tiles outer and row tiles inner) the row tiles
// that share a weight slab are adjacent; each round of the table gives every
// XCD (workgroup b runs on XCD b % 8) a run of consecutive natural tiles, so
// the row tiles sharing a slab meet in that XCD's L2.  For K loops of at least
// 32 steps the pre-pass also balances each round's partial tiles (an expert's
// last rows) across the XCD's workgroups (gemm1_prep_kernel).  A compute
// wavefront whose 64 rows all lie past the expert's last row skips its MFMAs.
#include "common.h"

#include <type_traits>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
using moe::u32x4;

constexpr int BN = 256, BK = 128;
constexpr int kMaxL = 1024;
constexpr int kXcds = 8;
constexpr int kMinBM = 128;   // tile descriptors are sized for the smallest row tile
constexpr int kPrepKb = 8;    // K blocks per row-scale gather work item
constexpr int kPrepWgPerCu = 4;   // gather workgroups of the pre-pass per CU
// schedule slots past the tile count (the balanced schedule's last round can
// leave up to one grid's worth of idle slots); also the largest main grid
constexpr int kMaxGrid = 1024;
// the cost-balanced tile schedule is used for K loops of at least this many
// steps (GEMM1's 56: -5 % and more); with short tiles (GEMM2's 16 steps) the
// drift it introduces between the workgroups that share a weight slab cost
// more L2 reuse than it saved (+18 %), so those keep the plain round-robin
constexpr int kBalanceMinKb = 32;
// the planner's limits: 32 workgroups per XCD (a half wavefront each), and
// every tile's expert in LDS (two bytes each; 24 KB keeps four gather
// workgroups of the pre-pass on a CU)
constexpr int kPlanMaxNx = 32;
constexpr int kPlanMaxTiles = 12288;

#define GPTR(p) ((const void __attribute__((address_space(1)))*)(p))
#define LPTR(p) ((void __attribute__((address_space(3)))*)(p))

// s_waitcnt immediate waiting until at most n vector-memory ops are outstanding
// (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14)
constexpr int wait_vm(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14); }
// s_waitcnt immediate waiting until every LDS operation has returned (lgkmcnt(0))
constexpr int kWaitLds0 = 0xF | (0x7 << 4) | (0x3 << 14);

// s_waitcnt vmcnt(n) for a wave-uniform n in [LO, HI] (the count is an
// immediate of the instruction, so each value is its own instruction)
template <int LO, int HI>
__device__ __forceinline__ void wait_vm_dyn(int n) {
    if constexpr (LO == HI) {
        __builtin_amdgcn_s_waitcnt(wait_vm(LO));
    } else {
        if (n == LO) __builtin_amdgcn_s_waitcnt(wait_vm(LO));
        else wait_vm_dyn<LO + 1, HI>(n);
    }
}

__device__ __forceinline__ void cbarrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Tile configuration: BM x 256 tile, WM x WN compute wavefronts, NLW loader
// wavefronts, NSTAGE-deep K ring.
template <int BM_, int WM_, int WN_, int NLW_, int NSTAGE_>
struct Cfg {
    static constexpr int BM = BM_, WM = WM_, WN = WN_, NLW = NLW_, NSTAGE = NSTAGE_;
    static constexpr int kCompute = WM * WN, kWaves = kCompute + NLW, kThreads = kWaves * MOE_WAVE;
    static constexpr int RW = BM / WM, CW = BN / WN, MI = RW / 16, NJ = CW / 16;
    static constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
    static constexpr int S_BYTES = NLW * 256;                 // row scales of rows 0 .. 64 NLW - 1
    static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
    // A: BM/8 loads of 8 rows (1 KB); loader lw takes A_LO of them, one more if
    // lw < A_EXTRA.  B: B_LOADS 1 KB loads each.
    static constexpr int A_GROUPS = BM / 8, A_LO = A_GROUPS / NLW, A_EXTRA = A_GROUPS % NLW;
    static constexpr int A_LOADS = A_LO + (A_EXTRA ? 1 : 0), B_LOADS = B_BYTES / (1024 * NLW);
    static constexpr int NLD = A_LOADS + B_LOADS + 2;         // most loads a loader issues per stage
    static_assert(RW % 16 == 0 && CW % 16 == 0 && CW <= 128 && 128 % CW == 0, "wavefront tile");
    static_assert(BM % 8 == 0 && B_BYTES % (1024 * NLW) == 0 && A_LO >= 1 && B_LOADS >= 1,
                  "whole 1 KB loads");
    static_assert(NLW * 64 >= BM && BM >= kMinBM && kThreads <= 1024, "scale rows, descriptors, size");
    static_assert(NSTAGE >= 2 && NSTAGE <= 4 && NSTAGE * STAGE <= 160 * 1024 && 2 * NLD < 64, "ring");
};

// MX: the operands carry e8m0 scales per 32 K elements (packed four per dword:
// rows' dwords gathered into the row-scale table, the weights' dwords stored
// [L, H/128, N]); they ride in the MFMA's block-scale operands, so the K blocks
// accumulate in the MFMA itself and there is no fold.
// DIRECT: the A operand's rows are the expert-major rows themselves (row r of
// the tile reads A row r; GEMM2 on stage2's output), instead of rows gathered
// through the rowmap; T is then the number of A rows.  MX && DIRECT (the MX
// GEMM2): each output row is multiplied by wtab[row] (its routing weight)
// before the bf16 rounding; a weight that is not a power of two cannot ride in
// the e8m0 codes.
template <class C, bool MX, bool DIRECT>
__global__ void __launch_bounds__(C::kThreads, 1)
grouped_gemm1_kernel(const uint8_t* __restrict__ q, const uint32_t* __restrict__ row_scale,
                     const int4* __restrict__ tiles, const int32_t* __restrict__ row_slot,
                     const uint8_t* __restrict__ w, const void* __restrict__ w_scale_v,
                     uint16_t* __restrict__ y, int N, int H, int64_t T, int64_t scale_ld,
                     const float* __restrict__ wtab) {
    MOE_TRACE_T0(tr0);
    // fp32 path: one float per (expert, 128 columns, K block), [L, N/128, H/128];
    // MX path: packed e8m0 codes per (expert, K block, column), [L, H/128, N]
    const float* w_scale = static_cast<const float*>(w_scale_v);
    const uint32_t* w_scale_mx = static_cast<const uint32_t*>(w_scale_v);
    constexpr int BM = C::BM, MI = C::MI, NJ = C::NJ, RW = C::RW, CW = C::CW, WN = C::WN;
    constexpr int A_BYTES = C::A_BYTES, B_BYTES = C::B_BYTES, NSTAGE = C::NSTAGE;
    // MX stages also hold the columns' scale dwords (1 KiB: BN columns)
    constexpr int STAGE = C::STAGE + (MX ? C::NLW * 256 : 0);
    constexpr int A_LOADS = C::A_LOADS, B_LOADS = C::B_LOADS;
    // Per stage each loader issues its A and B loads plus at most one scale load:
    // loaders lw < NSA bring rows lw*64 .. lw*64+63's scales (4 B a lane), and
    // loader SB_LOADER brings the columns' scales: in MX mode the BN columns'
    // dwords (16 B a lane, after the row scales' NLW * 256 bytes), else the two
    // 128-column blocks' floats (lane l: block l & 1) at byte NSA * 256
    constexpr int NSA = (C::BM + 63) / 64, SB_LOADER = NSA;
    constexpr int NLD = C::NLD;
    static_assert(SB_LOADER < C::NLW && (NSA + 1) * 256 <= C::S_BYTES, "scale loaders");
    static_assert(BN * 4 == 64 * 16, "one 16 B-a-lane load covers the column scales");
    static_assert(NSTAGE * STAGE <= 160 * 1024 && 2 * NLD < 64, "ring");
    __shared__ __align__(16) uint8_t ring[NSTAGE * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid % MOE_WAVE;
    const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);
    const int KB = H / BK;
    const int NB = N / 128;
    const int total = tiles[0].x;
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int my = (b % kXcds) * (G / kXcds) + b / kXcds;   // G is a multiple of 8
    const int ntiles = total > my ? (total - my + G - 1) / G : 0;

    if (wave >= C::kCompute) {
        // ---------------- loader wavefronts ----------------
        const int lw = wave - C::kCompute;
        // this loader's A groups: a_cnt of them from a_start (wave-uniform)
        const int a_cnt = C::A_LO + (lw < C::A_EXTRA ? 1 : 0);
        const int a_start = lw * C::A_LO + min(lw, C::A_EXTRA);
        const int lrow = lane >> 3;
        const int gchunk = (lane & 7) ^ lrow;
        // 16 B chunk of the row's 128 K bytes that goes to logical chunk c: c itself,
        // or in MX mode the MFMA's K order (logical 2q, 2q+1 = K chunks q, 4+q), so
        // the compute reads pairs (2q, 2q+1) either way
        auto kchunk = [](int c) { return MX ? ((c >> 1) | ((c & 1) << 2)) : c; };
        int cur = -1;
        uint32_t a_off[A_LOADS];
        const uint8_t* wexp = w;
        const uint32_t* srow = row_scale;
        int ncols = BN;
        const uint32_t* wsc_mx = w_scale_mx;
        const float* wsc_f = w_scale;
        // steps of this workgroup: its slots' tiles, up to the first idle slot
        int nsteps = ntiles * KB;
        auto setup = [&](int it) __attribute__((always_inline)) {
            const int4 td = tiles[1 + it * G + my];
            const int e = td.x, r0 = td.z, nvalid = td.w & 511;
            if (nvalid == 0) return false;
            const int n0 = td.y * BN;
            ncols = min(BN, N - n0);
            if (MX) {
                // lane l: columns 4l .. 4l+3 (past a half tile: the last four again);
                // N % 128 == 0 and n0 % 256 == 0 keep every address 16 B aligned
                wsc_mx = w_scale_mx + (int64_t)e * KB * N + n0 + 4 * min(lane, ncols / 4 - 1);
            } else {
                wsc_f = w_scale + ((int64_t)e * NB + min(n0 / 128 + (lane & 1), NB - 1)) * KB;
            }
            int s0 = DIRECT ? r0 : row_slot[r0];
            if ((uint64_t)s0 >= (uint64_t)T) s0 = 0;
            // all row ids first (one wait), then the selection: rows past the
            // expert's last row reuse the first row's slot
            int sl[A_LOADS];
#pragma unroll
            for (int i = 0; i < A_LOADS; ++i) {
                const int rr = r0 + min((a_start + min(i, a_cnt - 1)) * 8 + lrow, nvalid - 1);
                sl[i] = DIRECT ? rr : row_slot[rr];
            }
#pragma unroll
            for (int i = 0; i < A_LOADS; ++i) {
                const int r = (a_start + i) * 8 + lrow;
                const int v = (r < nvalid && (uint64_t)sl[i] < (uint64_t)T) ? sl[i] : s0;
                a_off[i] = (uint32_t)v * (uint32_t)H + kchunk(gchunk ^ ((a_start + i) & 1)) * 16;
            }
            wexp = w + ((int64_t)e * N + n0) * H;
            srow = row_scale + r0 + lw * 64;
            return true;
        };
        const uint32_t b_lane0 = (uint32_t)lrow * (uint32_t)H + kchunk(gchunk) * 16;
        const uint32_t b_lane1 = (uint32_t)lrow * (uint32_t)H + kchunk(gchunk ^ 1) * 16;
        const uint32_t s_lane = (uint32_t)lane * 4u;
        auto issue = [&](int s) __attribute__((always_inline)) {
            const int it = s / KB, kb = s - it * KB;
            if (it != cur) {
                if (!setup(it)) {                 // an idle slot: this workgroup's tiles end here
                    nsteps = s;
                    return;
                }
                cur = it;
            }
            uint8_t* base = ring + (s % NSTAGE) * STAGE;
#pragma unroll
            for (int i = 0; i < A_LOADS; ++i)
                if (i < a_cnt)
                    __builtin_amdgcn_global_load_lds(GPTR((q + kb * BK) + a_off[i]),
                                                     LPTR(base + (a_start + i) * 1024), 16, 0, 0);
#pragma unroll
            for (int i = 0; i < B_LOADS; ++i) {
                // rows past a half tile re-read the first half (their columns are not stored)
                int rb = (lw * B_LOADS + i) * 8;
                if (rb >= ncols) rb -= ncols;
                __builtin_amdgcn_global_load_lds(
                    GPTR((wexp + kb * BK + (uint32_t)rb * (uint32_t)H) + (((lw * B_LOADS + i) & 1) ? b_lane1 : b_lane0)),
                    LPTR(base + A_BYTES + (lw * B_LOADS + i) * 1024), 16, 0, 0);
            }
            if (lw < NSA)
                __builtin_amdgcn_global_load_lds(GPTR(reinterpret_cast<const uint8_t*>(srow + kb * scale_ld) + s_lane),
                                                 LPTR(base + A_BYTES + B_BYTES + lw * 256), 4, 0, 0);
            else if (lw == SB_LOADER) {
                if (MX)
                    __builtin_amdgcn_global_load_lds(GPTR(wsc_mx + (int64_t)kb * N),
                                                     LPTR(base + A_BYTES + B_BYTES + C::NLW * 256), 16, 0, 0);
                else
                    __builtin_amdgcn_global_load_lds(GPTR(wsc_f + kb), LPTR(base + A_BYTES + B_BYTES + NSA * 256),
                                                     4, 0, 0);
            }
        };
        // loads this loader issues per stage (wave-uniform)
        const int nld = a_cnt + B_LOADS + ((lw < NSA || lw == SB_LOADER) ? 1 : 0);
        constexpr int NLD_MIN = C::A_LO + B_LOADS;
        for (int s = 0; s < NSTAGE - 1 && s < nsteps; ++s) issue(s);
        for (int g = 0; g < nsteps; ++g) {
            // stage g has landed once at most the later stages' loads are outstanding
            const int later = min(NSTAGE - 2, nsteps - 1 - g);
            if (later >= 2) wait_vm_dyn<2 * NLD_MIN, 2 * NLD>(2 * nld);
            else if (later == 1) wait_vm_dyn<NLD_MIN, NLD>(nld);
            else __builtin_amdgcn_s_waitcnt(wait_vm(0));
            cbarrier();
            if (g + NSTAGE - 1 < nsteps) issue(g + NSTAGE - 1);
        }
        __builtin_amdgcn_s_waitcnt(wait_vm(0));
        if (lw == 0 && lane == 0) MOE_TRACE_PUT(moe::kTrGemmLoader, blockIdx.x, 0, 0, tr0);
        return;
    }

    // ---------------- compute wavefronts ----------------
    // issue priority over the loaders, which mostly sleep on their waits: when
    // both are ready the SIMD serves the MFMA stream first (≈1 % faster in
    // interleaved timing of GEMM1 and GEMM2; loader priority measured ±0)
    __builtin_amdgcn_s_setprio(2);
    const int wm = wave / WN, wn = wave % WN;
    int g = 0;
    for (int it = 0; it < ntiles; ++it) {
        MOE_TRACE_T0(tr_tile);
        const int4 td = tiles[1 + it * G + my];
        const int e = td.x, r0 = td.z, nvalid = td.w & 511;
        if (nvalid == 0) break;                   // an idle slot: this workgroup's tiles end here
        const int n0 = td.y * BN;
        const int ncols = min(BN, N - n0);
        const bool active = wm * RW < nvalid && wn * CW < ncols;

        v4f acc[MI][NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        // MX GEMM2: the rows' routing weights, loaded now and used by the epilogue
        float wr[MI];
        if constexpr (MX && DIRECT) {
#pragma unroll
            for (int i = 0; i < MI; ++i) wr[i] = wtab[r0 + min(wm * RW + i * 16 + (lane & 15), nvalid - 1)];
        }

        // The barrier of step g+1 is taken inside step g, once every fragment of
        // step g is in registers (after the read of the last column group's B
        // fragment): the last column group's MFMAs then run after the barrier,
        // interleaved with the first reads of step g+1, so the MFMA pipe has work
        // while those reads are in flight instead of idling at the start of every
        // step.  A tile's last step keeps its barrier at the top of the next tile:
        // the epilogue stages its outputs in that step's ring slot, which the
        // loaders refill only after that barrier.  Inactive wavefronts take the
        // same barriers (one per step).
        if (!active) {
            for (int kb = 0; kb < KB; ++kb, ++g) cbarrier();
        } else if constexpr (MX) {
            // hardware K order of the 16x16x128 fp8 operand: lane quarter q holds
            // K [16q, 16q+16) and [64+16q, 64+16q+16), K chunks q and 4+q, which the
            // loaders placed at logical chunks 2q and 2q+1; the scale of (row or
            // column l & 15, K group l >> 4) comes from lane l
            const int qq = lane >> 4;
            auto read_a = [&](const uint8_t* As, int i, v8i& a, uint32_t& sa) __attribute__((always_inline)) {
                const int row = wm * RW + i * 16 + (lane & 15);
                const int sw_r = (row & 7) ^ ((row >> 3) & 1);
                const u32x4 a0 = *reinterpret_cast<const u32x4*>(As + row * BK + (((2 * qq) ^ sw_r) << 4));
                const u32x4 a1 = *reinterpret_cast<const u32x4*>(As + row * BK + (((2 * qq + 1) ^ sw_r) << 4));
                a = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                const uint32_t* Sa = reinterpret_cast<const uint32_t*>(As + A_BYTES + B_BYTES);
                sa = Sa[row];
            };
            auto read_b = [&](const uint8_t* As, int j, uint32_t& sraw) __attribute__((always_inline)) {
                const uint8_t* Bs = As + A_BYTES;
                const uint32_t* Sb = reinterpret_cast<const uint32_t*>(Bs + B_BYTES) + C::NLW * 64;
                const int col = wn * CW + j * 16 + (lane & 15);
                const int sw_c = (col & 7) ^ ((col >> 3) & 1);
                const u32x4 b0 = *reinterpret_cast<const u32x4*>(Bs + col * BK + (((2 * qq) ^ sw_c) << 4));
                const u32x4 b1 = *reinterpret_cast<const u32x4*>(Bs + col * BK + (((2 * qq + 1) ^ sw_c) << 4));
                sraw = Sb[col];
                return v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
            };
            v8i af[MI], bnext;
            // the rows' scale words as read (sa) and this step's codes extracted
            // from them at the step's first column group (sae): the extraction
            // waits for the read, which the next step's reads then overlap
            uint32_t sa[MI];
            int sae[MI];
            uint32_t sbn;
            // column groups 0 .. NJ-2 of a step; the next group's reads are issued
            // before this group's MFMAs (left alone, the compiler reuses one register
            // set and waits on every read)
            auto groups = [&](const uint8_t* As) __attribute__((always_inline)) {
#pragma unroll
                for (int j = 0; j < NJ - 1; ++j) {
                    const v8i bf = bnext;
                    // the code is extracted here, after the fence below of the group
                    // before, so only this group's scale read is waited on
                    const int sb = (int)((sbn >> (8 * qq)) & 0xFFu);
                    if (j == 0) {
#pragma unroll
                        for (int i = 0; i < MI; ++i) sae[i] = (int)((sa[i] >> (8 * qq)) & 0xFFu);
                    }
                    bnext = read_b(As, j + 1, sbn);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < MI; ++i)
                        // transposed sub-tile: weights' fragment and scale first
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            bf, af[i], acc[i][j], 0, 0, 0, sb, 0, sae[i]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            cbarrier();
            {
                const uint8_t* As = ring + (g % NSTAGE) * STAGE;
#pragma unroll
                for (int i = 0; i < MI; ++i) read_a(As, i, af[i], sa[i]);
                bnext = read_b(As, 0, sbn);
            }
            for (int kb = 0; kb + 1 < KB; ++kb, ++g) {
                groups(ring + (g % NSTAGE) * STAGE);
                const v8i bf = bnext;
                const int sb = (int)((sbn >> (8 * qq)) & 0xFFu);
                // every read of this step has returned: its ring slot is free
                __builtin_amdgcn_s_waitcnt(kWaitLds0);
                cbarrier();
                const uint8_t* As1 = ring + ((g + 1) % NSTAGE) * STAGE;
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    acc[i][NJ - 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        bf, af[i], acc[i][NJ - 1], 0, 0, 0, sb, 0, sae[i]);
                    read_a(As1, i, af[i], sa[i]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                bnext = read_b(As1, 0, sbn);
                __builtin_amdgcn_sched_barrier(0);
            }
            // the tile's last step: no barrier inside it
            groups(ring + (g % NSTAGE) * STAGE);
            const int sb = (int)((sbn >> (8 * qq)) & 0xFFu);
#pragma unroll
            for (int i = 0; i < MI; ++i)
                acc[i][NJ - 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    bnext, af[i], acc[i][NJ - 1], 0, 0, 0, sb, 0, sae[i]);
            ++g;
        } else {
            auto read_b = [&](const uint8_t* As, int j) __attribute__((always_inline)) {
                const uint8_t* Bs = As + A_BYTES;
                const int col = wn * CW + j * 16 + (lane & 15);
                const int c0 = (lane >> 4) * 2;
                const int sw_c = (col & 7) ^ ((col >> 3) & 1);
                const u32x4 b0 = *reinterpret_cast<const u32x4*>(Bs + col * BK + ((c0 ^ sw_c) << 4));
                const u32x4 b1 = *reinterpret_cast<const u32x4*>(Bs + col * BK + (((c0 + 1) ^ sw_c) << 4));
                return v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
            };
            auto read_a = [&](const uint8_t* As, int i) __attribute__((always_inline)) {
                const int row = wm * RW + i * 16 + (lane & 15);
                const int c0 = (lane >> 4) * 2;
                const int sw_r = (row & 7) ^ ((row >> 3) & 1);
                const u32x4 a0 = *reinterpret_cast<const u32x4*>(As + row * BK + ((c0 ^ sw_r) << 4));
                const u32x4 a1 = *reinterpret_cast<const u32x4*>(As + row * BK + (((c0 + 1) ^ sw_r) << 4));
                return v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            };
            // the weights' scale of this wavefront's 128-column block and its rows'
            // scales (first used by the folds of column group 0, one group later)
            auto read_scales = [&](const uint8_t* As, float& sw, float* sr) __attribute__((always_inline)) {
                const uint8_t* Bs = As + A_BYTES;
                sw = reinterpret_cast<const float*>(Bs + B_BYTES + NSA * 256)[(wn * CW) / 128];
                const float* Ss = reinterpret_cast<const float*>(Bs + B_BYTES);
#pragma unroll
                for (int i = 0; i < MI; ++i) sr[i] = Ss[wm * RW + i * 16 + (lane & 15)];
            };
            v8i bnext, af[MI];
            float sw, sr[MI], f[MI];
            v4f pp[MI];
            // column groups 0 .. NJ-2 of a step.  Unit (j, i): the MFMA of row group i,
            // then the fold of row group i's product from column group j-1, whose MFMA
            // went out MI units earlier; the fences keep that order so no unit waits on
            // its own MFMA.  Group j+1's B fragment is read before group j's MFMAs.
            auto groups = [&](const uint8_t* As) __attribute__((always_inline)) {
#pragma unroll
                for (int j = 0; j < NJ - 1; ++j) {
                    const v8i bf = bnext;
                    bnext = read_b(As, j + 1);
#pragma unroll
                    for (int i = 0; i < MI; ++i) {
                        // transposed sub-tile: lane l holds row (l & 15), columns 4*(l >> 4) + v
                        const v4f pc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            bf, af[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                        if (j == 1) f[i] = sr[i] * sw;
                        if (j > 0) {
#pragma unroll
                            for (int v = 0; v < 4; ++v) acc[i][j - 1][v] = fmaf(pp[i][v], f[i], acc[i][j - 1][v]);
                        }
                        pp[i] = pc;
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            };
            // the last column group's unit i: its MFMA and the fold of group NJ-2's product
            auto last_unit = [&](const v8i& bf, int i) __attribute__((always_inline)) {
                const v4f pc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    bf, af[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[i][NJ - 2][v] = fmaf(pp[i][v], f[i], acc[i][NJ - 2][v]);
                pp[i] = pc;
            };
            auto last_folds = [&]() __attribute__((always_inline)) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[i][NJ - 1][v] = fmaf(pp[i][v], f[i], acc[i][NJ - 1][v]);
            };
            cbarrier();
            {
                // reads in the order of first use: column group 0, the row groups, the scales
                const uint8_t* As = ring + (g % NSTAGE) * STAGE;
                bnext = read_b(As, 0);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    af[i] = read_a(As, i);
                    __builtin_amdgcn_sched_barrier(0);
                }
                read_scales(As, sw, sr);
                __builtin_amdgcn_sched_barrier(0);
            }
            for (int kb = 0; kb + 1 < KB; ++kb, ++g) {
                groups(ring + (g % NSTAGE) * STAGE);
                const v8i bf = bnext;
                // every read of this step has returned: its ring slot is free
                __builtin_amdgcn_s_waitcnt(kWaitLds0);
                cbarrier();
                const uint8_t* As1 = ring + ((g + 1) % NSTAGE) * STAGE;
                bnext = read_b(As1, 0);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    last_unit(bf, i);
                    af[i] = read_a(As1, i);
                    __builtin_amdgcn_sched_barrier(0);
                }
                last_folds();
                read_scales(As1, sw, sr);
                __builtin_amdgcn_sched_barrier(0);
            }
            // the tile's last step: no barrier inside it
            groups(ring + (g % NSTAGE) * STAGE);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                last_unit(bnext, i);
                __builtin_amdgcn_sched_barrier(0);
            }
            last_folds();
            ++g;
        }
        // epilogue: bf16 (RNE), valid rows only.  Each 16 x 64 piece (one row group
        // of this wavefront's columns) goes through LDS so that the global stores
        // write whole 128 B rows, 8 lanes x 16 B per row (written straight from the
        // MFMA layout, a lane's 8 B pieces would land as 32 B slivers of 16 rows per
        // store instruction).  Staging: 2 KB per wavefront in the ring slot of the
        // tile's last K step, which the loaders refill only after the next barrier,
        // one these wavefronts have not reached yet; 16 B chunks XOR-swizzled by row.
        static_assert(C::CW == 64 && C::kCompute * 2048 <= STAGE, "epilogue staging: 128 B rows, 2 KB a wavefront");
        if (active) {
            uint8_t* stg = ring + ((g - 1) % NSTAGE) * STAGE + wave * 2048;
            // the lane id through an opaque move, so that the staging offsets and
            // row indices below are computed here and not hoisted out of the tile
            // loop: held across the K loop they cost 16 VGPRs, and at 168 one of
            // them was spilled, whose reload made the tile's last store wait for
            // every store before it
            int el;
            asm volatile("v_mov_b32 %0, %1" : "=v"(el) : "v"(lane));
            const int srow = el & 15, q = el >> 4;
            // MX GEMM2: the row weights' loads (issued at the tile's start) are
            // waited for here, before any store; the in-order count would make a
            // wait placed after a store wait for that store as well
            if constexpr (MX && DIRECT) __builtin_amdgcn_s_waitcnt(wait_vm(0));
#pragma unroll
            for (int i = 0; i < MI; ++i) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    if constexpr (MX && DIRECT) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[i][j][v] *= wr[i];
                    }
                    const uint32_t lo = moe::pack_bf16x2(acc[i][j][0], acc[i][j][1]);
                    const uint32_t hi = moe::pack_bf16x2(acc[i][j][2], acc[i][j][3]);
                    // columns j*16 + 4q .. +3 = byte 32j + 8q of the 128 B row: chunk 2j + q/2
                    *reinterpret_cast<uint2*>(stg + srow * 128 + (((2 * j + (q >> 1)) ^ (srow & 7)) << 4) + (q & 1) * 8) =
                        make_uint2(lo, hi);
                }
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int rr = p * 8 + (el >> 3), c = el & 7;
                    const moe::u32x4 v = *reinterpret_cast<const moe::u32x4*>(stg + rr * 128 + ((c ^ (rr & 7)) << 4));
                    const int row = wm * RW + i * 16 + rr;
                    if (row < nvalid)
                        *reinterpret_cast<moe::u32x4*>(y + (int64_t)(r0 + row) * N + n0 + wn * CW + c * 8) = v;
                }
            }
        }
        if (wave == 0 && lane == 0) MOE_TRACE_PUT(moe::kTrGemmTile, (uint32_t)(it * G + my), (uint32_t)(it * G + my), (uint32_t)it, tr_tile);
    }
    if (wave == 0 && lane == 0) MOE_TRACE_PUT(moe::kTrGemmCompute, blockIdx.x, 0, 0, tr0);
}

// Pre-pass, one launch:
//  * row-scale table: out[kb * scale_ld + r] = q_scale[row_slot[r], kb] for the
//    R expert-major rows (R = expert_offsets[L]), copied as 32-bit words (a
//    float scale, or four packed e8m0 codes); with no rowmap (row_slot null)
//    row r's own scales.  With row weights (row_assign and topk_w non-null,
//    fp32 scales only) each scale is multiplied by the row's routing weight
//    topk_w[row_assign[r]], which so scales the row's whole output.  One
//    thread per row reads its slot's contiguous scales; for a fixed kb,
//    consecutive threads write consecutive words.  A row id outside [0, T)
//    gets the word 0 (fp32 scale 0: a zero row; e8m0 codes 0: the scale
//    2^-127 on slot 0's payload), as does a weight index outside [0, n_assign).
//    With e8m0 codes the weights are not folded in (wtab non-null): row r's
//    weight goes to wtab[r] for the main kernel's epilogue.
//  * tile descriptors (workgroup 0, dispatched first, so its serial work runs
//    beside the gather instead of after the dispatch of every gather
//    workgroup): per local expert ceil(count / BM) row tiles times NT column
//    tiles, {expert, column tile, first row, valid rows | row tile << 9}, in
//    the main kernel's schedule order (slot it * G + my is tile it of
//    workgroup my; zero valid rows: an idle slot); tiles[0].x = number of
//    slots, tiles[1 + slot] = the descriptors.
template <int BM>
__global__ void __launch_bounds__(256)
gemm1_prep_kernel(const uint32_t* __restrict__ q_scale, const int32_t* __restrict__ row_slot,
                  const int32_t* __restrict__ row_assign, const float* __restrict__ topk_w, int64_t n_assign,
                  float* __restrict__ wtab,
                  const int32_t* __restrict__ expert_offsets, int L, int KB, int NT, int64_t T,
                  int64_t rows_cap, int64_t scale_ld, uint32_t* __restrict__ out, int4* __restrict__ tiles,
                  int64_t tiles_cap, int G) {
    MOE_TRACE_T0(tr0);
    if (blockIdx.x == 0) {
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
        // tile t of the natural order: experts in order, column tiles outer, row
        // tiles inner (the row tiles that share a weight slab adjacent)
        auto natural = [&](int t) __attribute__((always_inline)) {
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
            return int4{e, nt, r0, nvalid | (mtile << 9)};
        };
        const int nx = G / kXcds;                  // workgroups per XCD
        if (KB < kBalanceMinKb || G % kXcds != 0 || nx < 1 || nx > kPlanMaxNx || total > kPlanMaxTiles) {
            // plain round-robin over the natural order
            for (int t = tid; t < total; t += 256) tiles[1 + t] = natural(t);
            if (tid == 0) tiles[0] = int4{total, 0, 0, 0};
        } else {
            // Balanced static schedule.  Round r gives XCD x the natural tiles
            // [r * G + x * nx, + nx), as the plain round-robin does, so the row tiles
            // that share a weight slab run in one round on one XCD (together in its
            // L2).  Within the round they go to the XCD's workgroups so that the work
            // evens out: a partial tile (an expert's last rows) costs about 0.7 of a
            // full one (it streams its whole weight slab whatever its rows), so the
            // workgroups that have had the fewest partial tiles carry the most work.
            // The XCD keeps a cyclic pointer to the next of them: a round's partial
            // tiles go to the workgroups from the pointer on, its full tiles to the
            // rest, and the pointer moves past the partial ones (the costliest tile
            // to the least-loaded workgroup, as a longest-processing-time rule would
            // do with these two costs); in a round with fewer tiles than workgroups
            // (only the last) the idle slots (zero rows), which end their workgroups,
            // go first, to the most-loaded ones.  Slot (round r, workgroup (x, w)) is
            // descriptor 1 + r * G + x * nx + w.  Every tile's expert goes to LDS
            // first (each thread fills its experts' ranges), so a tile's descriptor
            // is a few reads and integer operations; then the rounds, in order, the
            // eight XCDs at once: wavefront wv, half h plans XCD wv + 4 h, lane j of
            // the half for the round's tile j.
            __shared__ uint16_t e_of[kPlanMaxTiles];
            for (int e = tid; e < L; e += 256)
                for (int t = tstart[e]; t < min(tstart[e + 1], total); ++t) e_of[t] = (uint16_t)e;
            __syncthreads();
            auto desc = [&](int t) __attribute__((always_inline)) {
                const int e = e_of[t];
                const int mt = (eoff[e + 1] - eoff[e] + BM - 1) / BM;
                const int local = t - tstart[e];
                const int nt = local / mt, mtile = local - nt * mt;
                const int r0 = eoff[e] + mtile * BM;
                return int4{e, nt, r0, min(BM, eoff[e + 1] - r0) | (mtile << 9)};
            };
            const int R = (total + G - 1) / G;                              // rounds
            const int half = lane >> 5, j = lane & 31;
            const int x = wv + 4 * half;
            const uint64_t half_mask = half ? 0xFFFFFFFF00000000ull : 0x00000000FFFFFFFFull;
            const uint64_t below = moe::lanemask_lt() & half_mask;         // this half's lanes below j
            int ptr = 0;                                                    // the XCD's cyclic pointer
            for (int r = 0; r < R; ++r) {
                const int c0 = r * G + x * nx;
                const int m = max(0, min(nx, total - c0));                  // tiles of this round
                const int4 d = j < m ? desc(c0 + j) : int4{0, 0, 0, 0};
                const bool part = j < m && (d.w & 511) < BM;
                const uint64_t pb = __ballot(part) & half_mask;
                const int kp = __popcll(pb), ip = __popcll(pb & below);     // partial tiles; this one's index
                const int idle = nx - m;
                int w;                                                      // the workgroup of lane j's slot
                if (j >= m) w = j - m;                                     // idle slots first
                else if (part) w = idle + ip;
                else w = idle + kp + (j - ip);
                w = (ptr + w) % nx;
                if (j < nx) tiles[1 + r * G + x * nx + w] = j < m ? d : int4{0, 0, 0, 0};
                ptr = (ptr + kp) % nx;
            }
            if (tid == 0) tiles[0] = int4{R * G, 0, 0, 0};
        }
        if (tid == 0) MOE_TRACE_PUT(moe::kTrGemmPrep, blockIdx.x, 0, 0, tr0);
        return;
    }
    int64_t R = expert_offsets[L];
    R = R < 0 ? 0 : (R > rows_cap ? rows_cap : R);
    // work item = (row, group of kPrepKb K blocks); consecutive items are
    // consecutive rows of one group, so every store instruction is contiguous
    const int KG = (KB + kPrepKb - 1) / kPrepKb;
    const int64_t nthr = (int64_t)(gridDim.x - 1) * 256;
    for (int64_t item = (int64_t)(blockIdx.x - 1) * 256 + threadIdx.x; item < R * KG; item += nthr) {
        const int kg = (int)(item / R);
        const int64_t r = item - (int64_t)kg * R;
        const int s = row_slot ? row_slot[r] : (int)r;
        bool ok = (uint64_t)s < (uint64_t)T;
        float wr = 1.0f;
        if (topk_w) {
            const int ra = row_assign[r];
            ok = ok && (uint64_t)ra < (uint64_t)n_assign;
            wr = ok ? topk_w[ra] : 0.0f;
        }
        const uint32_t* src = q_scale + (int64_t)(ok ? s : 0) * KB;
        const int k0 = kg * kPrepKb;
        uint32_t v[kPrepKb];
#pragma unroll
        for (int i = 0; i < kPrepKb; ++i) v[i] = (ok && k0 + i < KB) ? src[k0 + i] : 0u;
        if (topk_w && !wtab) {
#pragma unroll
            for (int i = 0; i < kPrepKb; ++i) v[i] = __float_as_uint(__uint_as_float(v[i]) * wr);
        }
        if (wtab && kg == 0) wtab[r] = wr;
#pragma unroll
        for (int i = 0; i < kPrepKb; ++i)
            if (k0 + i < KB) out[(int64_t)(k0 + i) * scale_ld + r] = v[i];
    }
    if (threadIdx.x == 0) MOE_TRACE_PUT(moe::kTrGemmPrep, blockIdx.x, 1, 0, tr0);
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

// The fold one column group later, with the MFMA / fold units fenced in
// order, measured fastest (about 10 % over folding each product at once, where
// the wavefront waits on its own MFMA's result).
using TileCfg = Cfg<128, 2, 4, 4, 3>;
static_assert(TileCfg::BM <= kMaxBM, "scale table padding covers one tile");

// Workspace: the row-scale table, then the tile descriptors (16 B each; the
// schedule may hold up to kMaxGrid idle slots beyond the tiles).
struct WsLayout {
    int64_t scale_ld, table_bytes, tiles_cap, wtab_off, bytes;
};
// rows_cap expert-major rows, KB K blocks, n output columns, L experts; with
// row weights (GEMM2), a float per row after the descriptors (256 B aligned)
WsLayout ws_layout(int64_t rows_cap, int64_t KB, int64_t n, int64_t L, bool row_weights) {
    WsLayout l;
    l.scale_ld = scale_ld_of(rows_cap);
    l.table_bytes = (KB * l.scale_ld * 4 + 255) & ~int64_t(255);
    l.tiles_cap = (rows_cap / kMinBM + L) * ((n + BN - 1) / BN);
    l.wtab_off = (l.table_bytes + (1 + l.tiles_cap + kMaxGrid) * 16 + 255) & ~int64_t(255);
    l.bytes = row_weights ? l.wtab_off + rows_cap * 4 : l.table_bytes + (1 + l.tiles_cap + kMaxGrid) * 16;
    return l;
}

// One grouped-GEMM call: y[r, c] = sum_k A[r, k] * B[e(r), c, k], K = kdim,
// c < n, for the rows_cap-capacity expert-major rows.  A row r is q[row_slot[r]]
// (q has a_rows rows) or, with DIRECT, q[r].  q_scale and w_scale are fp32
// scales or packed e8m0 codes (MX).  Row weights (row_assign, topk_w) scale
// each row's output (fp32 path only).
template <bool MX, bool DIRECT>
moe_status run_gemm(const moe::Dims& d, int64_t a_rows, int64_t kdim, int64_t n, const uint8_t* q_e4m3,
                    const uint32_t* q_scale, const int32_t* row_slot, const int32_t* row_assign,
                    const float* topk_w, const int32_t* expert_offsets, const uint8_t* w_e4m3,
                    const void* w_scale, uint16_t* y_bf16, void* ws, size_t ws_bytes, void* hip_stream) {
    if (n < 128 || n % 128 != 0 || kdim < 128 || kdim % 128 != 0) return MOE_ERR_INVALID_ARG;
    if (d.L > kMaxL) return MOE_ERR_UNSUPPORTED;
    if (d.T == 0) return MOE_OK;
    if (!q_e4m3 || !q_scale || (!DIRECT && !row_slot) || !expert_offsets || !w_e4m3 || !w_scale || !y_bf16)
        return MOE_ERR_INVALID_ARG;
    if ((topk_w != nullptr) != (row_assign != nullptr)) return MOE_ERR_INVALID_ARG;
    const int64_t rows_cap = d.T * d.k;
    // 32-bit offsets inside the kernel: rows of q, rows of one expert's weight;
    // row tile ids in 22 bits of a descriptor
    if (a_rows * kdim >= ((int64_t)1 << 32) || n * kdim >= ((int64_t)1 << 31) ||
        rows_cap * n >= ((int64_t)1 << 40) || rows_cap / kMinBM >= ((int64_t)1 << 22))
        return MOE_ERR_UNSUPPORTED;
    const int64_t KB = kdim / BK;
    const WsLayout wl = ws_layout(rows_cap, KB, n, d.L, DIRECT);
    if (!ws || ws_bytes < (size_t)wl.bytes) return MOE_ERR_WORKSPACE;
    if (KB * wl.scale_ld >= ((int64_t)1 << 31) || wl.tiles_cap >= ((int64_t)1 << 31) - 1)
        return MOE_ERR_UNSUPPORTED;
    int cus = cu_count();
    if (cus <= 0) return MOE_ERR_HIP;
    hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
    uint32_t* row_scale = reinterpret_cast<uint32_t*>(ws);
    int4* tiles = reinterpret_cast<int4*>(static_cast<uint8_t*>(ws) + wl.table_bytes);
    // MX GEMM2's per-row weights (the fp32 path folds them into the row scales)
    float* wtab = (MX && DIRECT) ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + wl.wtab_off) : nullptr;
    const int NT = (int)((n + BN - 1) / BN);
    // the planning workgroup (the first one) plus the gather workgroups; the
    // gather loop strides over the grid, so its size is capped at four
    // workgroups a CU (the row count R, read on the device, is usually far
    // below rows_cap)
    const int64_t KG = (KB + kPrepKb - 1) / kPrepKb;
    const int pgrid = (int)std::min<int64_t>((rows_cap * KG + 255) / 256, kPrepWgPerCu * (int64_t)cus) + 1;
    using C = TileCfg;
    const int grid = ((cus + kXcds - 1) / kXcds) * kXcds;
    if (grid > kMaxGrid) return MOE_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((gemm1_prep_kernel<C::BM>), dim3(pgrid), dim3(256), 0, stream, q_scale,
                       DIRECT ? nullptr : row_slot, row_assign, topk_w, rows_cap, wtab, expert_offsets, (int)d.L,
                       (int)KB, NT, a_rows, rows_cap, wl.scale_ld, row_scale, tiles, wl.tiles_cap, grid);
    moe_status st;
    if ((st = moe::launch_status()) != MOE_OK) return st;
    hipLaunchKernelGGL((grouped_gemm1_kernel<C, MX, DIRECT>), dim3(grid), dim3(C::kThreads), 0,
                       stream, q_e4m3, row_scale, tiles, row_slot, w_e4m3, w_scale, y_bf16, (int)n, (int)kdim,
                       a_rows, wl.scale_ld, wtab);
    return moe::launch_status();
}

moe_status load(const moe_dims* dims, moe::Dims* d) { return moe::load_dims(dims, d, true); }

}  // namespace

extern "C" moe_status moe_grouped_gemm1_workspace(const moe_dims* dims, int32_t n, size_t* bytes) {
    moe::Dims d;
    moe_status st = load(dims, &d);
    if (st != MOE_OK) return st;
    if (!bytes || n < 128 || n % 128 != 0) return MOE_ERR_INVALID_ARG;
    *bytes = (size_t)ws_layout(d.T * d.k, d.H / BK, n, d.L, false).bytes;
    return MOE_OK;
}

extern "C" moe_status moe_grouped_gemm1(const moe_dims* dims, int32_t n, const uint8_t* q_e4m3,
                                        const float* q_scale, const int32_t* row_slot,
                                        const int32_t* expert_offsets, const int32_t* totals,
                                        const uint8_t* w_e4m3, const float* w_scale, uint16_t* y_bf16,
                                        void* ws, size_t ws_bytes, void* hip_stream) {
    (void)totals;
    moe::Dims d;
    moe_status st = load(dims, &d);
    if (st != MOE_OK) return st;
    return run_gemm<false, false>(d, d.T, d.H, n, q_e4m3, reinterpret_cast<const uint32_t*>(q_scale), row_slot,
                                  nullptr, nullptr, expert_offsets, w_e4m3, w_scale, y_bf16, ws, ws_bytes,
                                  hip_stream);
}

extern "C" moe_status moe_grouped_gemm1_mx(const moe_dims* dims, int32_t n, const uint8_t* q_e4m3,
                                           const uint32_t* q_scale, const int32_t* row_slot,
                                           const int32_t* expert_offsets, const uint8_t* w_e4m3,
                                           const uint32_t* w_scale, uint16_t* y_bf16, void* ws,
                                           size_t ws_bytes, void* hip_stream) {
    moe::Dims d;
    moe_status st = load(dims, &d);
    if (st != MOE_OK) return st;
    return run_gemm<true, false>(d, d.T, d.H, n, q_e4m3, q_scale, row_slot, nullptr, nullptr, expert_offsets,
                                 w_e4m3, w_scale, y_bf16, ws, ws_bytes, hip_stream);
}

extern "C" moe_status moe_grouped_gemm2_workspace(const moe_dims* dims, int32_t inter, size_t* bytes) {
    moe::Dims d;
    moe_status st = load(dims, &d);
    if (st != MOE_OK) return st;
    if (!bytes || inter < 128 || inter % 128 != 0) return MOE_ERR_INVALID_ARG;
    *bytes = (size_t)ws_layout(d.T * d.k, inter / BK, d.H, d.L, true).bytes;
    return MOE_OK;
}

extern "C" moe_status moe_grouped_gemm2(const moe_dims* dims, int32_t inter, const uint8_t* h_e4m3,
                                        const float* h_scale, const int32_t* expert_offsets,
                                        const int32_t* row_assign, const float* topk_w,
                                        const uint8_t* w2_e4m3, const float* w2_scale, uint16_t* y2_bf16,
                                        void* ws, size_t ws_bytes, void* hip_stream) {
    moe::Dims d;
    moe_status st = load(dims, &d);
    if (st != MOE_OK) return st;
    if (d.T != 0 && (!row_assign || !topk_w)) return MOE_ERR_INVALID_ARG;
    return run_gemm<false, true>(d, d.T * d.k, inter, d.H, h_e4m3, reinterpret_cast<const uint32_t*>(h_scale),
                                 nullptr, row_assign, topk_w, expert_offsets, w2_e4m3, w2_scale, y2_bf16, ws,
                                 ws_bytes, hip_stream);
}

extern "C" moe_status moe_grouped_gemm2_mx(const moe_dims* dims, int32_t inter, const uint8_t* h_e4m3,
                                           const uint32_t* h_scale, const int32_t* expert_offsets,
                                           const int32_t* row_assign, const float* topk_w,
                                           const uint8_t* w2_e4m3, const uint32_t* w2_scale, uint16_t* y2_bf16,
                                           void* ws, size_t ws_bytes, void* hip_stream) {
    moe::Dims d;
    moe_status st = load(dims, &d);
    if (st != MOE_OK) return st;
    if (d.T != 0 && (!row_assign || !topk_w)) return MOE_ERR_INVALID_ARG;
    return run_gemm<true, true>(d, d.T * d.k, inter, d.H, h_e4m3, h_scale, nullptr, row_assign, topk_w,
                                expert_offsets, w2_e4m3, w2_scale, y2_bf16, ws, ws_bytes, hip_stream);
}
