/*
 * moe_hotpath.h - C ABI of the MoE expert-dispatch hot path on one MI355X.
 *
 * One GPU's share of an expert-parallel MoE layer: the tokens of S source
 * regions (the stand-in for the S peer ranks whose rows would land here) are
 * routed top-k over E experts, of which this GPU owns [e0, e0+L).  Four steps:
 *
 *   1. moe_route_layout   - stable counting sort of the (token, expert)
 *                           assignments into an expert-major row layout with
 *                           a rowmap and a compact landed-token slot list.
 *   2. moe_quant_dispatch - each landed token's bf16 row is read once and
 *                           quantised to fp8 e4m3 with 1x128 block scales into
 *                           its slot.
 *   3. moe_grouped_gemm1  - per local expert, Y1 = A * W with A's rows read in
 *                           place through the rowmap.
 *   4. moe_combine        - top-k weighted sum of expert outputs back to token
 *                           order.
 *
 * Pages this follows (the text of each is the authority on what is computed):
 *   "poc(cco): MegaMoE stage1 dispatch over SDMA" (mori pull request 1):
 *     "What", "How it works now", and the commits "each token read and
 *     quantised once", "recv_layout", "ready-first / quant-lds-store".
 *   "EPDispatchKernel" (Mojo ep_comm): wait_for_arrivals_and_compute_offsets,
 *     copy_received_tokens_to_output.
 *   "TilePipe": dispatch / push combine kernels.
 *
 * Conventions for every call:
 *   - Every array argument is a DEVICE pointer owned by the caller.  The
 *     library allocates, frees and synchronises nothing and keeps no state
 *     between calls; work is enqueued on `hip_stream` (a hipStream_t, NULL for
 *     the default stream) and the call returns without waiting for it.
 *   - Counts produced on the device (totals, expert_offsets) stay there; the
 *     later calls read them on the device, so the four calls can be captured
 *     in one graph with no host read-back.
 *   - Returned status codes cover argument validation and launch errors only.
 *     A fault inside a kernel surfaces at the caller's next synchronisation.
 *   - Calls are re-entrant.  Calls in flight at the same time need distinct
 *     output and workspace buffers.
 *   - Notation: T = S*Ts tokens; global token g = s*Ts + t; R = number of
 *     local assignments (rows); U = number of landed tokens (slots).
 */
#ifndef MOE_HOTPATH_H
#define MOE_HOTPATH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_dims {
    int32_t num_sources;        /* S  >= 1                                      */
    int32_t tokens_per_source;  /* Ts >= 0                                      */
    int32_t top_k;              /* k, 1 <= k <= num_experts                     */
    int32_t num_experts;        /* E  >= 1                                      */
    int32_t expert_begin;       /* e0 >= 0, first local expert                  */
    int32_t num_local_experts;  /* L, 1 <= L, e0 + L <= E, L <= 1024            */
    int32_t hidden;             /* H, multiple of 128 (the quant block)         */
} moe_dims;

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,   /* null pointer, size out of range, bad dims   */
    MOE_ERR_WORKSPACE = -2,     /* workspace missing or smaller than required  */
    MOE_ERR_UNSUPPORTED = -3,   /* valid but outside what the kernels support  */
    MOE_ERR_HIP = -4            /* a HIP launch returned an error              */
} moe_status;

/* Human-readable name of a status code (static storage). */
const char* moe_status_string(moe_status status);

/*
 * Buffer capacities for the layout's outputs.
 *   rows_cap  = T*k  (upper bound of R; a token naming one expert twice gets two
 *               rows, so R can exceed T)
 *   slots_cap = T    (upper bound of U)
 * Host-only; no GPU work.
 */
moe_status moe_capacity(const moe_dims* dims, int64_t* rows_cap, int64_t* slots_cap);

/* Workspace bytes moe_route_layout needs for these dims (host-only). */
moe_status moe_route_layout_workspace(const moe_dims* dims, size_t* bytes);

/*
 * Step 1: layout.  Stable counting sort of the local assignments by local
 * expert ("MegaMoE stage1 dispatch over SDMA", commit "recv_layout": the
 * receiver counts the routes per expert and writes the rowmap and srcmap
 * tables; "EPDispatchKernel", wait_for_arrivals_and_compute_offsets: the
 * per-local-expert offsets).  Rows of one expert are contiguous and in
 * ascending (g, j); experts are not padded.
 *
 * In:  topk_ids   int32 [T, k] row-major; id - e0 in [0, L) is local, any other
 *                 value (negative too) is skipped.
 * Out (all int32):
 *      expert_counts    [L]       rows per local expert
 *      expert_offsets   [L+1]     exclusive prefix of expert_counts; [L] = R
 *      row_slot         [rows_cap] rowmap: row r -> slot of its token (0..U-1)
 *      row_assign       [rows_cap] row r -> assignment index g*k + j
 *      assign_row       [T*k]     assignment -> row, -1 if not local
 *      tok_slot         [T]       token -> slot, -1 if the token has no local
 *                                 assignment
 *      slot_tok         [slots_cap] slot u -> token g, ascending in g
 *      src_slot_offsets [S+1]     first slot of each source region; [S] = U
 *      totals           [2]       {R, U}
 * Entries of row_slot / row_assign past R and of slot_tok past U are not
 * written.  ws: device workspace of at least moe_route_layout_workspace bytes.
 */
moe_status moe_route_layout(const moe_dims* dims, const int32_t* topk_ids,
                            int32_t* expert_counts, int32_t* expert_offsets,
                            int32_t* row_slot, int32_t* row_assign, int32_t* assign_row,
                            int32_t* tok_slot, int32_t* slot_tok, int32_t* src_slot_offsets,
                            int32_t* totals, void* ws, size_t ws_bytes, void* hip_stream);

/*
 * Allocation-free variant of moe_route_layout, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, outputs and results as
 * moe_route_layout, without the workspace: the layout's histogram and landed
 * counts live in a static device array of the library, 256 KiB per GPU,
 * held on each GPU the library runs on until the process ends.
 *   - The call allocates nothing; its first call on a device looks up that
 *     device's copy of the array (no allocation).
 *   - Returns MOE_ERR_WORKSPACE when the layout needs more than the array holds
 *     (moe_route_layout_workspace(dims) > 262144 bytes; every configuration
 *     with T*L <= 2^22 fits, e.g. 16384 tokens over 256 local experts uses
 *     132 KiB).  Nothing is launched then.
 *   - Every call on one GPU uses that GPU's one array: calls that overlap in
 *     time on one GPU (on different streams, or from different host threads)
 *     race and give undefined results; serialise them, e.g. on one stream.
 *     The array needs no clearing: each call writes every entry it reads.
 */
moe_status moe_route_layout_noalloc(const moe_dims* dims, const int32_t* topk_ids,
                                    int32_t* expert_counts, int32_t* expert_offsets,
                                    int32_t* row_slot, int32_t* row_assign, int32_t* assign_row,
                                    int32_t* tok_slot, int32_t* slot_tok, int32_t* src_slot_offsets,
                                    int32_t* totals, void* hip_stream);

/*
 * Step 2: quant + dispatch.  Each landed token's row is read once and
 * quantised once into its slot ("MegaMoE stage1 dispatch over SDMA", commit
 * "each token read and quantised once"; "How it works now": the quant writes
 * each row once, one contiguous 16 B per lane).
 *
 * For slot u < U (U read from totals[1] on the device), token g = slot_tok[u],
 * and block b < H/128:
 *   a = max |x[g, 128b .. 128b+127]|;  s = a / 448 (IEEE fp32 division);
 *   q[u, 128b+i] = e4m3(x[g,128b+i] / s) (IEEE division, round to nearest
 *   even, saturating at 448, sign kept on zero);  q_scale[u, b] = s;
 *   a == 0 gives s = 0 and zero bytes.
 * In:  x_bf16  uint16 (bf16 bits) [T, H];  slot_tok, totals from step 1.
 * Out: q_e4m3  uint8 [slots_cap, H];  q_scale float32 [slots_cap, H/128].
 * Rows past U are not written.
 */
moe_status moe_quant_dispatch(const moe_dims* dims, const uint16_t* x_bf16,
                              const int32_t* slot_tok, const int32_t* totals,
                              uint8_t* q_e4m3, float* q_scale, void* hip_stream);

/* Workspace bytes moe_grouped_gemm1 needs (host-only): a K-block-major table of
 * the rows' activation scales, (H/128) x (rows_cap + 256, rounded up to 64) floats
 * (padded to 256 B), then 16 B tile descriptors, (1 + (rows_cap/128 + L) *
 * ceil(n/256) + 1024) of them (the tile schedule's slots, idle ones
 * included).  Both are rewritten by every call. */
moe_status moe_grouped_gemm1_workspace(const moe_dims* dims, int32_t n, size_t* bytes);

/*
 * Step 3: grouped GEMM1 over the local experts, A rows read in place through
 * the rowmap ("MegaMoE stage1 dispatch over SDMA", "What" and commit 1: GEMM1
 * reads its fp8 A rows and their block scales through a rowmap).
 *
 * For local expert le, row r in [expert_offsets[le], expert_offsets[le+1]) and
 * column c < n:
 *   y[r, c] = bf16( sum_h  q[row_slot[r], h] * q_scale[row_slot[r], h/128]
 *                        * w[le, c, h]    * w_scale[le, c/128, h/128] )
 * accumulated in fp32 (fp8 MFMA per 128-wide K block, then scaled).
 * In:  q_e4m3, q_scale from step 2; row_slot, expert_offsets from step 1
 *      (expert_offsets is read on the device: R = expert_offsets[L]);
 *      totals: accepted for symmetry with the other calls and not read (may
 *      be NULL);
 *      w_e4m3  uint8 [L, n, H]  (each expert's weight stored K-contiguous:
 *              element (h, c) of the logical [H, n] weight at [le, c, h]);
 *      w_scale float32 [L, n/128, H/128]  one scale per 128x128 block.
 * Out: y_bf16 uint16 (bf16 bits) [rows_cap, n]; rows past R are not written.
 * ws: device workspace of at least moe_grouped_gemm1_workspace bytes (its
 * contents need no initialisation; the call rewrites what it reads).
 * n must be a positive multiple of 128.  Row ids outside [0, T) read as zero
 * rows (they cannot come from step 1).
 */
moe_status moe_grouped_gemm1(const moe_dims* dims, int32_t n,
                             const uint8_t* q_e4m3, const float* q_scale,
                             const int32_t* row_slot, const int32_t* expert_offsets,
                             const int32_t* totals,
                             const uint8_t* w_e4m3, const float* w_scale,
                             uint16_t* y_bf16, void* ws, size_t ws_bytes, void* hip_stream);

/*
 * MX-style variants of steps 2 and 3: fp8 e4m3 payloads with power-of-two
 * (e8m0) scales per 32 consecutive hidden elements, the scales applied by the
 * matrix cores' block-scale operands ("poc(cco): MegaMoE stage1 dispatch over
 * SDMA", "Where we stand": the stage1 runs use e8m0 block scales; commit
 * "ready-first / quant-lds-store": four e8m0 codes packed per dword).  The
 * pages fix neither the scale rule nor the packing order; the reading taken:
 *
 * For slot u < U, token g = slot_tok[u], group j < H/32 (elements 32j .. 32j+31):
 *   a = max |x[g, group j]|;  a == 0: E = -127 and zero bytes;
 *   else t = a / 448 (IEEE fp32), E = ceil(log2 t) exactly (an exact power of
 *   two keeps its exponent), clamped to [-127, 127];
 *   q[u, 32j+i] = e4m3(x[g, 32j+i] * 2^-E)  (the scaling is exact; round to
 *   nearest even; never above 448 in magnitude; sign kept on zero);
 *   code = E + 127 (e8m0: value 2^(code-127));
 *   q_scale[u, b] = codes of groups 4b, 4b+1, 4b+2, 4b+3 in bytes 0, 1, 2, 3.
 * In:  as moe_quant_dispatch.
 * Out: q_e4m3 uint8 [slots_cap, H];  q_scale uint32 [slots_cap, H/128].
 * Rows past U are not written.
 */
moe_status moe_quant_dispatch_mx(const moe_dims* dims, const uint16_t* x_bf16,
                                 const int32_t* slot_tok, const int32_t* totals,
                                 uint8_t* q_e4m3, uint32_t* q_scale, void* hip_stream);

/*
 * MX GEMM1: as moe_grouped_gemm1 with both operands' scales per 32-element K
 * group: for local expert le, row r of it, column c < n,
 *   y[r, c] = bf16( sum_h  q[row_slot[r], h] * 2^(Ea(row_slot[r], h/32))
 *                        * w[le, c, h]    * 2^(Eb(le, c, h/32)) )
 * accumulated in fp32 by the fp8 MFMA with its e8m0 block-scale operands.
 * In:  q_e4m3, q_scale (uint32 [slots_cap, H/128]) from moe_quant_dispatch_mx;
 *      row_slot, expert_offsets from step 1 (read on the device);
 *      w_e4m3  uint8 [L, n, H] (as moe_grouped_gemm1);
 *      w_scale uint32 [L, H/128, n]: the packed codes of column c's groups
 *              4kb .. 4kb+3 at [le, kb, c] (K-block-major, so one K block's
 *              scales for consecutive columns are contiguous).
 * Out: y_bf16 uint16 (bf16 bits) [rows_cap, n]; rows past R are not written.
 * ws: the workspace moe_grouped_gemm1_workspace sizes for (dims, n).
 * n must be a positive multiple of 128.  A row id outside [0, T) (which step 1
 * cannot produce) reads slot 0's payload with the scale 2^-127: no access
 * leaves the buffers, and that row's values are not specified.
 */
moe_status moe_grouped_gemm1_mx(const moe_dims* dims, int32_t n,
                                const uint8_t* q_e4m3, const uint32_t* q_scale,
                                const int32_t* row_slot, const int32_t* expert_offsets,
                                const uint8_t* w_e4m3, const uint32_t* w_scale,
                                uint16_t* y_bf16, void* ws, size_t ws_bytes, void* hip_stream);

/*
 * Stage2 (after GEMM1), the expert MLP's second half ("poc(cco): MegaMoE
 * stage1 dispatch over SDMA", "What": stage1's output feeds stage2 + combine;
 * commit "recv_layout": the layout's per-row routing weights serve stage2).
 * The pages do not state stage2's arithmetic; the reading: GEMM1's width is
 * n = 2*inter, columns [0, inter) the gate and [inter, 2*inter) the up
 * projection of the same row.
 *
 * moe_silu_mul_quant: for expert-major row r < R (R = totals[0], read on the
 * device) and i < inter:
 *   h[r, i] = silu(gate) * up,  silu(x) = x / (1 + e^-x), in fp32 from the
 *   bf16 inputs (the exponential and reciprocal are the hardware's
 *   approximations: h carries a few fp32 ulps of error);
 * then GEMM1's quant rule per block b of 128 elements of h: s = amax / 448
 * (IEEE), q = e4m3(h / s) (IEEE quotient, round to nearest even; exact given
 * the kernel's h), a == 0 giving s = 0 and zero bytes.
 * In:  y1_bf16 uint16 (bf16 bits) [rows_cap, 2*inter] (GEMM1's output);
 *      totals from step 1.
 * Out: h_e4m3 uint8 [rows_cap, inter]; h_scale float32 [rows_cap, inter/128].
 * Rows past R are not written.  inter must be a positive multiple of 128.
 */
moe_status moe_silu_mul_quant(const moe_dims* dims, int32_t inter, const uint16_t* y1_bf16,
                              const int32_t* totals, uint8_t* h_e4m3, float* h_scale,
                              void* hip_stream);

/* Workspace bytes moe_grouped_gemm2 and moe_grouped_gemm2_mx need (host-only):
 * the K-block-major row scale table, (inter/128) x (rows_cap + 256, rounded up
 * to 64) words (padded to 256 B), then (1 + (rows_cap/128 + L) * ceil(H/256) +
 * 1024) 16 B tile descriptors (as GEMM1's), then (from a 256 B boundary) one
 * float per row. */
moe_status moe_grouped_gemm2_workspace(const moe_dims* dims, int32_t inter, size_t* bytes);

/*
 * GEMM2: the grouped down projection, each row scaled by its routing weight
 * (the pages' per-row weights table of the layout).  For local expert le, row
 * r in [expert_offsets[le], expert_offsets[le+1]) and column c < H:
 *   y2[r, c] = bf16( w_r * sum_i  h[r, i] * h_scale[r, i/128]
 *                                * w2[le, c, i] * w2_scale[le, c/128, i/128] )
 *   w_r = topk_w[row_assign[r]]   (flat index g*k + j of the row's assignment)
 * accumulated in fp32 (fp8 MFMA per 128-wide K block; w_r folded into the
 * row's scales).  A rows are the expert-major rows themselves (row r reads
 * h row r, no rowmap).
 * In:  h_e4m3, h_scale from moe_silu_mul_quant; expert_offsets, row_assign
 *      from step 1 (a layout of the same dims); topk_w float32 [T, k];
 *      w2_e4m3  uint8 [L, H, inter] (element (i, c) of the logical [inter, H]
 *               weight at [le, c, i], K-contiguous);
 *      w2_scale float32 [L, H/128, inter/128], one per 128x128 block.
 * Out: y2_bf16 uint16 (bf16 bits) [rows_cap, H]; rows past R are not written.
 * ws: device workspace of at least moe_grouped_gemm2_workspace bytes.
 * A row_assign entry outside [0, T*k) gives that row weight 0 (it cannot
 * come from step 1).
 */
moe_status moe_grouped_gemm2(const moe_dims* dims, int32_t inter,
                             const uint8_t* h_e4m3, const float* h_scale,
                             const int32_t* expert_offsets, const int32_t* row_assign,
                             const float* topk_w,
                             const uint8_t* w2_e4m3, const float* w2_scale,
                             uint16_t* y2_bf16, void* ws, size_t ws_bytes, void* hip_stream);

/*
 * MX variants of stage2 (the pages' e8m0 format, as moe_quant_dispatch_mx and
 * moe_grouped_gemm1_mx):
 *
 * moe_silu_mul_quant_mx: h as in moe_silu_mul_quant, quantised per group of
 * 32 elements: E = ceil(log2(max|h| / 448)) exactly from the fp32 quotient
 * (clamped to [-127, 127]; an all-zero group -127 with zero bytes), payload
 * e4m3(h * 2^-E); the codes E + 127 of a 128-element block packed into one
 * uint32 (group g of the block in byte g).
 * Out: h_e4m3 uint8 [rows_cap, inter]; h_scale uint32 [rows_cap, inter/128].
 *
 * moe_grouped_gemm2_mx: y2 as in moe_grouped_gemm2 with e8m0 group scales on
 * both operands (w2_scale uint32 [L, inter/128, H]: the packed codes of column
 * c's groups 4kb .. 4kb+3 at [le, kb, c]); the routing weight w_r multiplies
 * the fp32 sum before the bf16 rounding (it is not a power of two, so it
 * cannot ride in the codes).  ws: moe_grouped_gemm2_workspace bytes.
 */
moe_status moe_silu_mul_quant_mx(const moe_dims* dims, int32_t inter, const uint16_t* y1_bf16,
                                 const int32_t* totals, uint8_t* h_e4m3, uint32_t* h_scale,
                                 void* hip_stream);

moe_status moe_grouped_gemm2_mx(const moe_dims* dims, int32_t inter,
                                const uint8_t* h_e4m3, const uint32_t* h_scale,
                                const int32_t* expert_offsets, const int32_t* row_assign,
                                const float* topk_w,
                                const uint8_t* w2_e4m3, const uint32_t* w2_scale,
                                uint16_t* y2_bf16, void* ws, size_t ws_bytes, void* hip_stream);

/*
 * Step 4: combine.  Top-k weighted gather-sum back to token order (TilePipe:
 * push combine to the token owners; "MegaMoE stage1 dispatch over SDMA",
 * "What": stage2 + combine).
 *
 * For token g < T and column c < width:
 *   acc = 0 (fp32); for j = 0..k-1: r = assign_row[g*k+j];
 *   if 0 <= r < y_rows: acc += topk_w[g*k+j] * y[r, c];
 *   out[g, c] = bf16(acc)  (round to nearest even)
 * In:  y_bf16 uint16 [y_rows, width]; assign_row int32 [T*k] (from step 1 of a
 *      layout whose rows index y); topk_w float32 [T, k].
 * Out: out_bf16 uint16 [T, width].
 * width must be a positive multiple of 8.
 */
moe_status moe_combine(const moe_dims* dims, int32_t width, const uint16_t* y_bf16,
                       int64_t y_rows, const int32_t* assign_row, const float* topk_w,
                       uint16_t* out_bf16, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_HOTPATH_H */
