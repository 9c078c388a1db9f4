/*
 * moe_dc.h -- C ABI of the MI355X (gfx950) MoE routing / dispatch / combine
 * library (libmoe_dc.so).
 *
 * The path: softmax top-k routing -> per-expert counting and prefix sum ->
 * stable scatter of token rows into contiguous expert-major buffers
 * (optionally grouped into segment-major blocks) -> expert compute -> weighted
 * top-k gather-sum back to token order.
 *
 * Sources of the operations (cited by page title and section):
 *   [MLX-EP]  "MLX expert parallelism all_to_all PR 3158", Facts list: the
 *             O(N*D) data-movement kernels dispatch_local, packet_gather,
 *             packet_scatter, combine_weighted_sum; dispatch/combine
 *             round-trip tests; no GPU sync in the middle of a primitive.
 *   [ET-PR]   "backends/mlx: runtime MoE expert-sort for decode (issue
 *             #20554)": Summary (one artifact serves sorted prefill and
 *             unsorted decode); reviews' correctness notes (switch
 *             cond = (M-1) // sort_cutoff; both branches emit the same N*top_k
 *             shape; outputs never alias inputs); author's follow-up "Handler
 *             fixes" (flatten [N, top_k] before a stable argsort, int32
 *             indices, token = order // top_k; the sorted flag of gather_mm is
 *             a caller's promise that rows are grouped, not a request to
 *             sort); CI write-up (unsorted inv_order = identity arange(N*k);
 *             unsorted rows = x.repeat_interleave(top_k)).
 *   [1SIDED]  "One-Sided Expert-Parallel All-to-All for Mixture-of-Experts
 *             Inference over NVLink", abstract: rank-major (here
 *             segment-major) buffers that grouped GEMMs read in place; the
 *             interface is agnostic to the activation quantisation format;
 *             fixed costs dominate small batches.
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless marked [host].  Buffers are
 *     row-major and contiguous.  Indices are int32.
 *   - The caller owns every buffer, including the workspace.  The library
 *     allocates no device memory, keeps no pointer after a call returns and
 *     has no global mutable state except the per-thread last-error string.
 *   - Every call enqueues its kernels on `stream` (a hipStream_t; NULL is the
 *     null stream) and returns without waiting.  Outputs are valid in stream
 *     order.  No call synchronises with the host, except in validate mode
 *     (environment variable MOE_DC_VALIDATE=1), where moe_dispatch and
 *     moe_route_dispatch wait for their kernels and report out-of-range
 *     expert ids as MOE_ERR_ARG (and a row copy that gave up waiting for its
 *     positions, see moe_dispatch, as MOE_ERR_HIP).
 *   - Outputs must not alias inputs.
 *   - Errors are returned as a status code before any kernel is launched;
 *     moe_last_error() describes the last failure on the calling thread.  No
 *     C++ exception crosses the ABI.
 *   - Kernels never read or write outside the buffers described below, also
 *     for out-of-range expert ids or positions: such entries are skipped and
 *     the corresponding outputs are unspecified.
 *
 * Symbols: N tokens, D hidden size, E experts, k experts per token, G
 * segments (E % G == 0; segment g holds experts [g*E/G, (g+1)*E/G)),
 * NK = N*k routed pairs, pair q = t*k + j (token t, slot j).
 */
#ifndef MOE_DC_H
#define MOE_DC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_DC_ABI_VERSION 1

/* Element types.  MOE_F8E4M3 is the OCP 8-bit E4M3FN format (bias 7, max 448,
 * no infinities); an F8 payload always travels with float32 scales, one per
 * 128 consecutive elements of a row ([1SIDED]: the data movement does not
 * look inside the activation format). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_F8E4M3 = 2 } moe_dtype;

/* Status codes. */
enum {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,          /* null required pointer, size out of range, bad enum value */
  MOE_ERR_UNSUPPORTED = 2,  /* a size or type combination outside what this library implements */
  MOE_ERR_WORKSPACE = 3,    /* workspace too small or misaligned */
  MOE_ERR_HIP = 4           /* a HIP launch or runtime call failed */
};

/* Sort modes of moe_dispatch ([ET-PR] reviews: the runtime sorted flag). */
enum { MOE_SORT_AUTO = -1, MOE_SORT_OFF = 0, MOE_SORT_ON = 1 };

/* Limits of this implementation. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 64

/* ABI version (MOE_DC_ABI_VERSION of the built library). */
int moe_abi_version(void);

/* Message of the last failed call on this thread ("" if none).  The pointer
 * stays valid until the next library call on the same thread. */
const char* moe_last_error(void);

/* ---------------------------------------------------------------- routing
 * moe_route_topk -- softmax top-k gating.
 *
 * Produces the routing output expert_indices [N, k] that [ET-PR] (follow-up
 * "Handler fixes") flattens and sorts, plus fp32 routing weights.
 * Per token t: the k largest logits in the total order (value descending,
 * then expert index ascending; -0.0 == +0.0) go to slots 0..k-1, slot 0 the
 * best.  Weights, with l_j the selected logits:
 *   renormalize != 0: w_j = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0)
 *   renormalize == 0: w_j = exp(l_j - m) / sum_{e<E} exp(l_e - m), m = l_0.
 * fp32 arithmetic with the accurate device expf.  NaN logits are outside the
 * contract (they do not fault, the result is unspecified).
 *
 *   logits    [N, E] float32
 *   topk_idx  [N, k] int32, output
 *   topk_w    [N, k] float32, output
 * Errors: MOE_ERR_ARG for null pointers (unless N == 0), N < 0, E < 1,
 * k < 1 or k > E; MOE_ERR_UNSUPPORTED for E > MOE_MAX_EXPERTS or
 * k > MOE_MAX_TOPK.  N == 0 is a no-op. */
int moe_route_topk(const float* logits, int64_t n_tokens, int32_t n_experts, int32_t k,
                   int32_t renormalize, int32_t* topk_idx, float* topk_w, void* stream);

/* ---------------------------------------------------------------- mode
 * moe_resolve_sorted -- the runtime sort switch, host only.
 *
 * [ET-PR] (reviews): cond = (M - 1) // sort_cutoff, M <= cutoff -> unsorted
 * (decode), M > cutoff -> sorted (prefill).  sort = MOE_SORT_ON / OFF forces
 * the mode; MOE_SORT_AUTO applies the switch with M = n_tokens.  A cutoff
 * <= 0 always sorts (the switch's divide-by-zero guard).
 *   sorted_out [host] int32: 1 sorted, 0 unsorted.
 * Errors: MOE_ERR_ARG for a sort value outside {-1, 0, 1}, null sorted_out or
 * n_tokens < 0. */
int moe_resolve_sorted(int32_t sort, int64_t n_tokens, int32_t sort_cutoff, int32_t* sorted_out);

/* ---------------------------------------------------------------- dispatch
 * moe_dispatch_workspace_bytes -- device workspace moe_dispatch needs for
 * these sizes (the same value in both sort modes).  0 for invalid sizes. */
size_t moe_dispatch_workspace_bytes(int64_t n_tokens, int32_t n_experts, int32_t k,
                                    int32_t n_segments);

/* moe_dispatch -- count, scan, stable position assignment and row copy.
 *
 * Mode: sorted = moe_resolve_sorted(sort, n_tokens, sort_cutoff).  Bucket of
 * pair q: its expert (sorted) or its segment (unsorted; with G == 1 every
 * pair is in one bucket, the identity layout of [ET-PR]'s unsorted branch).
 * Row position of pair q:
 *   dst_pos[q] = start of its bucket + #{q' < q with the same bucket},
 * i.e. a stable sort of the flattened [N*k] keys ([ET-PR] follow-up).
 *
 * Outputs (all written in both modes, same shapes -- [ET-PR] reviews):
 *   expert_counts   [E]    int32  pairs routed to each expert
 *   expert_offsets  [E+1]  int32  exclusive prefix sum; [E] = NK.  These are
 *                                 row ranges of experts only when sorted.
 *   segment_offsets [G+1]  int32  start of each segment's block =
 *                                 expert_offsets[g*E/G]; valid in both modes.
 *   dst_pos         [NK]   int32  row of pair q (the inv_order map)
 *   src_pair        [NK]   int32  pair q = t*k + j held by row p (argsort order)
 *   row_expert      [NK]   int32  expert of row p; may be NULL
 *   rows            [NK, D]       rows[p] = x[src_pair[p] / k], bytes copied
 *                                 unchanged (dispatch_local / packet_scatter of
 *                                 [MLX-EP]); NULL together with x to compute
 *                                 the maps only
 *   row_scales      [NK, D/128] float32, rows' block scales (F8 only)
 * Inputs:
 *   x               [N, D] of `dtype` (NULL: maps only)
 *   x_scales        [N, D/128] float32 for MOE_F8E4M3, else NULL
 *   topk_idx        [N, k] int32 expert ids in [0, E)
 *   sorted_used     [host] int32, may be NULL: receives the resolved mode
 *   workspace       device memory of at least
 *                   moe_dispatch_workspace_bytes(N, E, k, G) bytes, 16-byte
 *                   aligned; contents need not be initialised and are
 *                   clobbered.
 * Errors: MOE_ERR_ARG for null required pointers, N < 0, D < 1, E < 1,
 * k < 1, k > E, G < 1, E % G != 0, D % 128 != 0 for F8, x_scales/row_scales
 * not given exactly for F8, an unknown dtype or sort value, or x/rows given
 * one without the other; MOE_ERR_UNSUPPORTED for E > MOE_MAX_EXPERTS,
 * k > MOE_MAX_TOPK or NK > INT32_MAX; MOE_ERR_WORKSPACE for a short or
 * misaligned workspace.  N == 0 writes zero counts and offsets.
 * Launches: with a payload whose row size and addresses (and those of the
 * scales) are multiples of 16 bytes, outside the identity layout, above 4096
 * pairs and with the rank's LDS within 16 KB (E <= 584 sorted), positions and
 * row copy share one launch.  dst_pos then serves
 * as the flag array between them (set to INT32_MIN first, then to each
 * position, with device-scope atomics).  A copy wave waits for its token's
 * positions for at most about 2^18 polls (milliseconds); should it ever give
 * up, it skips those rows, and validate mode reports it.  (Test hook: the
 * environment variable MOE_DC_SPIN_LIMIT=<n> sets that limit, so tests can
 * force the give-up path.) */
int moe_dispatch(const void* x, const float* x_scales, int32_t dtype,
                 int64_t n_tokens, int64_t hidden,
                 const int32_t* topk_idx, int32_t n_experts, int32_t k, int32_t n_segments,
                 int32_t sort, int32_t sort_cutoff, int32_t* sorted_used,
                 void* rows, float* row_scales,
                 int32_t* expert_counts, int32_t* expert_offsets, int32_t* segment_offsets,
                 int32_t* src_pair, int32_t* dst_pos, int32_t* row_expert,
                 void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- route + dispatch
 * moe_route_dispatch_workspace_bytes -- workspace of moe_route_dispatch
 * (at least moe_dispatch_workspace_bytes for the same sizes).  0 for invalid
 * sizes. */
size_t moe_route_dispatch_workspace_bytes(int64_t n_tokens, int32_t n_experts, int32_t k,
                                          int32_t n_segments);

/* moe_route_dispatch -- moe_route_topk followed by moe_dispatch in one call,
 * with the same outputs as the two calls made in sequence (bit for bit).
 *   logits [N, E] f32, renormalize, topk_idx [N, k] i32 (output, then read
 *   by the dispatch), topk_w [N, k] f32 (output); every other argument as in
 *   moe_dispatch; workspace of moe_route_dispatch_workspace_bytes(N, E, k, G).
 * In the identity layout (unsorted, G == 1) row t*k+j is x[t] whatever the
 * routing chooses, so the routing and the row copy run in one launch; other
 * layouts take moe_dispatch's launches after the routing launch (with its
 * shared positions + row copy launch, bounded wait and validate-mode report).
 * Errors: those of moe_route_topk and moe_dispatch. */
int moe_route_dispatch(const float* logits, int32_t renormalize, int32_t* topk_idx, float* topk_w,
                       const void* x, const float* x_scales, int32_t dtype, int64_t n_tokens,
                       int64_t hidden, int32_t n_experts, int32_t k, int32_t n_segments,
                       int32_t sort, int32_t sort_cutoff, int32_t* sorted_used, void* rows,
                       float* row_scales, int32_t* expert_counts, int32_t* expert_offsets,
                       int32_t* segment_offsets, int32_t* src_pair, int32_t* dst_pos,
                       int32_t* row_expert, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Bytes of the static per-GPU scratch array of moe_route_dispatch_noalloc. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)1048576 + 256)

/* moe_route_dispatch_noalloc -- moe_route_dispatch for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments and outputs (bit for bit)
 * without the workspace: its scratch is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until the
 * process ends; the array's device address is looked up on the first call on
 * a device (the device of `stream`, or the current one for the null stream)
 * and kept.  The call allocates nothing (no hipMalloc, no allocating library
 * routine) and needs no zeroed memory: every scratch byte it reads was
 * written earlier in the same call.  All calls on one GPU share the array, so
 * calls that overlap on one GPU (other streams, other host threads) race:
 * serialise them.  Validate mode does not apply (it would copy to the host
 * and wait).
 * Errors: those of moe_route_dispatch; MOE_ERR_UNSUPPORTED when
 * moe_route_dispatch_workspace_bytes(N, E, k, G) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES (E <= 256 always fits; E = 1024 fits up to
 * N*k = 262144 pairs), checked before any device call; MOE_ERR_HIP if the
 * scratch address cannot be obtained. */
int moe_route_dispatch_noalloc(const float* logits, int32_t renormalize, int32_t* topk_idx,
                               float* topk_w, const void* x, const float* x_scales, int32_t dtype,
                               int64_t n_tokens, int64_t hidden, int32_t n_experts, int32_t k,
                               int32_t n_segments, int32_t sort, int32_t sort_cutoff,
                               int32_t* sorted_used, void* rows, float* row_scales,
                               int32_t* expert_counts, int32_t* expert_offsets,
                               int32_t* segment_offsets, int32_t* src_pair, int32_t* dst_pos,
                               int32_t* row_expert, void* stream);

/* moe_scatter_rows -- the row copy of moe_dispatch on its own, scatter form
 * (packet_scatter / dispatch_local of [MLX-EP]):
 *   rows[dst_pos[t*k + j]] = x[t]   for every token t and slot j,
 * moving `row_bytes` bytes per row unchanged (any payload format: bf16, fp32,
 * fp8 codes, or fp8 block scales as a second call).  Each token row is read
 * once and written k times.
 *   x [N, row_bytes], dst_pos [N*k] int32 (from moe_dispatch),
 *   rows [N*k, row_bytes], output; entries of dst_pos outside [0, N*k) are
 *   skipped.
 * Errors: MOE_ERR_ARG for null pointers (unless N == 0), N < 0,
 * row_bytes < 1, k < 1; MOE_ERR_UNSUPPORTED for k > MOE_MAX_TOPK or
 * N*k > INT32_MAX. */
int moe_scatter_rows(const void* x, int64_t n_tokens, int64_t row_bytes, int32_t k,
                     const int32_t* dst_pos, void* rows, void* stream);

/* moe_gather_rows -- gather form of the same copy (packet_gather of
 * [MLX-EP]; the Take of [ET-PR]'s sorted branch with token = order // top_k):
 *   rows[p] = x[src_pair[p] / k]   for p in [0, n_rows).
 *   x [N, row_bytes], src_pair [n_rows] int32, rows [n_rows, row_bytes];
 *   rows whose src_pair is negative or names a token >= N are left untouched.
 * Errors: MOE_ERR_ARG for null pointers (unless n_rows == 0), negative
 * sizes, row_bytes < 1, k < 1; MOE_ERR_UNSUPPORTED beyond the int32 range. */
int moe_gather_rows(const void* x, int64_t n_tokens, int64_t row_bytes, int32_t k,
                    const int32_t* src_pair, int64_t n_rows, void* rows, void* stream);

/* ---------------------------------------------------------------- combine
 * moe_combine -- weighted top-k gather-sum back to token order
 * (combine_weighted_sum of [MLX-EP]; the unscatter through inv_order of
 * [ET-PR] is folded in as dst_pos):
 *   out[t, i] = sum_{j<k} w[t, j] * y[dst_pos[t*k + j], i]
 * evaluated as one fp32 FMA chain in slot order j = 0..k-1 (acc = 0;
 * acc = fma(w_j, y_j, acc)), then rounded to nearest-even into out_dtype.
 * The order is fixed, so the result does not depend on the dispatch layout.
 *
 *   y        [NK, D] of y_dtype (MOE_F32 or MOE_BF16): expert outputs in
 *            dispatched row order (identity experts: y = rows)
 *   dst_pos  [NK] int32 from moe_dispatch; entries outside [0, NK) add 0
 *   topk_w   [N, k] float32
 *   out      [N, D] of out_dtype (MOE_F32 or MOE_BF16)
 * Errors: MOE_ERR_ARG for null pointers (unless N == 0), N < 0, D < 1,
 * k < 1, dtypes outside {MOE_F32, MOE_BF16}; MOE_ERR_UNSUPPORTED for
 * k > MOE_MAX_TOPK or NK > INT32_MAX. */
int moe_combine(const void* y, int32_t y_dtype, int64_t n_tokens, int64_t hidden, int32_t k,
                const int32_t* dst_pos, const float* topk_w,
                void* out, int32_t out_dtype, void* stream);

/* ---------------------------------------------------------------- experts
 * moe_dequant_rows -- identity expert for an F8 payload: turns dispatched
 * E4M3FN rows and their block scales into bfloat16 rows,
 *   y[p, i] = round_to_nearest_even_bf16( value(rows[p, i]) * row_scales[p, i/128] )
 * with the product taken exactly before the single rounding.
 *   rows [n_rows, D] uint8, row_scales [n_rows, D/128] float32,
 *   y [n_rows, D] bfloat16 (uint16 bit patterns).
 * Errors: MOE_ERR_ARG for null pointers (unless n_rows == 0), n_rows < 0,
 * D < 1 or D % 128 != 0. */
int moe_dequant_rows(const uint8_t* rows, const float* row_scales, int64_t n_rows,
                     int64_t hidden, uint16_t* y, void* stream);

/* moe_grouped_swiglu_workspace_bytes -- workspace of moe_grouped_swiglu. */
size_t moe_grouped_swiglu_workspace_bytes(int64_t n_rows, int32_t n_experts, int64_t hidden,
                                          int64_t ffn);

/* moe_grouped_swiglu -- grouped expert FFN reading the dispatched rows in
 * place ([1SIDED]: grouped GEMMs read the buffers in place instead of from a
 * per-expert copy; [ET-PR]: the sorted flag is the caller's promise that rows
 * are grouped by expert; expert weights laid out [E, out, in]).  For expert e
 * and every row p in [expert_offsets[e], expert_offsets[e+1]):
 *   h = bf16( silu(W_gate[e] r_p) * (W_up[e] r_p) ),  silu(a) = a / (1 + e^-a)
 *   y[p] = bf16( W_down[e] h )
 * bf16 inputs, fp32 accumulation on the matrix cores, h stored as bf16 in the
 * workspace between the two products.  Tiles of a last, partial round of
 * workgroups are split along K; their fp32 partials (in the workspace) are
 * summed in a fixed order, so the output is the same on every call.
 *
 *   rows            [n_rows, D] bfloat16, grouped by expert (sorted dispatch)
 *   expert_offsets  [E+1] int32, device-resident (never read by the host);
 *                   offsets[0] == 0, non-decreasing, offsets[E] == n_rows
 *   w_gate, w_up    [E, F, D] bfloat16;  w_down [E, D, F] bfloat16
 *   y               [n_rows, D] bfloat16, output, same row order as rows
 * Errors: MOE_ERR_ARG for null pointers (unless n_rows == 0), sizes < 1;
 * MOE_ERR_UNSUPPORTED for D % 64 != 0, F % 64 != 0, D or F above 2^22,
 * E > MOE_MAX_EXPERTS, more than 2^31 tiles of 256 x 256, or rows, a weight
 * tensor or y not 16-byte aligned;
 * MOE_ERR_WORKSPACE for a short workspace or one not 256-byte aligned. */
int moe_grouped_swiglu(const void* rows, int64_t n_rows, int64_t hidden,
                       const int32_t* expert_offsets, int32_t n_experts,
                       const void* w_gate, const void* w_up, const void* w_down, int64_t ffn,
                       void* y, void* workspace, size_t workspace_bytes, void* stream);

/* moe_gather_swiglu_workspace_bytes -- workspace of moe_gather_swiglu. */
size_t moe_gather_swiglu_workspace_bytes(int64_t n_rows, int32_t n_experts, int64_t hidden,
                                         int64_t ffn);

/* moe_gather_swiglu -- the expert FFN of moe_grouped_swiglu over rows left in
 * any order, each row naming its own expert ([ET-PR]: decode keeps the rows in
 * token order, with no argsort, and the expert product takes a per-row expert
 * id, gather_mm with unsorted right-hand indices).  For every row r with
 * e = row_expert[r] in [0, E):
 *   h = bf16( silu(W_gate[e] rows[r]) * (W_up[e] rows[r]) )
 *   y[r] = bf16( W_down[e] h )
 * Rows whose id lies outside [0, E) are skipped: their y rows are left as they
 * were.  The rows are not moved: a stable counting sort of the ids lists each
 * expert's rows, every active expert's weights are read once for all of them,
 * and y[r] lands at row r.  Meant for few rows per expert (decode); grouped
 * rows at prefill sizes are the case of moe_grouped_swiglu.
 *
 *   rows            [n_rows, D] bfloat16, any order (e.g. the unsorted dispatch)
 *   row_expert      [n_rows] int32, device-resident
 *   w_gate, w_up    [E, F, D] bfloat16;  w_down [E, D, F] bfloat16
 *   y               [n_rows, D] bfloat16, output, same row order as rows
 *   workspace       moe_gather_swiglu_workspace_bytes(n_rows, E, D, F) bytes
 * Errors: MOE_ERR_ARG for null pointers (unless n_rows == 0), n_rows < 0,
 * sizes < 1; MOE_ERR_UNSUPPORTED for D % 128 != 0, F % 128 != 0,
 * E > MOE_MAX_EXPERTS, n_rows beyond the int32 range, rows or a weight tensor
 * not 16-byte aligned, y not 2-byte aligned;
 * MOE_ERR_WORKSPACE for a short workspace or one not 256-byte aligned. */
int moe_gather_swiglu(const void* rows, int64_t n_rows, int64_t hidden,
                      const int32_t* row_expert, int32_t n_experts,
                      const void* w_gate, const void* w_up, const void* w_down, int64_t ffn,
                      void* y, void* workspace, size_t workspace_bytes, void* stream);

/* moe_gather_swiglu_combine -- EXPERIMENTAL: moe_gather_swiglu with the
 * weighted top-k sum fused into its down product (the zero-copy combine
 * planned in [MLX-EP]): y is never written.  On MI355X it is slower than the
 * unfused moe_gather_swiglu + moe_combine pair (the decode layer with
 * DeepSeek-sized experts: 3.74-3.87 against 3.65-3.77 ms; the atomics cost
 * more than the y round trip they save) and its output is not bit-stable
 * between calls; prefer the unfused pair unless the layer is to be added
 * straight into an fp32 residual.  For every row r whose expert e = row_expert[r] lies in
 * [0, E) and whose pair q (row_pair[r], or r itself when row_pair is null)
 * lies in [0, n_tokens * k):
 *   out[q / k] += topk_w[q] * (W_down[e] h),  h as in moe_gather_swiglu,
 * with the product's fp32 value (y is not rounded to bf16) added by fp32
 * atomics.  out accumulates: pass zeros for the plain combine, or the residual
 * stream to add the layer into it.  The order of the k additions into one
 * element is not fixed, so results can differ between calls in the last bits
 * of fp32 (the unfused moe_gather_swiglu + moe_combine pair is bit-stable).
 *
 *   rows            [n_rows, D] bfloat16, any order (e.g. the unsorted dispatch)
 *   row_expert      [n_rows] int32;  row_pair [n_rows] int32 or null (the
 *                   dispatch's src_pair: the pair q = t*k + j each row holds)
 *   topk_w          [n_tokens, k] float32 (the routing weights)
 *   out             [n_tokens, D] float32, read and written
 *   w_gate, w_up    [E, F, D] bfloat16;  w_down [E, D, F] bfloat16
 *   workspace       moe_gather_swiglu_workspace_bytes(n_rows, E, D, F) bytes
 * Errors: those of moe_gather_swiglu, with k outside [1, 64] or n_tokens < 0
 * as MOE_ERR_ARG, n_tokens * k beyond the int32 range or out / topk_w not
 * 4-byte aligned as MOE_ERR_UNSUPPORTED. */
int moe_gather_swiglu_combine(const void* rows, int64_t n_rows, int64_t hidden,
                              const int32_t* row_expert, const int32_t* row_pair,
                              const float* topk_w, int64_t n_tokens, int32_t k, int32_t n_experts,
                              const void* w_gate, const void* w_up, const void* w_down,
                              int64_t ffn, float* out, void* workspace, size_t workspace_bytes,
                              void* stream);

/* moe_grouped_gemm_fp8 -- fp8 block-scaled grouped expert GEMM reading the
 * dispatched fp8 rows in place ([1SIDED]: the dispatch is agnostic to the
 * activation quantisation format, and grouped GEMMs read the received buffers
 * in place).  Rows are the fp8 dispatch's output: E4M3FN codes with one
 * float32 scale per 128 elements of a row, grouped by expert.  For expert e and
 * every row p in [expert_offsets[e], expert_offsets[e+1]):
 *   y[p, n] = bf16( sum_b row_scales[p, b] * w_scales[e, n/128, b]
 *                   * sum_{k in block b} q(rows[p, k]) * q(w[e, n, k]) )
 * with b over the K/128 blocks of 128 and q() the E4M3FN value.  fp8 products
 * on the matrix cores, fp32 per-block partial sums scaled and accumulated in
 * fp32, one rounding to bf16.
 *
 *   rows            [n_rows, K] E4M3FN codes (uint8), 16-byte aligned
 *   row_scales      [n_rows, K/128] float32
 *   expert_offsets  [E+1] int32, device-resident; rows outside
 *                   [offsets[0], offsets[E]) are neither read nor written
 *   w               [E, N, K] E4M3FN codes, 16-byte aligned
 *   w_scales        [E, N/128, K/128] float32
 *   y               [n_rows, N] bfloat16, output, same row order as rows,
 *                   16-byte aligned
 * No workspace.  Errors: MOE_ERR_ARG for null pointers (unless n_rows == 0),
 * sizes < 1, misaligned scales; MOE_ERR_UNSUPPORTED for K % 128 != 0,
 * N % 128 != 0, E > MOE_MAX_EXPERTS or misaligned rows / w / y. */
int moe_grouped_gemm_fp8(const void* rows, const float* row_scales, int64_t n_rows,
                         int64_t k_dim, const int32_t* expert_offsets, int32_t n_experts,
                         const void* w, const float* w_scales, int64_t n_dim, void* y,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DC_H */
