// Host-side launchers of the MoE kernels.  Argument checking happens in
// api.cpp before any of these is called; the launchers only shape grids.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_dc.h"

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 64;

hipError_t launch_route_topk(const float* logits, int64_t n_tokens, int n_experts, int k,
                             int renormalize, int32_t* topk_idx, float* topk_w,
                             hipStream_t stream);

// ---- dispatch
struct DispatchPlan {
  int64_t nk;          // routed pairs
  int chunk;           // pairs per counting chunk (multiple of 256)
  int n_chunks;        // P
  int small;           // 1: one workgroup computes counts, scan and positions
};

DispatchPlan plan_dispatch(int64_t n_tokens, int n_experts, int k, int n_segments);
size_t dispatch_workspace_bytes(int64_t n_tokens, int n_experts, int k, int n_segments);

struct DispatchArgs {
  const void* x;
  const float* x_scales;
  int64_t row_bytes;        // D * element size
  int64_t scale_bytes;      // D/128 * 4 for F8, else 0
  int64_t n_tokens;
  const int32_t* topk_idx;
  int n_experts, k, n_segments, sorted;
  void* rows;
  float* row_scales;
  int32_t* expert_counts;
  int32_t* expert_offsets;
  int32_t* segment_offsets;
  int32_t* src_pair;
  int32_t* dst_pos;
  int32_t* row_expert;
  void* workspace;
  int32_t* status;          // device word set to 1 on an out-of-range id, or null
  int maps_done;            // identity layout: the maps are already written
  int spin_limit = -1;      // polls before a copy wave of the shared rank + copy launch
                            // gives up (< 0: the default)
};

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream);

// Routing followed by dispatch on the same stream.
struct RouteArgs {
  const float* logits;
  int renormalize;
  float* topk_w;
};
// Routing and, side by side in the same launch, the identity-layout row copy
// (unsorted, one segment): rows [N*k, row_bytes] with row t*k+j = x[t], and
// the identity maps (dst_pos = src_pair = q, row_expert = the routed expert,
// row_expert may be null).  Requires 16-byte aligned x, rows and row_bytes;
// n_tokens > 0.
hipError_t launch_route_copy_identity(const float* logits, int64_t n_tokens, int n_experts, int k,
                                      int renormalize, int32_t* topk_idx, float* topk_w,
                                      const void* x, int64_t row_bytes, void* rows,
                                      int32_t* dst_pos, int32_t* src_pair, int32_t* row_expert,
                                      hipStream_t stream);
size_t route_dispatch_workspace_bytes(int64_t n_tokens, int n_experts, int k, int n_segments);
hipError_t launch_route_dispatch(const RouteArgs& r, const DispatchArgs& a, hipStream_t stream);

// Allocation-free variant: the device address of a static per-GPU scratch
// array of kNoAllocScratchBytes (256-byte aligned) on the stream's device,
// looked up on the first call on that device and kept.
constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);

// Row copies on their own (byte payloads): scatter form rows[dst_pos[q]] =
// x[q / k] and gather form rows[p] = x[src_pair[p] / k].
hipError_t launch_scatter_rows(const void* x, int64_t n_tokens, int64_t row_bytes, int k,
                               const int32_t* dst_pos, void* rows, hipStream_t stream);
hipError_t launch_gather_rows(const void* x, int64_t n_tokens, int64_t row_bytes, int k,
                              const int32_t* src_pair, int64_t n_rows, void* rows,
                              hipStream_t stream);

// ---- combine
hipError_t launch_combine(const void* y, int y_bf16, int64_t n_tokens, int64_t hidden, int k,
                          const int32_t* dst_pos, const float* topk_w, void* out, int out_bf16,
                          hipStream_t stream);

// ---- experts
hipError_t launch_dequant_rows(const uint8_t* rows, const float* row_scales, int64_t n_rows,
                               int64_t hidden, uint16_t* y, hipStream_t stream);

size_t grouped_swiglu_workspace_bytes(int64_t n_rows, int n_experts, int64_t hidden, int64_t ffn);
// Worst-case workgroup count of the larger of the two grouped SwiGLU launches.
int64_t grouped_swiglu_tiles(int64_t n_rows, int n_experts, int64_t hidden, int64_t ffn);
hipError_t launch_grouped_swiglu(const void* rows, int64_t n_rows, int64_t hidden,
                                 const int32_t* expert_offsets, int n_experts, const void* w_gate,
                                 const void* w_up, const void* w_down, int64_t ffn, void* y,
                                 void* workspace, hipStream_t stream);

// SwiGLU experts over rows in any order, row r taking expert row_expert[r]
// (hidden and ffn multiples of 128).  tiles: workgroup count of the larger
// of the two products, for the caller's int32 range check.
//
// With `fused`, y is not written: the down product adds topk_w[q] * y(r)
// straight into out[q / k] (fp32, [N, D]), q = row_pair[r] (q = r if row_pair
// is null); rows whose q lies outside [0, n_pairs) add nothing.
struct FusedCombine {
  const int32_t* row_pair;
  const float* topk_w;
  float* out;
  int k;
  int n_pairs;
};
size_t gather_swiglu_workspace_bytes(int64_t n_rows, int n_experts, int64_t hidden, int64_t ffn);
int64_t gather_swiglu_tiles(int64_t n_rows, int n_experts, int64_t hidden, int64_t ffn);
hipError_t launch_gather_swiglu(const void* rows, int64_t n_rows, int64_t hidden,
                                const int32_t* row_expert, int n_experts, const void* w_gate,
                                const void* w_up, const void* w_down, int64_t ffn, void* y,
                                void* workspace, hipStream_t stream,
                                const FusedCombine* fused = nullptr);

// fp8 block-scaled grouped GEMM (K and N multiples of 128).
hipError_t launch_grouped_gemm_fp8(const void* rows, const float* row_scales, int64_t n_rows,
                                   int64_t k_dim, const int32_t* expert_offsets, int n_experts,
                                   const void* w, const float* w_scales, int64_t n_dim, void* y,
                                   hipStream_t stream);

}  // namespace moe
