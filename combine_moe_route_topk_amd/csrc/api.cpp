// C ABI of libmoe_dc: argument checking, mode resolution, workspace sizing and
// error reporting.  Every check runs on the host before any HIP call, so a
// rejected call touches no device state.
#include "../../include/moe_dc.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return MOE_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool validate_mode() {
  const char* v = std::getenv("MOE_DC_VALIDATE");
  return v && v[0] == '1';
}

// Test hook: MOE_DC_SPIN_LIMIT=<n> caps the polls of a copy wave that waits for
// positions of its own launch (so tests can force the give-up path); unset or
// malformed: the library default.
int spin_limit() {
  const char* v = std::getenv("MOE_DC_SPIN_LIMIT");
  if (!v || !*v) return -1;
  char* end = nullptr;
  const long n = std::strtol(v, &end, 10);
  return (end && *end == '\0' && n >= 0 && n < (1L << 30)) ? int(n) : -1;
}

int check_routing_sizes(const char* fn, int64_t n_tokens, int32_t n_experts, int32_t k) {
  if (n_tokens < 0) return fail(MOE_ERR_ARG, "%s: n_tokens < 0", fn);
  if (n_experts < 1) return fail(MOE_ERR_ARG, "%s: n_experts < 1", fn);
  if (k < 1 || k > n_experts) return fail(MOE_ERR_ARG, "%s: need 1 <= k <= n_experts (k=%d, E=%d)", fn, k, n_experts);
  if (n_experts > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "%s: n_experts > %d", fn, MOE_MAX_EXPERTS);
  if (k > MOE_MAX_TOPK) return fail(MOE_ERR_UNSUPPORTED, "%s: k > %d", fn, MOE_MAX_TOPK);
  if (n_tokens > 0 && n_tokens * int64_t(k) > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "%s: n_tokens * k exceeds the int32 index range", fn);
  return MOE_OK;
}

int resolve_sorted(int32_t sort, int64_t n_tokens, int32_t cutoff, int32_t* out) {
  if (sort == MOE_SORT_ON) { *out = 1; return MOE_OK; }
  if (sort == MOE_SORT_OFF) { *out = 0; return MOE_OK; }
  if (sort != MOE_SORT_AUTO) return fail(MOE_ERR_ARG, "sort must be -1, 0 or 1 (got %d)", sort);
  if (cutoff <= 0) { *out = 1; return MOE_OK; }
  // (M - 1) // cutoff >= 1  <=>  M > cutoff, for M >= 1
  *out = n_tokens > cutoff ? 1 : 0;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_DC_ABI_VERSION; }

const char* moe_last_error(void) { return g_last_error.c_str(); }

int moe_resolve_sorted(int32_t sort, int64_t n_tokens, int32_t sort_cutoff, int32_t* sorted_out) {
  if (!sorted_out) return fail(MOE_ERR_ARG, "moe_resolve_sorted: sorted_out is null");
  if (n_tokens < 0) return fail(MOE_ERR_ARG, "moe_resolve_sorted: n_tokens < 0");
  const int rc = resolve_sorted(sort, n_tokens, sort_cutoff, sorted_out);
  return rc == MOE_OK ? ok() : rc;
}

int moe_route_topk(const float* logits, int64_t n_tokens, int32_t n_experts, int32_t k,
                   int32_t renormalize, int32_t* topk_idx, float* topk_w, void* stream) {
  const char* fn = "moe_route_topk";
  int rc = check_routing_sizes(fn, n_tokens, n_experts, k);
  if (rc) return rc;
  if (n_tokens == 0) return ok();
  if (!logits || !topk_idx || !topk_w) return fail(MOE_ERR_ARG, "%s: null pointer argument", fn);
  return hip_status(moe::launch_route_topk(logits, n_tokens, n_experts, k, renormalize ? 1 : 0,
                                           topk_idx, topk_w, static_cast<hipStream_t>(stream)),
                    fn);
}

size_t moe_dispatch_workspace_bytes(int64_t n_tokens, int32_t n_experts, int32_t k,
                                    int32_t n_segments) {
  if (n_tokens < 0 || n_experts < 1 || n_experts > MOE_MAX_EXPERTS || k < 1 || k > n_experts ||
      k > MOE_MAX_TOPK || n_segments < 1 || n_experts % n_segments != 0 ||
      n_tokens * int64_t(k) > INT32_MAX)
    return 0;
  return moe::dispatch_workspace_bytes(n_tokens, n_experts, k, n_segments);
}

}  // extern "C"

namespace {

// Shared argument checking and packing of moe_dispatch / moe_route_dispatch.
// Returns MOE_OK and fills `a` (and `sorted`) or returns the error status.
int prepare_dispatch(const char* fn, const void* x, const float* x_scales, int32_t dtype,
                     int64_t n_tokens, int64_t hidden, const int32_t* topk_idx, int32_t n_experts,
                     int32_t k, int32_t n_segments, int32_t sort, int32_t sort_cutoff, void* rows,
                     float* row_scales, int32_t* expert_counts, int32_t* expert_offsets,
                     int32_t* segment_offsets, int32_t* src_pair, int32_t* dst_pos,
                     int32_t* row_expert, void* workspace, size_t workspace_bytes, size_t need,
                     moe::DispatchArgs& a) {
  int rc = check_routing_sizes(fn, n_tokens, n_experts, k);
  if (rc) return rc;
  if (hidden < 1) return fail(MOE_ERR_ARG, "%s: hidden < 1", fn);
  if (n_segments < 1 || n_experts % n_segments != 0)
    return fail(MOE_ERR_ARG, "%s: n_segments must divide n_experts (E=%d, G=%d)", fn, n_experts, n_segments);
  int64_t elem = 0;
  switch (dtype) {
    case MOE_F32: elem = 4; break;
    case MOE_BF16: elem = 2; break;
    case MOE_F8E4M3: elem = 1; break;
    default: return fail(MOE_ERR_ARG, "%s: unknown dtype %d", fn, dtype);
  }
  if ((x == nullptr) != (rows == nullptr))
    return fail(MOE_ERR_ARG, "%s: x and rows must both be given or both be null", fn);
  if (dtype == MOE_F8E4M3) {
    if (hidden % 128 != 0) return fail(MOE_ERR_ARG, "%s: F8 payload needs hidden %% 128 == 0", fn);
    if (x && (!x_scales || !row_scales))
      return fail(MOE_ERR_ARG, "%s: F8 payload needs x_scales and row_scales", fn);
  } else if (x_scales || row_scales) {
    return fail(MOE_ERR_ARG, "%s: block scales are only for the F8 payload", fn);
  }
  if (!x && (x_scales || row_scales))
    return fail(MOE_ERR_ARG, "%s: scales given without a payload", fn);
  if (!expert_counts || !expert_offsets || !segment_offsets)
    return fail(MOE_ERR_ARG, "%s: null offsets/counts output", fn);
  if (n_tokens > 0 && (!topk_idx || !src_pair || !dst_pos))
    return fail(MOE_ERR_ARG, "%s: null index input or map output", fn);
  int32_t sorted = 0;
  rc = resolve_sorted(sort, n_tokens, sort_cutoff, &sorted);
  if (rc) return rc;
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : size_t(0));
  if (reinterpret_cast<uintptr_t>(workspace) & 15)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace must be 16-byte aligned", fn);
  a = moe::DispatchArgs{};
  a.x = x;
  a.x_scales = x_scales;
  a.row_bytes = hidden * elem;
  a.scale_bytes = dtype == MOE_F8E4M3 ? hidden / 128 * 4 : 0;
  a.n_tokens = n_tokens;
  a.topk_idx = topk_idx;
  a.n_experts = n_experts;
  a.k = k;
  a.n_segments = n_segments;
  a.sorted = sorted;
  a.rows = rows;
  a.row_scales = row_scales;
  a.expert_counts = expert_counts;
  a.expert_offsets = expert_offsets;
  a.segment_offsets = segment_offsets;
  a.src_pair = src_pair;
  a.dst_pos = dst_pos;
  a.row_expert = row_expert;
  a.workspace = workspace;
  a.spin_limit = spin_limit();
  return MOE_OK;
}

// Validate mode: clear the status word before the launches, then wait and
// report out-of-range expert ids.
int32_t* validate_begin(void* workspace, size_t need, hipStream_t s, int* rc, const char* fn) {
  int32_t* status = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + need - 16);
  hipError_t e = hipMemsetAsync(status, 0, sizeof(int32_t), s);
  *rc = e == hipSuccess ? MOE_OK : hip_status(e, fn);
  return status;
}

int validate_end(int32_t* status, hipStream_t s, int32_t n_experts, const char* fn) {
  int32_t host_status = 0;
  hipError_t e = hipMemcpyAsync(&host_status, status, sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, fn);
  if (host_status & 1) return fail(MOE_ERR_ARG, "%s: topk_idx holds expert ids outside [0, %d)", fn, n_experts);
  if (host_status & 2)
    return fail(MOE_ERR_HIP, "%s: the row copy gave up waiting for positions of its own launch", fn);
  return ok();
}

}  // namespace

extern "C" {

int moe_dispatch(const void* x, const float* x_scales, int32_t dtype, int64_t n_tokens,
                 int64_t hidden, const int32_t* topk_idx, int32_t n_experts, int32_t k,
                 int32_t n_segments, int32_t sort, int32_t sort_cutoff, int32_t* sorted_used,
                 void* rows, float* row_scales, int32_t* expert_counts, int32_t* expert_offsets,
                 int32_t* segment_offsets, int32_t* src_pair, int32_t* dst_pos,
                 int32_t* row_expert, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "moe_dispatch";
  const int early = check_routing_sizes(fn, n_tokens, n_experts, k);
  if (early) return early;
  const size_t need = moe::dispatch_workspace_bytes(n_tokens, n_experts, k, n_segments > 0 ? n_segments : 1);
  moe::DispatchArgs a;
  int rc = prepare_dispatch(fn, x, x_scales, dtype, n_tokens, hidden, topk_idx, n_experts, k,
                            n_segments, sort, sort_cutoff, rows, row_scales, expert_counts,
                            expert_offsets, segment_offsets, src_pair, dst_pos, row_expert,
                            workspace, workspace_bytes, need, a);
  if (rc) return rc;
  if (sorted_used) *sorted_used = a.sorted;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool validate = validate_mode();
  if (validate) {
    a.status = validate_begin(workspace, need, s, &rc, fn);
    if (rc) return rc;
  }
  rc = hip_status(moe::launch_dispatch(a, s), fn);
  if (rc || !validate) return rc;
  return validate_end(a.status, s, n_experts, fn);
}

size_t moe_route_dispatch_workspace_bytes(int64_t n_tokens, int32_t n_experts, int32_t k,
                                          int32_t n_segments) {
  if (moe_dispatch_workspace_bytes(n_tokens, n_experts, k, n_segments) == 0) return 0;
  return moe::route_dispatch_workspace_bytes(n_tokens, n_experts, k, n_segments);
}

}  // extern "C"

namespace {

// moe_route_dispatch and its allocation-free variant: the same checks and
// launches; `workspace` is the caller's buffer or the static scratch.
int route_dispatch_impl(const char* fn, const float* logits, int32_t renormalize,
                        int32_t* topk_idx, float* topk_w, const void* x, const float* x_scales,
                        int32_t dtype, int64_t n_tokens, int64_t hidden, int32_t n_experts,
                        int32_t k, int32_t n_segments, int32_t sort, int32_t sort_cutoff,
                        int32_t* sorted_used, void* rows, float* row_scales,
                        int32_t* expert_counts, int32_t* expert_offsets,
                        int32_t* segment_offsets, int32_t* src_pair, int32_t* dst_pos,
                        int32_t* row_expert, void* workspace, size_t workspace_bytes,
                        void* stream, bool static_scratch) {
  const int early = check_routing_sizes(fn, n_tokens, n_experts, k);
  if (early) return early;
  if (n_tokens > 0 && (!logits || !topk_idx || !topk_w))
    return fail(MOE_ERR_ARG, "%s: null routing pointer", fn);
  const size_t need = moe::route_dispatch_workspace_bytes(n_tokens, n_experts, k, n_segments > 0 ? n_segments : 1);
  if (static_scratch && need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_UNSUPPORTED,
                "%s: these sizes need %zu bytes of scratch, more than the %zu-byte static array "
                "(use moe_route_dispatch with a workspace)",
                fn, need, size_t(MOE_NOALLOC_SCRATCH_BYTES));
  // every argument is checked before the scratch is looked up, so a rejected
  // call touches no device state (a placeholder address stands in for it)
  moe::DispatchArgs a;
  int rc = prepare_dispatch(fn, x, x_scales, dtype, n_tokens, hidden, topk_idx, n_experts, k,
                            n_segments, sort, sort_cutoff, rows, row_scales, expert_counts,
                            expert_offsets, segment_offsets, src_pair, dst_pos, row_expert,
                            static_scratch ? reinterpret_cast<void*>(uintptr_t(256)) : workspace,
                            static_scratch ? size_t(MOE_NOALLOC_SCRATCH_BYTES) : workspace_bytes,
                            need, a);
  if (rc) return rc;
  if (static_scratch) {
    const hipError_t e = moe::noalloc_scratch(static_cast<hipStream_t>(stream), &a.workspace);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  if (sorted_used) *sorted_used = a.sorted;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // validate mode: moe_route_dispatch only (its host copy and wait have no
  // place in the allocation-free variant)
  const bool validate = !static_scratch && validate_mode();
  if (validate) {
    a.status = validate_begin(workspace, need, s, &rc, fn);
    if (rc) return rc;
  }
  moe::RouteArgs r{logits, renormalize ? 1 : 0, topk_w};
  rc = hip_status(moe::launch_route_dispatch(r, a, s), fn);
  if (rc || !validate) return rc;
  return validate_end(a.status, s, n_experts, fn);
}

}  // namespace

extern "C" {

int moe_route_dispatch(const float* logits, int32_t renormalize, int32_t* topk_idx, float* topk_w,
                       const void* x, const float* x_scales, int32_t dtype, int64_t n_tokens,
                       int64_t hidden, int32_t n_experts, int32_t k, int32_t n_segments,
                       int32_t sort, int32_t sort_cutoff, int32_t* sorted_used, void* rows,
                       float* row_scales, int32_t* expert_counts, int32_t* expert_offsets,
                       int32_t* segment_offsets, int32_t* src_pair, int32_t* dst_pos,
                       int32_t* row_expert, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return route_dispatch_impl("moe_route_dispatch", logits, renormalize, topk_idx, topk_w, x,
                             x_scales, dtype, n_tokens, hidden, n_experts, k, n_segments, sort,
                             sort_cutoff, sorted_used, rows, row_scales, expert_counts,
                             expert_offsets, segment_offsets, src_pair, dst_pos, row_expert,
                             workspace, workspace_bytes, stream, false);
}

int moe_route_dispatch_noalloc(const float* logits, int32_t renormalize, int32_t* topk_idx,
                               float* topk_w, const void* x, const float* x_scales, int32_t dtype,
                               int64_t n_tokens, int64_t hidden, int32_t n_experts, int32_t k,
                               int32_t n_segments, int32_t sort, int32_t sort_cutoff,
                               int32_t* sorted_used, void* rows, float* row_scales,
                               int32_t* expert_counts, int32_t* expert_offsets,
                               int32_t* segment_offsets, int32_t* src_pair, int32_t* dst_pos,
                               int32_t* row_expert, void* stream) {
  return route_dispatch_impl("moe_route_dispatch_noalloc", logits, renormalize, topk_idx, topk_w,
                             x, x_scales, dtype, n_tokens, hidden, n_experts, k, n_segments, sort,
                             sort_cutoff, sorted_used, rows, row_scales, expert_counts,
                             expert_offsets, segment_offsets, src_pair, dst_pos, row_expert,
                             nullptr, 0, stream, true);
}

int moe_scatter_rows(const void* x, int64_t n_tokens, int64_t row_bytes, int32_t k,
                     const int32_t* dst_pos, void* rows, void* stream) {
  const char* fn = "moe_scatter_rows";
  if (n_tokens < 0 || row_bytes < 1 || k < 1) return fail(MOE_ERR_ARG, "%s: need n_tokens >= 0, row_bytes >= 1, k >= 1", fn);
  // one lane of a wave holds each of a token's k destinations
  if (k > MOE_MAX_TOPK) return fail(MOE_ERR_UNSUPPORTED, "%s: k > %d", fn, MOE_MAX_TOPK);
  if (n_tokens * int64_t(k) > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "%s: n_tokens * k exceeds the int32 index range", fn);
  if (n_tokens == 0) return ok();
  if (!x || !dst_pos || !rows) return fail(MOE_ERR_ARG, "%s: null pointer argument", fn);
  return hip_status(moe::launch_scatter_rows(x, n_tokens, row_bytes, k, dst_pos, rows,
                                             static_cast<hipStream_t>(stream)),
                    fn);
}

int moe_gather_rows(const void* x, int64_t n_tokens, int64_t row_bytes, int32_t k,
                    const int32_t* src_pair, int64_t n_rows, void* rows, void* stream) {
  const char* fn = "moe_gather_rows";
  if (n_tokens < 0 || n_rows < 0 || row_bytes < 1 || k < 1)
    return fail(MOE_ERR_ARG, "%s: need n_tokens, n_rows >= 0, row_bytes >= 1, k >= 1", fn);
  if (n_tokens * int64_t(k) > INT32_MAX || n_rows > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "%s: sizes exceed the int32 index range", fn);
  if (n_rows == 0) return ok();
  if (!x || !src_pair || !rows) return fail(MOE_ERR_ARG, "%s: null pointer argument", fn);
  return hip_status(moe::launch_gather_rows(x, n_tokens, row_bytes, k, src_pair, n_rows, rows,
                                            static_cast<hipStream_t>(stream)),
                    fn);
}

int moe_combine(const void* y, int32_t y_dtype, int64_t n_tokens, int64_t hidden, int32_t k,
                const int32_t* dst_pos, const float* topk_w, void* out, int32_t out_dtype,
                void* stream) {
  const char* fn = "moe_combine";
  if (n_tokens < 0) return fail(MOE_ERR_ARG, "%s: n_tokens < 0", fn);
  if (hidden < 1) return fail(MOE_ERR_ARG, "%s: hidden < 1", fn);
  if (k < 1) return fail(MOE_ERR_ARG, "%s: k < 1", fn);
  if (k > MOE_MAX_TOPK) return fail(MOE_ERR_UNSUPPORTED, "%s: k > %d", fn, MOE_MAX_TOPK);
  if ((y_dtype != MOE_F32 && y_dtype != MOE_BF16) || (out_dtype != MOE_F32 && out_dtype != MOE_BF16))
    return fail(MOE_ERR_ARG, "%s: y and out must be MOE_F32 or MOE_BF16", fn);
  if (n_tokens * int64_t(k) > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "%s: n_tokens * k exceeds the int32 index range", fn);
  if (n_tokens == 0) return ok();
  if (!y || !dst_pos || !topk_w || !out) return fail(MOE_ERR_ARG, "%s: null pointer argument", fn);
  return hip_status(moe::launch_combine(y, y_dtype == MOE_BF16, n_tokens, hidden, k, dst_pos,
                                        topk_w, out, out_dtype == MOE_BF16,
                                        static_cast<hipStream_t>(stream)),
                    fn);
}

int moe_dequant_rows(const uint8_t* rows, const float* row_scales, int64_t n_rows, int64_t hidden,
                     uint16_t* y, void* stream) {
  const char* fn = "moe_dequant_rows";
  if (n_rows < 0) return fail(MOE_ERR_ARG, "%s: n_rows < 0", fn);
  if (hidden < 1 || hidden % 128 != 0) return fail(MOE_ERR_ARG, "%s: hidden must be a positive multiple of 128", fn);
  if (n_rows == 0) return ok();
  if (!rows || !row_scales || !y) return fail(MOE_ERR_ARG, "%s: null pointer argument", fn);
  if ((reinterpret_cast<uintptr_t>(rows) | reinterpret_cast<uintptr_t>(y)) & 15)
    return fail(MOE_ERR_ARG, "%s: rows and y must be 16-byte aligned", fn);
  return hip_status(moe::launch_dequant_rows(rows, row_scales, n_rows, hidden, y,
                                             static_cast<hipStream_t>(stream)),
                    fn);
}

size_t moe_grouped_swiglu_workspace_bytes(int64_t n_rows, int32_t n_experts, int64_t hidden,
                                          int64_t ffn) {
  if (n_rows < 0 || n_experts < 1 || hidden < 1 || ffn < 1) return 0;
  return moe::grouped_swiglu_workspace_bytes(n_rows, n_experts, hidden, ffn);
}

int moe_grouped_swiglu(const void* rows, int64_t n_rows, int64_t hidden,
                       const int32_t* expert_offsets, int32_t n_experts, const void* w_gate,
                       const void* w_up, const void* w_down, int64_t ffn, void* y,
                       void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "moe_grouped_swiglu";
  if (n_rows < 0) return fail(MOE_ERR_ARG, "%s: n_rows < 0", fn);
  if (hidden < 1 || ffn < 1 || n_experts < 1) return fail(MOE_ERR_ARG, "%s: sizes must be >= 1", fn);
  if (n_experts > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "%s: n_experts > %d", fn, MOE_MAX_EXPERTS);
  if (hidden % 64 != 0 || ffn % 64 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: hidden and ffn must be multiples of 64", fn);
  if (n_rows > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "%s: n_rows exceeds the int32 range", fn);
  // per-lane load offsets within a 256-row tile are 32-bit
  if (hidden > (int64_t(1) << 22) || ffn > (int64_t(1) << 22))
    return fail(MOE_ERR_UNSUPPORTED, "%s: hidden and ffn must be at most %d", fn, 1 << 22);
  // the grid also holds up to 256 extra workgroups for the split parts of the last round
  if (moe::grouped_swiglu_tiles(n_rows, n_experts, hidden, ffn) > INT32_MAX - 8 - 256)
    return fail(MOE_ERR_UNSUPPORTED, "%s: too many tiles", fn);
  if (n_rows == 0) return ok();
  if (!rows || !expert_offsets || !w_gate || !w_up || !w_down || !y)
    return fail(MOE_ERR_ARG, "%s: null pointer argument", fn);
  // the operands are read in 16-byte runs straight into LDS
  if ((reinterpret_cast<uintptr_t>(rows) | reinterpret_cast<uintptr_t>(w_gate) |
       reinterpret_cast<uintptr_t>(w_up) | reinterpret_cast<uintptr_t>(w_down) |
       reinterpret_cast<uintptr_t>(y)) & 15)
    return fail(MOE_ERR_UNSUPPORTED, "%s: rows, weights and y must be 16-byte aligned", fn);
  const size_t need = moe::grouped_swiglu_workspace_bytes(n_rows, n_experts, hidden, ffn);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : size_t(0));
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  return hip_status(moe::launch_grouped_swiglu(rows, n_rows, hidden, expert_offsets, n_experts,
                                               w_gate, w_up, w_down, ffn, y, workspace,
                                               static_cast<hipStream_t>(stream)),
                    fn);
}

size_t moe_gather_swiglu_workspace_bytes(int64_t n_rows, int32_t n_experts, int64_t hidden,
                                         int64_t ffn) {
  if (n_rows < 0 || n_rows > INT32_MAX || n_experts < 1 || n_experts > MOE_MAX_EXPERTS ||
      hidden < 1 || ffn < 1)
    return 0;
  return moe::gather_swiglu_workspace_bytes(n_rows, n_experts, hidden, ffn);
}

int moe_gather_swiglu(const void* rows, int64_t n_rows, int64_t hidden,
                      const int32_t* row_expert, int32_t n_experts, const void* w_gate,
                      const void* w_up, const void* w_down, int64_t ffn, void* y,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "moe_gather_swiglu";
  if (n_rows < 0) return fail(MOE_ERR_ARG, "%s: n_rows < 0", fn);
  if (hidden < 1 || ffn < 1 || n_experts < 1) return fail(MOE_ERR_ARG, "%s: sizes must be >= 1", fn);
  if (n_experts > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "%s: n_experts > %d", fn, MOE_MAX_EXPERTS);
  if (hidden % 128 != 0 || ffn % 128 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: hidden and ffn must be multiples of 128", fn);
  if (n_rows > INT32_MAX || hidden > INT32_MAX || ffn > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "%s: sizes exceed the int32 range", fn);
  if (moe::gather_swiglu_tiles(n_rows, n_experts, hidden, ffn) > INT32_MAX - 8)
    return fail(MOE_ERR_UNSUPPORTED, "%s: too many tiles", fn);
  if (n_rows == 0) return ok();
  if (!rows || !row_expert || !w_gate || !w_up || !w_down || !y)
    return fail(MOE_ERR_ARG, "%s: null pointer argument", fn);
  // rows and weights are read in 16-byte runs; y is written element by element
  if ((reinterpret_cast<uintptr_t>(rows) | reinterpret_cast<uintptr_t>(w_gate) |
       reinterpret_cast<uintptr_t>(w_up) | reinterpret_cast<uintptr_t>(w_down)) & 15)
    return fail(MOE_ERR_UNSUPPORTED, "%s: rows and weights must be 16-byte aligned", fn);
  if (reinterpret_cast<uintptr_t>(y) & 1)
    return fail(MOE_ERR_UNSUPPORTED, "%s: y must be 2-byte aligned", fn);
  const size_t need = moe::gather_swiglu_workspace_bytes(n_rows, n_experts, hidden, ffn);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : size_t(0));
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  return hip_status(moe::launch_gather_swiglu(rows, n_rows, hidden, row_expert, n_experts,
                                              w_gate, w_up, w_down, ffn, y, workspace,
                                              static_cast<hipStream_t>(stream)),
                    fn);
}

int moe_gather_swiglu_combine(const void* rows, int64_t n_rows, int64_t hidden,
                              const int32_t* row_expert, const int32_t* row_pair,
                              const float* topk_w, int64_t n_tokens, int32_t k, int32_t n_experts,
                              const void* w_gate, const void* w_up, const void* w_down,
                              int64_t ffn, float* out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  const char* fn = "moe_gather_swiglu_combine";
  if (n_rows < 0 || n_tokens < 0) return fail(MOE_ERR_ARG, "%s: n_rows and n_tokens must be >= 0", fn);
  if (hidden < 1 || ffn < 1 || n_experts < 1) return fail(MOE_ERR_ARG, "%s: sizes must be >= 1", fn);
  if (k < 1 || k > moe::kMaxTopK) return fail(MOE_ERR_ARG, "%s: k must be in [1, %d]", fn, moe::kMaxTopK);
  if (n_experts > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "%s: n_experts > %d", fn, MOE_MAX_EXPERTS);
  if (hidden % 128 != 0 || ffn % 128 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: hidden and ffn must be multiples of 128", fn);
  if (n_rows > INT32_MAX || hidden > INT32_MAX || ffn > INT32_MAX || n_tokens * k > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "%s: sizes exceed the int32 range", fn);
  if (moe::gather_swiglu_tiles(n_rows, n_experts, hidden, ffn) > INT32_MAX - 8)
    return fail(MOE_ERR_UNSUPPORTED, "%s: too many tiles", fn);
  if (n_rows == 0 || n_tokens == 0) return ok();
  if (!rows || !row_expert || !topk_w || !w_gate || !w_up || !w_down || !out)
    return fail(MOE_ERR_ARG, "%s: null pointer argument", fn);
  if ((reinterpret_cast<uintptr_t>(rows) | reinterpret_cast<uintptr_t>(w_gate) |
       reinterpret_cast<uintptr_t>(w_up) | reinterpret_cast<uintptr_t>(w_down)) & 15)
    return fail(MOE_ERR_UNSUPPORTED, "%s: rows and weights must be 16-byte aligned", fn);
  if ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(topk_w)) & 3)
    return fail(MOE_ERR_UNSUPPORTED, "%s: out and topk_w must be 4-byte aligned", fn);
  const size_t need = moe::gather_swiglu_workspace_bytes(n_rows, n_experts, hidden, ffn);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : size_t(0));
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  const moe::FusedCombine fc{row_pair, topk_w, out, int(k), int(n_tokens * k)};
  return hip_status(moe::launch_gather_swiglu(rows, n_rows, hidden, row_expert, n_experts,
                                              w_gate, w_up, w_down, ffn, nullptr, workspace,
                                              static_cast<hipStream_t>(stream), &fc),
                    fn);
}

int moe_grouped_gemm_fp8(const void* rows, const float* row_scales, int64_t n_rows,
                         int64_t k_dim, const int32_t* expert_offsets, int32_t n_experts,
                         const void* w, const float* w_scales, int64_t n_dim, void* y,
                         void* stream) {
  const char* fn = "moe_grouped_gemm_fp8";
  if (n_rows < 0) return fail(MOE_ERR_ARG, "%s: n_rows < 0", fn);
  if (k_dim < 1 || n_dim < 1 || n_experts < 1) return fail(MOE_ERR_ARG, "%s: sizes must be >= 1", fn);
  if (n_experts > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "%s: n_experts > %d", fn, MOE_MAX_EXPERTS);
  if (k_dim % 128 != 0 || n_dim % 128 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: k_dim and n_dim must be multiples of 128", fn);
  if (n_rows > INT32_MAX || n_dim > INT32_MAX || k_dim > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "%s: sizes exceed the int32 range", fn);
  const int64_t tiles = ((n_rows + 63) / 64 + n_experts + 7) / 8 * 8 * (n_dim / 128);
  if (tiles > INT32_MAX - 8) return fail(MOE_ERR_UNSUPPORTED, "%s: too many tiles", fn);
  if (n_rows == 0) return ok();
  if (!rows || !row_scales || !expert_offsets || !w || !w_scales || !y)
    return fail(MOE_ERR_ARG, "%s: null pointer argument", fn);
  // operands are read in 16-byte runs; scales as 4-byte words
  if ((reinterpret_cast<uintptr_t>(rows) | reinterpret_cast<uintptr_t>(w) |
       reinterpret_cast<uintptr_t>(y)) & 15)
    return fail(MOE_ERR_UNSUPPORTED, "%s: rows, w and y must be 16-byte aligned", fn);
  if ((reinterpret_cast<uintptr_t>(row_scales) | reinterpret_cast<uintptr_t>(w_scales)) & 3)
    return fail(MOE_ERR_ARG, "%s: scales must be 4-byte aligned", fn);
  return hip_status(moe::launch_grouped_gemm_fp8(rows, row_scales, n_rows, k_dim, expert_offsets,
                                                 n_experts, w, w_scales, n_dim, y,
                                                 static_cast<hipStream_t>(stream)),
                    fn);
}

}  // extern "C"
