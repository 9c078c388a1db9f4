// Softmax top-k routing: one wavefront per token.
//
// Produces expert_indices [N, k] (the routing output flattened and sorted by
// the sorted gather branch of "backends/mlx: runtime MoE expert-sort for
// decode (issue #20554)", author's follow-up "Handler fixes") and fp32
// weights.  Each lane holds R = ceil(E/64) logits of the contiguous experts
// R*lane + r (one 16-byte load per lane when the row allows) as
// order-preserving unsigned images of their values (-0.0 folded onto +0.0),
// and tracks its own best (largest value, lowest expert on ties; for R <= 4
// the lane sorts its keys once and pops its head when it wins).  Each of
// the k rounds takes the wave maximum of the lanes' bests with DPP row
// operations and a ballot of the lanes that hold it; since lower lanes hold
// lower experts, the lowest such lane holds the lowest expert with that value
// and wins.  The winner retires its key.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

__device__ __forceinline__ uint32_t ordered_bits(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0;                       // -0.0 == +0.0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float value_of_ordered(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// DPP controls (GFX9 encoding).
constexpr int kQuadPerm1032 = 0xB1;   // quad_perm:[1,0,3,2]
constexpr int kQuadPerm2301 = 0x4E;   // quad_perm:[2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;

// One step of a DPP maximum.  Lanes outside ROW_MASK and lanes whose source
// is out of range read 0, the identity of an unsigned maximum, so the move
// folds into a single v_max_u32 with a DPP operand.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v) {
  const uint32_t o = uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, ROW_MASK, 0xF, true));
  return o > v ? o : v;
}

// Maximum over the wave, returned uniformly (from lane 63).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_step<kQuadPerm1032, 0xF>(v);
  v = dpp_max_step<kQuadPerm2301, 0xF>(v);
  v = dpp_max_step<kRowHalfMirror, 0xF>(v);
  v = dpp_max_step<kRowMirror, 0xF>(v);
  v = dpp_max_step<kRowBcast15, 0xA>(v);
  v = dpp_max_step<kRowBcast31, 0xC>(v);
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}

// One step of a DPP sum: lanes outside ROW_MASK and lanes whose source is out
// of range add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_sum_step(float v) {
  const float o = __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, true));
  return v + o;
}

// Sum over the wave with DPP row operations (a tree of depth 6), returned
// uniformly (from lane 63).
__device__ __forceinline__ float wave_sum_f32(float v) {
  v = dpp_sum_step<kQuadPerm1032, 0xF>(v);
  v = dpp_sum_step<kQuadPerm2301, 0xF>(v);
  v = dpp_sum_step<kRowHalfMirror, 0xF>(v);
  v = dpp_sum_step<kRowMirror, 0xF>(v);
  v = dpp_sum_step<kRowBcast15, 0xA>(v);
  v = dpp_sum_step<kRowBcast31, 0xC>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// exp(a - b) without the rounding error of the fp32 difference.  Knuth's
// two-sum splits a - b exactly into s + r with s = fl(a - b) and |r| <= ulp(s)/2;
// then exp(a - b) = exp(s) * exp(r) = exp(s) * (1 + r) to far below fp32
// precision.  A plain expf(a - b) would carry the difference's relative error
// times |a - b| into the result (up to ~5e-6 relative at |a - b| ~ 80).
__device__ __forceinline__ float exp_diff(float a, float b) {
  const float c = -b;
  const float s = a + c;
  const float cc = s - a;
  const float r = (a - (s - cc)) + (c - cc);
  const float e = expf(s);
  return fmaf(e, r, e);
}

// Loads one token's logits: lane l holds experts R*l + r, with 16-byte loads
// when R is a multiple of 4, the row is 16-byte aligned and the lane's
// experts all exist (the choice is uniform over the lanes that take it).
template <int R>
__device__ __forceinline__ void load_token(const float* __restrict__ row, int n_experts,
                                           float (&val)[R]) {
  const int e0 = lane_id() * R;
  if (R % 4 == 0 && (reinterpret_cast<uintptr_t>(row) & 15) == 0 && e0 + R <= n_experts) {
#pragma unroll
    for (int r = 0; r < R; r += 4) {
      const float4 v = *reinterpret_cast<const float4*>(row + e0 + r);
      val[r] = v.x;
      val[r + 1] = v.y;
      val[r + 2] = v.z;
      val[r + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) val[r] = e0 + r < n_experts ? row[e0 + r] : 0.f;
  }
}

// Routes one token with the calling wave from its loaded logits: returns, in
// lane j < k, the expert of slot j and its weight.
template <int R>
__device__ __forceinline__ void select_token(const float (&val)[R], int n_experts, int k,
                                             int renormalize, int& out_e, float& out_w) {
  const int lane = lane_id();
  uint32_t ov[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    ov[r] = lane * R + r < n_experts ? ordered_bits(val[r]) : 0u;   // 0: below every value
  int my_e = 0;          // lane j < k ends up holding slot j ...
  uint32_t my_o = 0u;    // ... and its key (decoded to the logit after the rounds)
  if constexpr (R <= 4) {
    // Each lane sorts its keys once (value descending, lower expert first on
    // ties: a strict total order, so any compare-exchange network sorts
    // them); a round's winner then pops its head, with no re-scan and no
    // branch.
    uint32_t key[R];
    int rid[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      key[r] = ov[r];
      rid[r] = r;
    }
    auto cex = [&](int a, int b) {      // positions a < b: put the larger pair first
      const bool sw = key[b] > key[a] || (key[b] == key[a] && rid[b] < rid[a]);
      const uint32_t ka = key[a], kb = key[b];
      const int ra = rid[a], rb = rid[b];
      key[a] = sw ? kb : ka;
      key[b] = sw ? ka : kb;
      rid[a] = sw ? rb : ra;
      rid[b] = sw ? ra : rb;
    };
    if constexpr (R == 2) cex(0, 1);
    if constexpr (R == 4) {
      cex(0, 1); cex(2, 3); cex(0, 2); cex(1, 3); cex(1, 2);
    }
    for (int j = 0; j < k; ++j) {
      const uint32_t m = wave_max_u32(key[0]);
      const uint64_t cand = ballot(key[0] == m);                // never empty
      const int wl = int(__builtin_ctzll(cand));                // lowest lane: lowest expert
      const int win = wl * R + __builtin_amdgcn_readlane(rid[0], wl);
      const bool me = lane == wl;
#pragma unroll
      for (int r = 0; r + 1 < R; ++r) {
        key[r] = me ? key[r + 1] : key[r];
        rid[r] = me ? rid[r + 1] : rid[r];
      }
      key[R - 1] = me ? 0u : key[R - 1];
      if (lane == j) {
        my_e = win;
        my_o = m;
      }
    }
  } else {
    auto local_best = [&](uint32_t& bo, int& br) {
      bo = ov[0];
      br = 0;
#pragma unroll
      for (int r = 1; r < R; ++r)
        if (ov[r] > bo) { bo = ov[r]; br = r; }         // strict: lower r wins ties
    };
    uint32_t best_o;
    int best_r;
    local_best(best_o, best_r);
    for (int j = 0; j < k; ++j) {
      const uint32_t m = wave_max_u32(best_o);
      const uint64_t cand = ballot(best_o == m);                // never empty
      const int wl = int(__builtin_ctzll(cand));                // lowest lane: lowest expert
      const int wr = __builtin_amdgcn_readlane(best_r, wl);
      const int win = wl * R + wr;
      if (lane == wl) {
#pragma unroll
        for (int r = 0; r < R; ++r)
          if (r == wr) ov[r] = 0u;
        local_best(best_o, best_r);
      }
      if (lane == j) {
        my_e = win;
        my_o = m;
      }
    }
  }

  const float my_v = value_of_ordered(my_o);
  // slot 0 holds the maximum
  const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
  const float num = lane < k ? exp_diff(my_v, top) : 0.f;
  float den;
  if (renormalize) {
    den = wave_sum_f32(num);
  } else {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (lane * R + r < n_experts) s += exp_diff(val[r], top);
    den = wave_sum_f32(s);
  }
  out_e = my_e;
  out_w = num / den;
}

template <int R>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int64_t n_tokens, int n_experts, int k,
                                                         int renormalize,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  const int lane = lane_id();
  const int64_t t = int64_t(blockIdx.x) * (blockDim.x / kWave) +
                    __builtin_amdgcn_readfirstlane(int(threadIdx.x / kWave));
  if (t >= n_tokens) return;                          // uniform per wave
  float val[R];
  load_token<R>(logits + t * n_experts, n_experts, val);
  int e;
  float w;
  select_token<R>(val, n_experts, k, renormalize, e, w);
  if (lane < k) {
    topk_idx[t * k + lane] = e;
    topk_w[t * k + lane] = w;
  }
}

// Routing and the identity-layout row copy in one launch.  With one segment
// and no sort, pair t*k+j lands in row t*k+j ("backends/mlx: runtime MoE
// expert-sort for decode (issue #20554)": the unsorted branch repeats each
// token top_k times with identity inv_order), so the copy needs nothing from
// the routing: workgroups [0, route_blocks) route (one wave per token) and
// the rest copy (one wave per (token, 2 KB slice), 16-byte accesses), side by
// side with no synchronisation between them.  The routing waves also write
// the identity maps of their pairs (dst_pos = src_pair = q, row_expert = the
// routed expert), leaving only the counts and offsets to the next launch.
template <int R, int U>
__global__ __launch_bounds__(256) void route_copy_kernel(
    const float* __restrict__ logits, int64_t n_tokens, int n_experts, int k, int renormalize,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int route_blocks,
    const uint4* __restrict__ x, int64_t nvec, int n_slices, uint4* __restrict__ rows,
    int32_t* __restrict__ dst_pos, int32_t* __restrict__ src_pair,
    int32_t* __restrict__ row_expert) {
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x / kWave));
  const int blk = __builtin_amdgcn_readfirstlane(int(blockIdx.x));
  if (blk < route_blocks) {
    const int64_t t = int64_t(blk) * (256 / kWave) + w;
    if (t >= n_tokens) return;
    float val[R];
    load_token<R>(logits + t * n_experts, n_experts, val);
    int e;
    float wt;
    select_token<R>(val, n_experts, k, renormalize, e, wt);
    if (lane < k) {
      const int32_t q = int32_t(t * k + lane);
      topk_idx[q] = e;
      topk_w[q] = wt;
      dst_pos[q] = q;
      src_pair[q] = q;
      if (row_expert) row_expert[q] = e;
    }
    return;
  }
  const int64_t item = int64_t(blk - route_blocks) * (256 / kWave) + w;
  const int64_t t = item / n_slices;
  if (t >= n_tokens) return;
  const int64_t v0 = (item - t * n_slices) * int64_t(kWave * U) + lane;
  const uint4* src = x + t * nvec;
  uint4 buf[U];
  int64_t vi[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    vi[u] = v0 + u * kWave < nvec ? v0 + u * kWave : nvec - 1;   // clamped lanes repeat a value
    const unsigned int __attribute__((ext_vector_type(4))) q =
        __builtin_nontemporal_load(reinterpret_cast<const unsigned int __attribute__((ext_vector_type(4)))*>(src + vi[u]));
    buf[u] = make_uint4(q.x, q.y, q.z, q.w);
  }
#pragma unroll
  for (int u = 0; u < U; ++u)   // wait for the loads once, before the stores
    asm volatile("" : "+v"(buf[u].x), "+v"(buf[u].y), "+v"(buf[u].z), "+v"(buf[u].w));
  // non-temporal stores: the copy leaves no dirty lines in L2, so the release
  // at the end of the launch has little to write back before the next one starts
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4* dst = reinterpret_cast<u32x4*>(rows + t * int64_t(k) * nvec);
  for (int j = 0; j < k; ++j) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x4 o = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
      __builtin_nontemporal_store(o, dst + vi[u]);
    }
    dst += nvec;
  }
}

}  // namespace

hipError_t launch_route_copy_identity(const float* logits, int64_t n_tokens, int n_experts, int k,
                                      int renormalize, int32_t* topk_idx, float* topk_w,
                                      const void* x, int64_t row_bytes, void* rows,
                                      int32_t* dst_pos, int32_t* src_pair, int32_t* row_expert,
                                      hipStream_t stream) {
  constexpr int kBlock = 256;
  const int per_block = kBlock / kWave;
  const int route_blocks = int((n_tokens + per_block - 1) / per_block);
  const int64_t nvec = row_bytes / 16;
  // decode-sized batches: 1 KB copy slices (twice the waves) instead of 2 KB
  const bool small = n_tokens * ((nvec + 127) / 128) < 4096;
  const int U = small ? 1 : 2;
  const int n_slices = int((nvec + kWave * U - 1) / (kWave * U));
  const int64_t copy_blocks = (n_tokens * n_slices + per_block - 1) / per_block;
  const dim3 grid(unsigned(route_blocks + copy_blocks));
  const int r = (n_experts + kWave - 1) / kWave;
#define MOE_ROUTE_COPY_CASE(RR)                                                              \
  if (small)                                                                                 \
    route_copy_kernel<RR, 1><<<grid, kBlock, 0, stream>>>(                                  \
        logits, n_tokens, n_experts, k, renormalize, topk_idx, topk_w, route_blocks,         \
        static_cast<const uint4*>(x), nvec, n_slices, static_cast<uint4*>(rows), dst_pos,    \
        src_pair, row_expert);                                                               \
  else                                                                                       \
    route_copy_kernel<RR, 2><<<grid, kBlock, 0, stream>>>(                                  \
        logits, n_tokens, n_experts, k, renormalize, topk_idx, topk_w, route_blocks,         \
        static_cast<const uint4*>(x), nvec, n_slices, static_cast<uint4*>(rows), dst_pos,    \
        src_pair, row_expert);                                                               \
  break;
  switch (r <= 1 ? 1 : r <= 2 ? 2 : r <= 4 ? 4 : r <= 8 ? 8 : 16) {
    case 1: MOE_ROUTE_COPY_CASE(1)
    case 2: MOE_ROUTE_COPY_CASE(2)
    case 4: MOE_ROUTE_COPY_CASE(4)
    case 8: MOE_ROUTE_COPY_CASE(8)
    default: MOE_ROUTE_COPY_CASE(16)
  }
#undef MOE_ROUTE_COPY_CASE
  return hipGetLastError();
}

hipError_t launch_route_topk(const float* logits, int64_t n_tokens, int n_experts, int k,
                             int renormalize, int32_t* topk_idx, float* topk_w,
                             hipStream_t stream) {
  constexpr int kBlock = 256;
  const int per_block = kBlock / kWave;
  const dim3 grid(unsigned((n_tokens + per_block - 1) / per_block));
  const int r = (n_experts + kWave - 1) / kWave;
#define MOE_ROUTE_CASE(RR)                                                                  \
  route_topk_kernel<RR><<<grid, kBlock, 0, stream>>>(logits, n_tokens, n_experts, k,       \
                                                     renormalize, topk_idx, topk_w);        \
  break;
  switch (r <= 1 ? 1 : r <= 2 ? 2 : r <= 4 ? 4 : r <= 8 ? 8 : 16) {
    case 1: MOE_ROUTE_CASE(1)
    case 2: MOE_ROUTE_CASE(2)
    case 4: MOE_ROUTE_CASE(4)
    case 8: MOE_ROUTE_CASE(8)
    default: MOE_ROUTE_CASE(16)
  }
#undef MOE_ROUTE_CASE
  return hipGetLastError();
}

}  // namespace moe
