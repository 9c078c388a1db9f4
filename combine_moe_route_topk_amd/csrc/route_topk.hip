// Softmax top-k routing: one wavefront per token.
//
// Produces expert_indices [N, k] (the routing output flattened and sorted by
// the sorted gather branch of "backends/mlx: runtime MoE expert-sort for
// decode (issue #20554)", author's follow-up "Handler fixes") and fp32
// weights.  Each lane holds R = ceil(E/64) logits of experts lane + 64*r as
// order-preserving unsigned images of their values (-0.0 folded onto +0.0),
// and tracks its own best (largest value, lowest expert on ties).  Each of
// the k rounds takes the wave maximum of the lanes' bests with DPP row
// operations and a ballot of the lanes that hold it; the lowest expert id
// among them wins (a second reduction runs only when values tie).  The winner
// retires its key.
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

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v) {
  const uint32_t o = uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), CTRL, ROW_MASK, 0xF, false));
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

__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const int o = __shfl_xor(v, off);
    v = o < v ? o : v;
  }
  return v;
}

// Loads one token's logits: lane l holds experts l + 64 r.
template <int R>
__device__ __forceinline__ void load_token(const float* __restrict__ row, int n_experts,
                                           float (&val)[R]) {
  const int lane = lane_id();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = lane + r * kWave;
    val[r] = e < n_experts ? row[e] : 0.f;
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
    ov[r] = lane + r * kWave < n_experts ? ordered_bits(val[r]) : 0u;   // 0: below every value
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

  int my_e = 0;          // lane j < k ends up holding slot j
  float my_v = 0.f;
  for (int j = 0; j < k; ++j) {
    const uint32_t m = wave_max_u32(best_o);
    const uint64_t cand = ballot(best_o == m);
    int win;
    if (__popcll(cand) == 1) {
      const int wl = __ffsll((unsigned long long)cand) - 1;
      win = wl + kWave * __builtin_amdgcn_readlane(best_r, wl);
    } else {
      win = wave_min_i32(best_o == m ? lane + kWave * best_r : 0x7fffffff);
    }
    if ((win & (kWave - 1)) == lane) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (r == (win >> 6)) ov[r] = 0u;
      local_best(best_o, best_r);
    }
    if (lane == j) {
      my_e = win;
      my_v = value_of_ordered(m);
    }
  }

  const float top = __shfl(my_v, 0);                  // slot 0 is the maximum
  const float num = lane < k ? expf(my_v - top) : 0.f;
  float den;
  if (renormalize) {
    den = wave_reduce_sum(num);
  } else {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (lane + r * kWave < n_experts) s += expf(val[r] - top);
    den = wave_reduce_sum(s);
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

}  // namespace

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
