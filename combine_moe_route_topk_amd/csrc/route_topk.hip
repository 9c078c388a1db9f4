// Softmax top-k routing: one wavefront per token.
//
// Produces expert_indices [N, k] (the routing output flattened and sorted by
// the sorted gather branch of "backends/mlx: runtime MoE expert-sort for
// decode (issue #20554)", author's follow-up "Handler fixes") and fp32
// weights.  Each lane holds R = ceil(E/64) logits as 64-bit keys
//   key = (order-preserving image of the fp32 value) << 32 | ~expert
// so one unsigned max picks the larger value and, among equal values, the
// lower expert index.  -0.0 is folded onto +0.0 first.  k rounds of a wave
// max select slots 0..k-1 in order; the winning lane retires its key.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

__device__ __forceinline__ uint32_t ordered_bits(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0;                       // -0.0 == +0.0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float value_of_ordered(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

template <int R>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int64_t n_tokens, int n_experts, int k,
                                                         int renormalize,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  const int lane = lane_id();
  const int64_t t = int64_t(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (t >= n_tokens) return;                          // uniform per wave
  const float* row = logits + t * n_experts;

  uint64_t key[R];
  float val[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = lane + r * kWave;
    if (e < n_experts) {
      const float v = row[e];
      val[r] = v;
      key[r] = (uint64_t(ordered_bits(v)) << 32) | uint32_t(~uint32_t(e));
    } else {
      val[r] = 0.f;
      key[r] = 0;                                     // below every real key
    }
  }

  int my_e = 0;          // lane j < k ends up holding slot j
  float my_v = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int r = 1; r < R; ++r) best = key[r] > best ? key[r] : best;
    best = wave_reduce_max(best);
    const int e = int(~uint32_t(best));
    if ((e & (kWave - 1)) == lane) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (r == (e >> 6)) key[r] = 0;
    }
    if (lane == j) {
      my_e = e;
      my_v = value_of_ordered(uint32_t(best >> 32));
    }
  }

  const float top = __shfl(my_v, 0);                  // slot 0 is the maximum
  float num = lane < k ? expf(my_v - top) : 0.f;
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
  if (lane < k) {
    topk_idx[t * k + lane] = my_e;
    topk_w[t * k + lane] = num / den;
  }
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
