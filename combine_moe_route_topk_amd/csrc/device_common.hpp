// Device-side helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Lanes below this one, as a 64-bit mask.
__device__ __forceinline__ uint64_t lanemask_lt() {
  return (uint64_t(1) << lane_id()) - 1;   // lane 0 -> 0
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// bfloat16 <-> float32.  Decoding is exact; encoding rounds to nearest even and
// keeps NaN quiet.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);   // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Two bf16 packed in a 32-bit word (low half first in memory).
__device__ __forceinline__ void unpack_bf16x2(uint32_t w, float& lo, float& hi) {
  lo = __uint_as_float(w << 16);
  hi = __uint_as_float(w & 0xffff0000u);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16_rne(lo)) | (uint32_t(f32_to_bf16_rne(hi)) << 16);
}

template <typename T>
__device__ __forceinline__ T wave_reduce_max(T v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    T o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_reduce_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Exclusive scan of one int per thread over a workgroup of up to 1024
// threads; returns the exclusive prefix and writes the total to *total.
// s_wave holds (waves + 1) ints of LDS; every thread of the workgroup calls it.
__device__ inline int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) s_wave[w] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < nw; ++i) {
      const int c = s_wave[i];
      s_wave[i] = run;
      run += c;
    }
    s_wave[nw] = run;
  }
  __syncthreads();
  const int excl = s_wave[w] + incl - v;
  *total = s_wave[nw];
  return excl;
}

}  // namespace moe
