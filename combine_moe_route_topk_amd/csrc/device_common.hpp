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

// One step of a DPP integer scan: lanes outside ROW_MASK and lanes whose
// source is out of range add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_add_step(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
}

// Inclusive prefix sum over the wave with DPP row operations (no LDS
// crossbar round trips): shifts by 1, 2, 4, 8 within each 16-lane row, then
// row 0's and row 2's last lanes are broadcast into rows 1 and 3, then lane
// 31 into rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v = dpp_add_step<0x111, 0xF>(v);    // row_shr:1
  v = dpp_add_step<0x112, 0xF>(v);    // row_shr:2
  v = dpp_add_step<0x114, 0xF>(v);    // row_shr:4
  v = dpp_add_step<0x118, 0xF>(v);    // row_shr:8
  v = dpp_add_step<0x142, 0xA>(v);    // row_bcast:15
  v = dpp_add_step<0x143, 0xC>(v);    // row_bcast:31
  return v;
}

// Inclusive running maximum over the wave, for values >= 0 (the same DPP
// steps as the scan; out-of-range sources read 0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_max_step_nonneg(int v) {
  const int o = __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
  return o > v ? o : v;
}
__device__ __forceinline__ int wave_inclusive_max_nonneg(int v) {
  v = dpp_max_step_nonneg<0x111, 0xF>(v);
  v = dpp_max_step_nonneg<0x112, 0xF>(v);
  v = dpp_max_step_nonneg<0x114, 0xF>(v);
  v = dpp_max_step_nonneg<0x118, 0xF>(v);
  v = dpp_max_step_nonneg<0x142, 0xA>(v);
  v = dpp_max_step_nonneg<0x143, 0xC>(v);
  return v;
}

// The value of lane l - 1 in lane l (lane 0 reads `first`).
__device__ __forceinline__ int wave_shift_up1(int v, int first) {
  const int o = __builtin_amdgcn_update_dpp(0, v, 0x138, 0xF, 0xF, true);   // wave_shr:1
  return lane_id() == 0 ? first : o;
}

// Value of lane `src` (wave-uniform) in every lane.
__device__ __forceinline__ int lane_value(int v, int src) {
  return __builtin_amdgcn_readlane(v, src);
}

// Exclusive scan of one int per thread over a workgroup of up to 1024
// threads; returns the exclusive prefix and writes the total to *total.
// s_wave holds (waves + 1) ints of LDS; every thread of the workgroup calls it.
__device__ inline int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const int incl = wave_inclusive_scan(v);
  if (lane == kWave - 1) s_wave[w] = incl;
  __syncthreads();
  if (w == 0) {                       // the per-wave totals, scanned by wave 0
    const int t = lane < nw ? s_wave[lane] : 0;
    const int inc = wave_inclusive_scan(t);
    if (lane < nw) s_wave[lane] = inc - t;
    if (lane == nw - 1) s_wave[nw] = inc;
  }
  __syncthreads();
  const int excl = s_wave[w] + incl - v;
  *total = s_wave[nw];
  return excl;
}

}  // namespace moe
