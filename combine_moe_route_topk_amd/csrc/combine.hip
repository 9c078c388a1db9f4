// Combine: weighted top-k gather-sum back to token order, and the fp8
// identity expert (dequantisation of dispatched rows).
//
//   out[t, i] = sum_{j<k} w[t, j] * y[dst_pos[t*k + j], i]
//
// combine_weighted_sum of "MLX expert parallelism all_to_all PR 3158" (Facts);
// dst_pos is the inv_order map with which "backends/mlx: runtime MoE
// expert-sort for decode (issue #20554)" (CI write-up) brings expert outputs
// back to token order, so unscatter and sum are one pass.
//
// One wave per (token, slice): for each slot j the wave reads a contiguous
// slice of row dst_pos[t*k+j] (16-byte loads), and every lane keeps an fp32
// FMA chain acc = fma(w_j, y_j, acc) in slot order j = 0..k-1.  The order
// never depends on where dispatch put the rows, so sorted and unsorted
// layouts give bit-identical outputs.  Rounding to bf16 is nearest-even.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kBlock = 256;
constexpr int kGroup = 8;          // elements per lane per load group

template <typename T> struct Elem;
template <> struct Elem<float> {   // a group of 8 floats is two 16-byte loads
  __device__ static void load(const float* row, int64_t g, float (&v)[kGroup]) {
    const uint4* p = reinterpret_cast<const uint4*>(row) + 2 * g;
    const uint4 a = p[0], b = p[1];
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
    v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
  __device__ static void store(float* row, int64_t g, const float (&v)[kGroup]) {
    uint4* p = reinterpret_cast<uint4*>(row) + 2 * g;
    p[0] = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                      __float_as_uint(v[3]));
    p[1] = make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
                      __float_as_uint(v[7]));
  }
  __device__ static float load1(const float* row, int64_t i) { return row[i]; }
  __device__ static void store1(float* row, int64_t i, float v) { row[i] = v; }
};
template <> struct Elem<uint16_t> {   // bfloat16 bit patterns
  __device__ static void load(const uint16_t* row, int64_t g, float (&v)[kGroup]) {
    const uint4 a = reinterpret_cast<const uint4*>(row)[g];
    unpack_bf16x2(a.x, v[0], v[1]);
    unpack_bf16x2(a.y, v[2], v[3]);
    unpack_bf16x2(a.z, v[4], v[5]);
    unpack_bf16x2(a.w, v[6], v[7]);
  }
  __device__ static void store(uint16_t* row, int64_t g, const float (&v)[kGroup]) {
    reinterpret_cast<uint4*>(row)[g] = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                  pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
  }
  __device__ static float load1(const uint16_t* row, int64_t i) { return bf16_to_f32(row[i]); }
  __device__ static void store1(uint16_t* row, int64_t i, float v) { row[i] = f32_to_bf16_rne(v); }
};

// Vector path: D % 8 == 0 and 16-byte aligned rows.  Each lane owns U groups
// of 8 consecutive elements; a slice is 64 * U groups.  Slots are taken KB at
// a time: all KB * U row loads of a batch are issued back to back from
// clamped (always valid) addresses, and slots that do not exist or carry an
// out-of-range position are masked out of the FMA chain instead of branched
// around, so no load waits for another.
// Row loads are non-temporal: each expert-output row is read exactly once.
// Measured on MI355X at the prefill shape, this keeps the combine from
// evicting the just-dispatched rows that are still dirty in the last-level
// cache through ordinary allocations, and cut the dispatch + combine pair
// from ~240 us to ~190 us.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load_stream(const void* p) {
  return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
}

template <typename TY> struct Raw;
template <> struct Raw<uint16_t> {
  u32x4 v;
  __device__ void load(const uint16_t* row, int64_t g) { v = load_stream(row + 8 * g); }
  __device__ void to_f32(float (&o)[kGroup]) const {
    unpack_bf16x2(v.x, o[0], o[1]); unpack_bf16x2(v.y, o[2], o[3]);
    unpack_bf16x2(v.z, o[4], o[5]); unpack_bf16x2(v.w, o[6], o[7]);
  }
};
template <> struct Raw<float> {
  u32x4 a, b;
  __device__ void load(const float* row, int64_t g) {
    a = load_stream(row + 8 * g);
    b = load_stream(row + 8 * g + 4);
  }
  __device__ void to_f32(float (&o)[kGroup]) const {
    o[0] = __uint_as_float(a.x); o[1] = __uint_as_float(a.y);
    o[2] = __uint_as_float(a.z); o[3] = __uint_as_float(a.w);
    o[4] = __uint_as_float(b.x); o[5] = __uint_as_float(b.y);
    o[6] = __uint_as_float(b.z); o[7] = __uint_as_float(b.w);
  }
};

template <typename TY, typename TO, int U, int KB>
__global__ __launch_bounds__(kBlock) void combine_kernel(const TY* __restrict__ y, int64_t n_tokens,
                                                         int64_t hidden, int k, int n_slices,
                                                         const int32_t* __restrict__ dst_pos,
                                                         const float* __restrict__ topk_w,
                                                         int64_t nk, TO* __restrict__ out) {
  const int lane = lane_id();
  const int64_t item = __builtin_amdgcn_readfirstlane(int(blockIdx.x)) * int64_t(kBlock / kWave) +
                       __builtin_amdgcn_readfirstlane(int(threadIdx.x / kWave));
  const int64_t t = item / n_slices;
  if (t >= n_tokens) return;
  const int64_t ngroups = hidden / kGroup;
  const int64_t g0 = (item - t * n_slices) * int64_t(kWave * U) + lane;
  int64_t gi[U];
  bool gok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    gok[u] = g0 + u * kWave < ngroups;
    gi[u] = gok[u] ? g0 + u * kWave : ngroups - 1;
  }

  float acc[U][kGroup];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int i = 0; i < kGroup; ++i) acc[u][i] = 0.f;

  // lane j < k holds slot j's position and weight; slots are read with readlane
  const int my_p = lane < k ? dst_pos[t * k + lane] : -1;
  const float my_w = lane < k ? topk_w[t * k + lane] : 0.f;
  for (int j0 = 0; j0 < k; j0 += KB) {
    Raw<TY> raw[KB][U];
    const TY* row[KB];
    bool use[KB];
    float wj[KB];
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
      const int p = __builtin_amdgcn_readlane(my_p, j0 + jj);   // -1 past the last slot
      use[jj] = unsigned(p) < uint64_t(nk);
      wj[jj] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), j0 + jj));
      row[jj] = y + int64_t(use[jj] ? p : 0) * hidden;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int jj = 0; jj < KB; ++jj)
#pragma unroll
      for (int u = 0; u < U; ++u) raw[jj][u].load(row[jj], gi[u]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float v[kGroup];
        raw[jj][u].to_f32(v);
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
          const float f = __builtin_fmaf(wj[jj], v[i], acc[u][i]);
          acc[u][i] = use[jj] ? f : acc[u][i];
        }
      }
    }
  }
  TO* orow = out + t * hidden;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (gok[u]) Elem<TO>::store(orow, gi[u], acc[u]);
}

// Scalar path for any D: one element per lane, a slice is 64 elements.
template <typename TY, typename TO>
__global__ __launch_bounds__(kBlock) void combine_scalar_kernel(
    const TY* __restrict__ y, int64_t n_tokens, int64_t hidden, int k, int n_slices,
    const int32_t* __restrict__ dst_pos, const float* __restrict__ topk_w, int64_t nk,
    TO* __restrict__ out) {
  const int lane = lane_id();
  const int64_t item = __builtin_amdgcn_readfirstlane(int(blockIdx.x)) * int64_t(kBlock / kWave) +
                       __builtin_amdgcn_readfirstlane(int(threadIdx.x / kWave));
  const int64_t t = item / n_slices;
  if (t >= n_tokens) return;
  const int64_t i = (item - t * n_slices) * kWave + lane;
  if (i >= hidden) return;
  float acc = 0.f;
  for (int j = 0; j < k; ++j) {
    const int p = dst_pos[t * k + j];
    if (unsigned(p) >= uint64_t(nk)) continue;
    acc = __builtin_fmaf(topk_w[t * k + j], Elem<TY>::load1(y + int64_t(p) * hidden, i), acc);
  }
  Elem<TO>::store1(out + t * hidden, i, acc);
}

template <typename TY, typename TO>
hipError_t launch_combine_typed(const void* y, int64_t n_tokens, int64_t hidden, int k,
                                const int32_t* dst_pos, const float* topk_w, void* out,
                                hipStream_t stream) {
  const int64_t nk = n_tokens * k;
  const int per_block = kBlock / kWave;
  const bool aligned = ((reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
  // Fewer than 4096 two-kilobyte items (decode-sized batches): 1 KB slices
  // double the waves of a launch that is latency-bound, not bandwidth-bound.
  if (hidden % kGroup == 0 && aligned && n_tokens * ((hidden / kGroup + 127) / 128) < 4096) {
    constexpr int U = 1;
    const int64_t ngroups = hidden / kGroup;
    const int n_slices = int((ngroups + kWave * U - 1) / (kWave * U));
    const int64_t items = n_tokens * n_slices;
    const unsigned blocks = unsigned((items + per_block - 1) / per_block);
    const TY* yy = static_cast<const TY*>(y);
    TO* oo = static_cast<TO*>(out);
    if (k >= 8)
      combine_kernel<TY, TO, U, 8><<<blocks, kBlock, 0, stream>>>(yy, n_tokens, hidden, k, n_slices, dst_pos, topk_w, nk, oo);
    else if (k >= 4)
      combine_kernel<TY, TO, U, 4><<<blocks, kBlock, 0, stream>>>(yy, n_tokens, hidden, k, n_slices, dst_pos, topk_w, nk, oo);
    else if (k >= 2)
      combine_kernel<TY, TO, U, 2><<<blocks, kBlock, 0, stream>>>(yy, n_tokens, hidden, k, n_slices, dst_pos, topk_w, nk, oo);
    else
      combine_kernel<TY, TO, U, 1><<<blocks, kBlock, 0, stream>>>(yy, n_tokens, hidden, k, n_slices, dst_pos, topk_w, nk, oo);
  } else if (hidden % kGroup == 0 && aligned) {
    constexpr int U = 2;
    const int64_t ngroups = hidden / kGroup;
    const int n_slices = int((ngroups + kWave * U - 1) / (kWave * U));
    const int64_t items = n_tokens * n_slices;
    const unsigned blocks = unsigned((items + per_block - 1) / per_block);
    const TY* yy = static_cast<const TY*>(y);
    TO* oo = static_cast<TO*>(out);
    if (k >= 8)
      combine_kernel<TY, TO, U, 8><<<blocks, kBlock, 0, stream>>>(yy, n_tokens, hidden, k, n_slices, dst_pos, topk_w, nk, oo);
    else if (k >= 4)
      combine_kernel<TY, TO, U, 4><<<blocks, kBlock, 0, stream>>>(yy, n_tokens, hidden, k, n_slices, dst_pos, topk_w, nk, oo);
    else if (k >= 2)
      combine_kernel<TY, TO, U, 2><<<blocks, kBlock, 0, stream>>>(yy, n_tokens, hidden, k, n_slices, dst_pos, topk_w, nk, oo);
    else
      combine_kernel<TY, TO, U, 1><<<blocks, kBlock, 0, stream>>>(yy, n_tokens, hidden, k, n_slices, dst_pos, topk_w, nk, oo);
  } else {
    const int n_slices = int((hidden + kWave - 1) / kWave);
    const int64_t items = n_tokens * n_slices;
    combine_scalar_kernel<TY, TO><<<unsigned((items + per_block - 1) / per_block), kBlock, 0, stream>>>(
        static_cast<const TY*>(y), n_tokens, hidden, k, n_slices, dst_pos, topk_w, nk,
        static_cast<TO*>(out));
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- fp8 identity expert
// E4M3FN decode from the format definition: exponent bias 7, subnormals
// m * 2^-9, no infinities (S.1111.111 is NaN).
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t b) {
  const uint32_t s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
  float v;
  if (e == 0) v = float(m) * 0x1p-9f;
  else if (e == 15 && m == 7) v = __uint_as_float(0x7fc00000u);
  else v = __uint_as_float(((e + 120u) << 23) | (m << 20));   // (1 + m/8) * 2^(e-7)
  return s ? -v : v;
}

// Correctly rounded bf16 of the exact product a*b.  a has at most 4
// significant bits and b 24, so the product is exact in fp64.  It is rounded
// to odd in fp32 (toward zero, last bit set when inexact) and that once more
// to nearest even in bf16; with 16 spare bits the double rounding equals a
// single correct rounding (Boldo & Melquiond, "When double rounding is odd",
// 2005).  Subnormal results are covered because the fp64 -> fp32 step rounds
// on the fp32 subnormal grid.
__device__ __forceinline__ uint16_t mul_to_bf16(float a, float b) {
  const double p = double(a) * double(b);
  float r = __double2float_rz(p);
  if (double(r) != p && !__builtin_isnan(p) && !__builtin_isinf(r))
    r = __uint_as_float(__float_as_uint(r) | 1u);
  return f32_to_bf16_rne(r);
}

__global__ __launch_bounds__(kBlock) void dequant_kernel(const uint8_t* __restrict__ rows,
                                                         const float* __restrict__ scales,
                                                         int64_t n_rows, int64_t hidden,
                                                         uint16_t* __restrict__ y) {
  // each thread: 16 consecutive elements of one row (hidden % 128 == 0)
  const int64_t per_row = hidden / 16;
  const int64_t gid = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  if (gid >= n_rows * per_row) return;
  const int64_t r = gid / per_row;
  const int64_t c = (gid - r * per_row) * 16;
  const uint4 q = *reinterpret_cast<const uint4*>(rows + r * hidden + c);
  const float s = scales[r * (hidden / 128) + c / 128];
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t a = mul_to_bf16(e4m3fn_to_f32(w[i] & 0xffu), s);
    const uint16_t b = mul_to_bf16(e4m3fn_to_f32((w[i] >> 8) & 0xffu), s);
    const uint16_t c2 = mul_to_bf16(e4m3fn_to_f32((w[i] >> 16) & 0xffu), s);
    const uint16_t d = mul_to_bf16(e4m3fn_to_f32(w[i] >> 24), s);
    o[2 * i] = uint32_t(a) | (uint32_t(b) << 16);
    o[2 * i + 1] = uint32_t(c2) | (uint32_t(d) << 16);
  }
  uint4* dst = reinterpret_cast<uint4*>(y + r * hidden + c);
  dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
  dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

}  // namespace

hipError_t launch_combine(const void* y, int y_bf16, int64_t n_tokens, int64_t hidden, int k,
                          const int32_t* dst_pos, const float* topk_w, void* out, int out_bf16,
                          hipStream_t stream) {
  if (y_bf16 && out_bf16)
    return launch_combine_typed<uint16_t, uint16_t>(y, n_tokens, hidden, k, dst_pos, topk_w, out, stream);
  if (y_bf16)
    return launch_combine_typed<uint16_t, float>(y, n_tokens, hidden, k, dst_pos, topk_w, out, stream);
  if (out_bf16)
    return launch_combine_typed<float, uint16_t>(y, n_tokens, hidden, k, dst_pos, topk_w, out, stream);
  return launch_combine_typed<float, float>(y, n_tokens, hidden, k, dst_pos, topk_w, out, stream);
}

hipError_t launch_dequant_rows(const uint8_t* rows, const float* row_scales, int64_t n_rows,
                               int64_t hidden, uint16_t* y, hipStream_t stream) {
  const int64_t threads = n_rows * (hidden / 16);
  dequant_kernel<<<unsigned((threads + kBlock - 1) / kBlock), kBlock, 0, stream>>>(
      rows, row_scales, n_rows, hidden, y);
  return hipGetLastError();
}

}  // namespace moe
