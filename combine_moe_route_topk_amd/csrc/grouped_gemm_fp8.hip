// fp8 block-scaled grouped expert GEMM reading the dispatched fp8 rows in
// place.
//
// "One-Sided Expert-Parallel All-to-All for Mixture-of-Experts Inference over
// NVLink" (abstract): the dispatch does not depend on the activation
// quantisation format, and the grouped GEMMs read the received buffers in
// place.  Here the consumer takes the dispatched rows exactly as the fp8
// dispatch leaves them: E4M3FN codes with one float32 scale per 128 elements
// of a row, grouped by expert (expert e owns rows [offs[e], offs[e+1])).
// Weights are E4M3FN codes [E, N, K] with one float32 scale per 128 x 128
// block [E, N/128, K/128].  For a row p of expert e:
//   y[p, n] = bf16( sum_b sx[p, b] * sw[e, n/128, b] * sum_{k in b} q(x[p,k]) q(w[e,n,k]) )
//
// With ~32 rows per expert (1024 tokens, top-8 over 256 experts) each weight
// byte feeds ~64 FLOP: the kernel streams weights from HBM, so it is shaped
// for that rather than for matrix-core peak.
//   * a tile is 64 rows x 128 columns of one expert; its 4 waves each own 32
//     columns and both 32-row halves, and run independently (no LDS operand
//     staging, no barrier in the K loop);
//   * operands go from global memory straight into registers in the
//     v_mfma_f32_32x32x16_fp8_fp8 layout: lane l holds row / column l % 32 and
//     64 contiguous bytes of each 128-wide K block (half l / 32), so every
//     weight row is read as whole 128-byte lines.  The eight MFMAs of a block
//     take 8-byte groups g of those 64 bytes, which permutes K identically on
//     both operands;
//   * each block's fp32 partial sum is scaled by sx * sw and added to the
//     accumulator; the row scales of the tile are staged once in LDS,
//     transposed, so a lane's four consecutive rows are one 16-byte read;
//   * the next block's operands are loaded while the current block is
//     multiplied (two register sets);
//   * tiles run column-fastest: the workgroups one XCD runs together share an
//     expert's rows from L2 while each streams its own weight slab.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kQB = 128;        // scale block (both operands)
constexpr int kTM = 64;         // rows per tile
constexpr int kTN = 128;        // columns per tile
constexpr int kThreads = 256;   // 4 waves x 32 columns
constexpr int kXcds = 8;
constexpr int kLoads = 4;       // 16-byte loads per operand row half per block

struct Fp8Tile {
  int expert;
  int64_t row0, row_end;
  bool valid;
};

// m-tile index -> expert and row range.  Lane j of each 64-expert chunk counts
// the 64-row tiles of expert c + j; a wave prefix sum finds the owner.  Row
// ranges are clamped into [0, n_rows], so no row outside the buffer is read
// whatever the offsets hold.
__device__ Fp8Tile find_fp8_tile(int m_idx, const int32_t* __restrict__ offs, int n_experts,
                                 int64_t n_rows) {
  Fp8Tile t{};
  t.valid = false;
  const int lane = lane_id();
  int base = 0;
  for (int c = 0; c < n_experts; c += kWave) {
    const int e = c + lane;
    int lo = 0, hi = 0, nt = 0;
    if (e < n_experts) {
      const int64_t a = offs[e], b = offs[e + 1];
      lo = int(a < 0 ? 0 : (a > n_rows ? n_rows : a));
      hi = int(b < lo ? lo : (b > n_rows ? n_rows : b));
      nt = (hi - lo + kTM - 1) / kTM;
    }
    int incl = nt;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    const int excl = incl - nt;
    const uint64_t own = ballot(nt > 0 && m_idx >= base + excl && m_idx < base + incl);
    if (own) {
      const int src = __ffsll((unsigned long long)own) - 1;
      const int lo_s = __shfl(lo, src), hi_s = __shfl(hi, src), ex_s = __shfl(excl, src);
      t.expert = c + src;
      t.row0 = lo_s + int64_t(m_idx - base - ex_s) * kTM;
      t.row_end = hi_s;
      t.valid = true;
      return t;
    }
    base += __shfl(incl, kWave - 1);
  }
  return t;
}

// 8-byte operand group g (0..7) of a lane's 64 bytes.
__device__ __forceinline__ long group8(const u32x4 (&v)[kLoads], int g) {
  const u32x4 q = v[g >> 1];
  const unsigned lo = (g & 1) ? q.z : q.x, hi = (g & 1) ? q.w : q.y;
  return long((unsigned long)lo | ((unsigned long)hi << 32));
}

struct Stage {
  u32x4 b[kLoads];    // weight column l % 32
  u32x4 a0[kLoads];   // row l % 32 of the tile
  u32x4 a1[kLoads];   // row 32 + l % 32
};

__device__ __forceinline__ void load_stage(Stage& s, const uint8_t* wb, const uint8_t* xa0,
                                           const uint8_t* xa1, int blk) {
  const int64_t o = int64_t(blk) * kQB;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    s.b[i] = *reinterpret_cast<const u32x4*>(wb + o + 16 * i);
    s.a0[i] = *reinterpret_cast<const u32x4*>(xa0 + o + 16 * i);
    s.a1[i] = *reinterpret_cast<const u32x4*>(xa1 + o + 16 * i);
  }
}

// acc += (sx * sw) * (the block's exact-order fp32 partial products)
__device__ __forceinline__ void block_step(f32x16& acc0, f32x16& acc1, const Stage& s,
                                           const float* __restrict__ sxt, int blk, float sw,
                                           int half) {
  f32x16 p0, p1;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    p0[v] = 0.f;
    p1[v] = 0.f;
  }
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const long bg = group8(s.b, g);
    p0 = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(group8(s.a0, g), bg, p0, 0, 0, 0);
    p1 = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(group8(s.a1, g), bg, p1, 0, 0, 0);
  }
  // lane holds rows 8*(v/4) + 4*half + v%4 of each 32-row half
  const float* col = sxt + blk * kTM + 4 * half;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 s0 = *reinterpret_cast<const float4*>(col + 8 * q);
    const float4 s1 = *reinterpret_cast<const float4*>(col + 32 + 8 * q);
    const float r0[4] = {s0.x, s0.y, s0.z, s0.w};
    const float r1[4] = {s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc0[4 * q + i] = __builtin_fmaf(r0[i] * sw, p0[4 * q + i], acc0[4 * q + i]);
      acc1[4 * q + i] = __builtin_fmaf(r1[i] * sw, p1[4 * q + i], acc1[4 * q + i]);
    }
  }
}

__global__ __launch_bounds__(kThreads) void grouped_gemm_fp8_kernel(
    const uint8_t* __restrict__ rows, const float* __restrict__ row_scales, int64_t n_rows,
    int K, const int32_t* __restrict__ offs, int n_experts, const uint8_t* __restrict__ w,
    const float* __restrict__ w_scales, int N, uint16_t* __restrict__ y, int max_m_tiles,
    int n_tiles) {
  // row scales of the tile, transposed: sxt[b * 64 + r]
  __shared__ __align__(16) float sxt[kMaxFp8Blocks * kTM];

  const int nb = gridDim.x;                 // a multiple of kXcds
  const int b = blockIdx.x;
  const int tile = (b % kXcds) * (nb / kXcds) + b / kXcds;
  if (int64_t(tile) >= int64_t(max_m_tiles) * n_tiles) return;
  const int m_idx = tile / n_tiles, n_tile = tile % n_tiles;
  const Fp8Tile ti = find_fp8_tile(m_idx, offs, n_experts, n_rows);
  if (!ti.valid) return;

  const int kb = K / kQB;
  for (int i = threadIdx.x; i < kb * kTM; i += kThreads) {
    const int r = i % kTM, blk = i / kTM;
    int64_t gr = ti.row0 + r;
    if (gr >= ti.row_end) gr = ti.row_end - 1;   // clamped rows are never stored
    sxt[blk * kTM + r] = row_scales[gr * kb + blk];
  }
  __syncthreads();

  const int lane = lane_id();
  const int w_id = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const int half = lane >> 5;
  const int64_t col = int64_t(n_tile) * kTN + w_id * 32 + (lane & 31);
  int64_t r0 = ti.row0 + (lane & 31), r1 = r0 + 32;
  if (r0 >= ti.row_end) r0 = ti.row_end - 1;
  if (r1 >= ti.row_end) r1 = ti.row_end - 1;
  const uint8_t* wb = w + (int64_t(ti.expert) * N + col) * K + half * 64;
  const uint8_t* xa0 = rows + r0 * K + half * 64;
  const uint8_t* xa1 = rows + r1 * K + half * 64;
  const float* swp = w_scales + (int64_t(ti.expert) * (N / kQB) + n_tile) * kb;

  f32x16 acc0, acc1;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    acc0[v] = 0.f;
    acc1[v] = 0.f;
  }
  Stage s0, s1;
  load_stage(s0, wb, xa0, xa1, 0);
  for (int blk = 0; blk < kb; blk += 2) {
    // past the last block the loads repeat it; the result is not used
    load_stage(s1, wb, xa0, xa1, min(blk + 1, kb - 1));
    block_step(acc0, acc1, s0, sxt, blk, swp[blk], half);
    load_stage(s0, wb, xa0, xa1, min(blk + 2, kb - 1));
    if (blk + 1 < kb) block_step(acc0, acc1, s1, sxt, blk + 1, swp[blk + 1], half);
  }

  // acc[v] = C[8*(v/4) + 4*half + v%4][lane % 32] of each 32-row half
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int rr = 8 * (v >> 2) + 4 * half + (v & 3);
    const int64_t g0 = ti.row0 + rr, g1 = g0 + 32;
    if (g0 < ti.row_end) y[g0 * N + col] = f32_to_bf16_rne(acc0[v]);
    if (g1 < ti.row_end) y[g1 * N + col] = f32_to_bf16_rne(acc1[v]);
  }
}

}  // namespace

hipError_t launch_grouped_gemm_fp8(const void* rows, const float* row_scales, int64_t n_rows,
                                   int64_t k_dim, const int32_t* expert_offsets, int n_experts,
                                   const void* w, const float* w_scales, int64_t n_dim, void* y,
                                   hipStream_t stream) {
  const int max_m_tiles = int((n_rows + kTM - 1) / kTM) + n_experts;
  const int n_tiles = int(n_dim / kTN);
  const int64_t tiles = int64_t(max_m_tiles) * n_tiles;
  const unsigned grid = unsigned((tiles + kXcds - 1) / kXcds * kXcds);
  grouped_gemm_fp8_kernel<<<grid, kThreads, 0, stream>>>(
      static_cast<const uint8_t*>(rows), row_scales, n_rows, int(k_dim), expert_offsets,
      n_experts, static_cast<const uint8_t*>(w), w_scales, int(n_dim),
      static_cast<uint16_t*>(y), max_m_tiles, n_tiles);
  return hipGetLastError();
}

}  // namespace moe
