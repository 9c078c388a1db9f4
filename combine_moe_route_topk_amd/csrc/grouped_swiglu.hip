// Grouped SwiGLU expert FFN on the matrix cores, reading the dispatched rows
// in place.
//
// "One-Sided Expert-Parallel All-to-All for Mixture-of-Experts Inference over
// NVLink" (abstract): the grouped GEMMs read the dispatched buffers in place
// instead of from a per-expert copy.  "backends/mlx: runtime MoE expert-sort
// for decode (issue #20554)": the sorted flag of gather_mm is the caller's
// promise that rows arrive grouped by expert (here: expert e owns rows
// [expert_offsets[e], expert_offsets[e+1])), and expert weights are laid out
// [E, out, in].
//
// Two launches of one kernel template, both C = A * B^T with A and B
// K-contiguous (the friendly layout for the matrix cores):
//   gate/up:  A = rows [R, D], B = W_gate[e] and W_up[e] [F, D] interleaved in
//             one B tile (64 gate rows + 64 up rows of the same F columns), so
//             a lane holds gate and up of the same output element and the
//             epilogue h = bf16(silu(g) * u) is lane-local;  h -> workspace;
//   down:     A = h [R, F], B = W_down[e] [D, F];  y = bf16(A B^T).
// Tiles: 128 rows x 128 B-rows x 64 K per workgroup of 4 waves; each wave
// owns a 64 x 64 block as 2 x 2 v_mfma_f32_32x32x16_bf16 tiles with fp32
// accumulators.  Global -> LDS staging is double-buffered; LDS rows are 128
// bytes with their 16-byte chunks XOR-swizzled by (row & 7), so both the
// coalesced tile writes and the per-lane 16-byte operand reads are free of
// bank conflicts.
//
// Tile scheduling is device-side: the grid is sized for the worst case
// (ceil(R/128) + E row tiles per column tile) and each workgroup finds its
// expert and row range from expert_offsets; workgroups past the last real
// tile exit.  Consecutive tile ids (same column tile, successive row tiles of
// one expert, so the same weight tile) are placed on one XCD so that the
// weight tile is reused from that XCD's L2.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;       // rows per tile
constexpr int kBN = 128;       // B rows per tile
constexpr int kBK = 64;        // K per stage
constexpr int kThreads = 256;
constexpr int kTileBytes = kBM * kBK * 2;       // 16 KB, same for the B tile
constexpr int kXcds = 8;

__device__ __forceinline__ int swz(int row, int chunk) {   // byte offset in a tile
  return row * (kBK * 2) + ((chunk ^ (row & 7)) << 4);
}

__device__ __forceinline__ float silu(float a) { return a / (1.f + expf(-a)); }

struct TileInfo {
  int expert;
  int64_t row0, row_end;
  int n_tile;
  bool valid;
};

// Linear tile id -> (expert, row range, column tile); m tiles run fastest.
__device__ TileInfo find_tile(int tile, int max_m_tiles, int n_col_tiles,
                              const int32_t* __restrict__ offs, int n_experts, int64_t n_rows) {
  TileInfo ti{};
  ti.valid = false;
  if (tile >= max_m_tiles * n_col_tiles) return ti;
  const int m_idx = tile % max_m_tiles;
  ti.n_tile = tile / max_m_tiles;
  // offsets are clamped into [0, n_rows] and made non-decreasing, so no row
  // outside the buffer is ever touched whatever the caller passed
  int cum = 0;
  int64_t lo = offs[0] < 0 ? 0 : (offs[0] > n_rows ? n_rows : offs[0]);
  for (int e = 0; e < n_experts; ++e) {
    int64_t hi = offs[e + 1];
    hi = hi < lo ? lo : (hi > n_rows ? n_rows : hi);
    const int nt = int((hi - lo + kBM - 1) / kBM);
    if (m_idx < cum + nt) {
      ti.expert = e;
      ti.row0 = lo + int64_t(m_idx - cum) * kBM;
      ti.row_end = hi;
      ti.valid = true;
      return ti;
    }
    cum += nt;
    lo = hi;
  }
  return ti;
}

template <int MODE>   // 0: gate/up with SwiGLU epilogue, 1: down projection
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(
    const uint16_t* __restrict__ A, int64_t n_rows, int K, const int32_t* __restrict__ offs,
    int n_experts, const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, int NB,
    uint16_t* __restrict__ C, int ldc, int max_m_tiles, int n_col_tiles) {
  // LDS: A tiles for stages 0/1, then B tiles for stages 0/1
  __shared__ __align__(16) unsigned char smem[4 * kTileBytes];

  // XCD-aware placement: workgroup b runs on XCD b % 8; give each XCD a
  // contiguous range of tile ids.
  const int nb = gridDim.x;                // a multiple of kXcds
  const int b = blockIdx.x;
  const int tile = (b % kXcds) * (nb / kXcds) + b / kXcds;
  const TileInfo ti = find_tile(tile, max_m_tiles, n_col_tiles, offs, n_experts, n_rows);
  if (!ti.valid) return;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid / kWave;
  const int wm = w >> 1, wn = w & 1;

  // global -> LDS assignment: 4 chunks of 16 bytes per thread per tile
  const uint16_t* a_src[4];
  const uint16_t* b_src[4];
  int l_off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int i = tid + s * kThreads;
    const int row = i >> 3, c = i & 7;
    int64_t gr = ti.row0 + row;
    if (gr >= ti.row_end) gr = ti.row_end - 1;            // clamped rows are never stored
    a_src[s] = A + gr * K + c * 8;
    const uint16_t* bp;
    if (MODE == 0) {
      const int64_t f = int64_t(ti.n_tile) * (kBN / 2) + (row & (kBN / 2 - 1));
      bp = (row < kBN / 2 ? B0 : B1) + (int64_t(ti.expert) * NB + f) * K;
    } else {
      int64_t n = int64_t(ti.n_tile) * kBN + row;
      if (n >= NB) n = NB - 1;                              // partial last column tile
      bp = B0 + (int64_t(ti.expert) * NB + n) * K;
    }
    b_src[s] = bp + c * 8;
    l_off[s] = swz(row, c);
  }

  u32x4 ra[4], rb[4];

  // operand rows of this lane
  const int a_row0 = wm * 64 + (lane & 31);
  int b_row[2];
  if (MODE == 0) {
    b_row[0] = wn * 32 + (lane & 31);                 // gate
    b_row[1] = kBN / 2 + wn * 32 + (lane & 31);       // up, same F column
  } else {
    b_row[0] = wn * 64 + (lane & 31);
    b_row[1] = wn * 64 + 32 + (lane & 31);
  }
  const int khalf = lane >> 5;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int kt_n = K / kBK;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    ra[s] = *reinterpret_cast<const u32x4*>(a_src[s]);
    rb[s] = *reinterpret_cast<const u32x4*>(b_src[s]);
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    *reinterpret_cast<u32x4*>(smem + l_off[s]) = ra[s];
    *reinterpret_cast<u32x4*>(smem + 2 * kTileBytes + l_off[s]) = rb[s];
  }
  __syncthreads();
  for (int kt = 0; kt < kt_n; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < kt_n;
    if (more) {
      const int k0 = (kt + 1) * kBK;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        ra[s] = *reinterpret_cast<const u32x4*>(a_src[s] + k0);
        rb[s] = *reinterpret_cast<const u32x4*>(b_src[s] + k0);
      }
    }
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int chunk = kk * 2 + khalf;
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        av[i] = *reinterpret_cast<const bf16x8*>(smem + buf * kTileBytes + swz(a_row0 + 32 * i, chunk));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bv[j] = *reinterpret_cast<const bf16x8*>(smem + (2 + buf) * kTileBytes + swz(b_row[j], chunk));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        *reinterpret_cast<u32x4*>(smem + (buf ^ 1) * kTileBytes + l_off[s]) = ra[s];
        *reinterpret_cast<u32x4*>(smem + (2 + (buf ^ 1)) * kTileBytes + l_off[s]) = rb[s];
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds C[8*(v/4) + 4*(lane/32) + v%4][lane%32] of each 32x32 tile
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * 64 + 32 * i + 8 * (v >> 2) + 4 * khalf + (v & 3);
      const int64_t gr = ti.row0 + r;
      if (gr >= ti.row_end) continue;
      if (MODE == 0) {
        const int64_t col = int64_t(ti.n_tile) * (kBN / 2) + wn * 32 + (lane & 31);
        const float h = silu(acc[i][0][v]) * acc[i][1][v];
        C[gr * ldc + col] = f32_to_bf16_rne(h);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t col = int64_t(ti.n_tile) * kBN + wn * 64 + 32 * j + (lane & 31);
          if (col < NB) C[gr * ldc + col] = f32_to_bf16_rne(acc[i][j][v]);
        }
      }
    }
  }
}

}  // namespace

size_t grouped_swiglu_workspace_bytes(int64_t n_rows, int n_experts, int64_t hidden, int64_t ffn) {
  (void)n_experts;
  (void)hidden;
  return size_t(n_rows) * size_t(ffn) * 2 + 256;
}

hipError_t launch_grouped_swiglu(const void* rows, int64_t n_rows, int64_t hidden,
                                 const int32_t* expert_offsets, int n_experts, const void* w_gate,
                                 const void* w_up, const void* w_down, int64_t ffn, void* y,
                                 void* workspace, hipStream_t stream) {
  const int max_m_tiles = int((n_rows + kBM - 1) / kBM) + n_experts;
  uint16_t* h = static_cast<uint16_t*>(workspace);
  auto grid_for = [&](int n_col_tiles) {
    const int64_t tiles = int64_t(max_m_tiles) * n_col_tiles;
    return unsigned((tiles + kXcds - 1) / kXcds * kXcds);
  };
  // gate/up: F/64 column tiles (64 gate + 64 up rows per B tile), K = D
  const int nct1 = int(ffn / (kBN / 2));
  grouped_gemm_kernel<0><<<grid_for(nct1), kThreads, 0, stream>>>(
      static_cast<const uint16_t*>(rows), n_rows, int(hidden), expert_offsets, n_experts,
      static_cast<const uint16_t*>(w_gate), static_cast<const uint16_t*>(w_up), int(ffn), h,
      int(ffn), max_m_tiles, nct1);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // down: ceil(D/128) column tiles, K = F
  const int nct2 = int((hidden + kBN - 1) / kBN);
  grouped_gemm_kernel<1><<<grid_for(nct2), kThreads, 0, stream>>>(
      h, n_rows, int(ffn), expert_offsets, n_experts, static_cast<const uint16_t*>(w_down),
      nullptr, int(hidden), static_cast<uint16_t*>(y), int(hidden), max_m_tiles, nct2);
  return hipGetLastError();
}

}  // namespace moe
