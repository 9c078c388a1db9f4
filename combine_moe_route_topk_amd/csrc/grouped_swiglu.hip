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
// Tiles: 256 rows x 256 B-rows x 64 K per workgroup of 8 waves; each wave
// owns a 128 x 64 block as 4 x 2 v_mfma_f32_32x32x16_bf16 tiles with fp32
// accumulators (128 registers, so two waves fit per SIMD and hide each
// other's LDS and global latency).  Global -> LDS
// staging is double-buffered (128 KB of LDS); LDS rows are 128 bytes with
// their 16-byte chunks XOR-swizzled by ((row >> 1) & 7), so both the
// coalesced tile writes and the per-lane 16-byte operand reads are free of
// bank conflicts.
//
// Tile scheduling is device-side: the grid is sized for the worst case
// (ceil(R/256) + E row tiles per column tile) and each workgroup finds its
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

constexpr int kBM = 256;       // rows per tile
constexpr int kBN = 256;       // B rows per tile
constexpr int kBK = 64;        // K per stage
constexpr int kThreads = 512;  // 8 waves: 2 (rows) x 4 (B rows)
constexpr int kTileBytes = kBM * kBK * 2;       // 32 KB, same for the B tile
constexpr int kLoads = kBM * kBK * 2 / 16 / kThreads;   // 16-byte chunks per thread per tile (4)
constexpr int kTI = 4;         // 32-row MFMA tiles per wave (128 rows)
constexpr int kTJ = 2;         // 32-column MFMA tiles per wave (64 B rows)
constexpr int kXcds = 8;

// Byte offset of 16-byte chunk `chunk` of tile row `row`.  Rows are 128 bytes,
// so two consecutive rows span the 256-byte bank window; XOR-ing the chunk
// with (row >> 1) & 7 gives the 16 rows read by one 16-lane phase of a
// ds_read_b128 sixteen distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * (kBK * 2) + ((chunk ^ ((row >> 1) & 7)) << 4);
}

__device__ __forceinline__ float silu(float a) { return a / (1.f + expf(-a)); }

struct TileInfo {
  int expert;
  int64_t row0, row_end;
  int n_tile;
  bool valid;
};

// Linear tile id -> (expert, row range, column tile); row tiles run fastest,
// so the tiles one XCD runs together walk one weight tile across an expert's
// rows and reuse it from that XCD's L2.
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
  // LDS: A tiles for stages 0/1, then B tiles for stages 0/1 (128 KB)
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
  const int wm = w >> 2, wn = w & 3;

  // global -> LDS assignment: kLoads chunks of 16 bytes per thread per tile
  const uint16_t* a_src[kLoads];
  const uint16_t* b_src[kLoads];
  int l_off[kLoads];
#pragma unroll
  for (int s = 0; s < kLoads; ++s) {
    const int i = tid + s * kThreads;
    const int row = i >> 3, c = i & 7;
    int64_t gr = ti.row0 + row;
    if (gr >= ti.row_end) gr = ti.row_end - 1;            // clamped rows are never stored
    a_src[s] = A + gr * K + c * 8;
    const uint16_t* bp;
    if (MODE == 0) {
      int64_t f = int64_t(ti.n_tile) * (kBN / 2) + (row & (kBN / 2 - 1));
      if (f >= NB) f = NB - 1;                              // partial last column tile
      bp = (row < kBN / 2 ? B0 : B1) + (int64_t(ti.expert) * NB + f) * K;
    } else {
      int64_t n = int64_t(ti.n_tile) * kBN + row;
      if (n >= NB) n = NB - 1;                              // partial last column tile
      bp = B0 + (int64_t(ti.expert) * NB + n) * K;
    }
    b_src[s] = bp + c * 8;
    l_off[s] = swz(row, c);
  }

  u32x4 ra[kLoads], rb[kLoads];

  // operand rows of this lane: wave (wm, wn) owns rows wm*128.. and B rows
  //   gate/up: gate wn*32 (j = 0) and up kBN/2 + wn*32 (j = 1): one F column block
  //   down:    wn*64 + 32j
  const int a_row0 = wm * (kTI * 32) + (lane & 31);
  int b_row[kTJ];
#pragma unroll
  for (int j = 0; j < kTJ; ++j) {
    if (MODE == 0)
      b_row[j] = j * (kBN / 2) + wn * 32 + (lane & 31);
    else
      b_row[j] = wn * (kTJ * 32) + 32 * j + (lane & 31);
  }
  const int khalf = lane >> 5;

  f32x16 acc[kTI][kTJ];
#pragma unroll
  for (int i = 0; i < kTI; ++i)
#pragma unroll
    for (int j = 0; j < kTJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int kt_n = K / kBK;
#pragma unroll
  for (int s = 0; s < kLoads; ++s) {
    ra[s] = *reinterpret_cast<const u32x4*>(a_src[s]);
    rb[s] = *reinterpret_cast<const u32x4*>(b_src[s]);
  }
#pragma unroll
  for (int s = 0; s < kLoads; ++s) {
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
      for (int s = 0; s < kLoads; ++s) {
        ra[s] = *reinterpret_cast<const u32x4*>(a_src[s] + k0);
        rb[s] = *reinterpret_cast<const u32x4*>(b_src[s] + k0);
      }
    }
    const unsigned char* tA = smem + buf * kTileBytes;
    const unsigned char* tB = smem + (2 + buf) * kTileBytes;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int chunk = kk * 2 + khalf;
      bf16x8 av[kTI], bv[kTJ];
#pragma unroll
      for (int i = 0; i < kTI; ++i)
        av[i] = *reinterpret_cast<const bf16x8*>(tA + swz(a_row0 + 32 * i, chunk));
#pragma unroll
      for (int j = 0; j < kTJ; ++j)
        bv[j] = *reinterpret_cast<const bf16x8*>(tB + swz(b_row[j], chunk));
#pragma unroll
      for (int i = 0; i < kTI; ++i)
#pragma unroll
        for (int j = 0; j < kTJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
#pragma unroll
      for (int s = 0; s < kLoads; ++s) {
        *reinterpret_cast<u32x4*>(smem + (buf ^ 1) * kTileBytes + l_off[s]) = ra[s];
        *reinterpret_cast<u32x4*>(smem + (2 + (buf ^ 1)) * kTileBytes + l_off[s]) = rb[s];
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds C[8*(v/4) + 4*(lane/32) + v%4][lane%32] of each 32x32 tile
#pragma unroll
  for (int i = 0; i < kTI; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * (kTI * 32) + 32 * i + 8 * (v >> 2) + 4 * khalf + (v & 3);
      const int64_t gr = ti.row0 + r;
      if (gr >= ti.row_end) continue;
      if (MODE == 0) {
        const int64_t col = int64_t(ti.n_tile) * (kBN / 2) + wn * 32 + (lane & 31);
        const float h = silu(acc[i][0][v]) * acc[i][1][v];
        if (col < NB) C[gr * ldc + col] = f32_to_bf16_rne(h);
      } else {
#pragma unroll
        for (int j = 0; j < kTJ; ++j) {
          const int64_t col = int64_t(ti.n_tile) * kBN + wn * (kTJ * 32) + 32 * j + (lane & 31);
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
  // gate/up: F/(kBN/2) column tiles (kBN/2 gate + kBN/2 up rows per B tile), K = D
  const int nct1 = int((ffn + kBN / 2 - 1) / (kBN / 2));
  grouped_gemm_kernel<0><<<grid_for(nct1), kThreads, 0, stream>>>(
      static_cast<const uint16_t*>(rows), n_rows, int(hidden), expert_offsets, n_experts,
      static_cast<const uint16_t*>(w_gate), static_cast<const uint16_t*>(w_up), int(ffn), h,
      int(ffn), max_m_tiles, nct1);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // down: ceil(D/kBN) column tiles, K = F
  const int nct2 = int((hidden + kBN - 1) / kBN);
  grouped_gemm_kernel<1><<<grid_for(nct2), kThreads, 0, stream>>>(
      h, n_rows, int(ffn), expert_offsets, n_experts, static_cast<const uint16_t*>(w_down),
      nullptr, int(hidden), static_cast<uint16_t*>(y), int(hidden), max_m_tiles, nct2);
  return hipGetLastError();
}

}  // namespace moe
