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
//             one B tile (128 gate rows + 128 up rows of the same F columns), so
//             a lane holds gate and up of the same output element and the
//             epilogue h = bf16(silu(g) * u) is lane-local;  h -> workspace;
//   down:     A = h [R, F], B = W_down[e] [D, F];  y = bf16(A B^T).
// Tiles: 256 rows x 256 B-rows per workgroup of 8 waves; each wave owns a
// 128 x 64 block as 4 x 2 v_mfma_f32_32x32x16_bf16 tiles with fp32
// accumulators, two waves per SIMD.
//
// Operands reach LDS through direct global->LDS loads (global_load_lds_dwordx4:
// no staging registers, no LDS write instructions).  K advances in stages of
// 32; a ring of four stages (4 x 32 KB) keeps the loads of stage kt+3 in flight
// while stage kt is multiplied, and one barrier per stage both publishes stage
// kt+1 and retires every read of the array that stage kt+3 overwrites.  Stage
// kt+1's first fragments are read before that barrier, so the MFMAs resume at
// once after it.  LDS rows are 64 bytes with their 16-byte chunks XOR-swizzled
// by ((row >> 2) & 3): the 16 rows one 16-lane phase of a ds_read_b128 reads
// land in 16 distinct 16-byte bank groups; the direct loads write whole
// 1 KB runs, so the swizzle sits in the global addresses they read.
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

constexpr int kBM = 256;       // rows per tile
constexpr int kBN = 256;       // B rows per tile
constexpr int kBK = 32;        // K per stage
constexpr int kStages = 4;     // LDS ring depth
constexpr int kThreads = 512;  // 8 waves: 2 (rows) x 4 (B rows)
constexpr int kRowBytes = kBK * 2;              // 64-byte LDS rows
constexpr int kTileBytes = kBM * kRowBytes;     // 16 KB per operand per stage
constexpr int kStageBytes = 2 * kTileBytes;     // A tile then B tile
constexpr int kDmaPerOperand = kTileBytes / (kThreads * 16);   // 1 KB runs per wave (2)
constexpr int kTI = 4;         // 32-row MFMA tiles per wave (128 rows)
constexpr int kTJ = 2;         // 32-column MFMA tiles per wave (64 B rows)
constexpr int kXcds = 8;

// Byte offset of 16-byte chunk `chunk` (0..3) of tile row `row`.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ ((row >> 2) & 3)) << 4);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8): wait until at most n vector-memory operations of this
// wave are outstanding, and (lgkm0) all of its LDS operations have returned.
constexpr unsigned wait_vm_lgkm0(int n) {
  return unsigned(n & 15) | (unsigned((n >> 4) & 3) << 14) | (0x7u << 4);
}
constexpr unsigned wait_vm(int n) {
  return unsigned(n & 15) | (unsigned((n >> 4) & 3) << 14) | (0x7u << 4) | (0xFu << 8);
}

typedef __attribute__((address_space(3))) void* lds_ptr;

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

struct Operands {
  const uint16_t* a_src[kDmaPerOperand];   // this lane's global source of each 1 KB run
  const uint16_t* b_src[kDmaPerOperand];
  int lds_off[kDmaPerOperand];             // wave-uniform LDS offset of each run
  int a_row0;                              // first A row of this lane's fragments
  int b_row[kTJ];                          // B row of this lane's fragment j
  int khalf;                               // which 8-element half of a 16-wide K slice
};

struct Frag {
  bf16x8 a[kTI];
  bf16x8 b[kTJ];
};

// Direct global->LDS loads of K stage `k0` (elements) into one ring slot.
__device__ __forceinline__ void load_stage(unsigned char* st, const Operands& op, int k0) {
#pragma unroll
  for (int s = 0; s < kDmaPerOperand; ++s) {
    __builtin_amdgcn_global_load_lds(op.a_src[s] + k0, (lds_ptr)(st + op.lds_off[s]), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(op.b_src[s] + k0, (lds_ptr)(st + kTileBytes + op.lds_off[s]),
                                     16, 0, 0);
  }
}

// Operand fragments of 16-wide K slice `kk` (0 or 1) of one ring slot.
__device__ __forceinline__ void read_frag(const unsigned char* st, const Operands& op, int kk,
                                          Frag& f) {
  const int chunk = kk * 2 + op.khalf;
#pragma unroll
  for (int i = 0; i < kTI; ++i)
    f.a[i] = *reinterpret_cast<const bf16x8*>(st + swz(op.a_row0 + 32 * i, chunk));
#pragma unroll
  for (int j = 0; j < kTJ; ++j)
    f.b[j] = *reinterpret_cast<const bf16x8*>(st + kTileBytes + swz(op.b_row[j], chunk));
}

__device__ __forceinline__ void mma(f32x16 (&acc)[kTI][kTJ], const Frag& f) {
#pragma unroll
  for (int i = 0; i < kTI; ++i)
#pragma unroll
    for (int j = 0; j < kTJ; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Barrier that publishes the direct loads each wave has waited for; the empty
// asm statements keep the compiler from moving LDS accesses across it.
template <unsigned kWait>
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(kWait);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One K stage.  On entry f0 holds slice 0 of stage kt (slot `cur`), stage
// kt+1 (slot `nxt`) may still be loading, stage kt+2 is loading.  The barrier
// waits for stage kt+1 (each wave leaves only stage kt+2's loads in flight)
// and for every LDS read of the slot that stage kt+3 (`dst`) overwrites.
__device__ __forceinline__ void stage_step(f32x16 (&acc)[kTI][kTJ], Frag& f0, Frag& f1,
                                           const unsigned char* cur, const unsigned char* nxt,
                                           unsigned char* dst, const Operands& op, int kt,
                                           int kt_n) {
  stage_barrier<wait_vm_lgkm0(2 * kDmaPerOperand)>();
  // past the last stage the loads repeat the last stage into a slot nobody reads
  load_stage(dst, op, min(kt + 3, kt_n - 1) * kBK);
  read_frag(cur, op, 1, f1);
  mma(acc, f0);
  read_frag(nxt, op, 0, f0);
  mma(acc, f1);
  // issue order: one MFMA per fragment read, the direct loads mid-stage
#pragma unroll
  for (int q = 0; q < kTI + kTJ; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x020, 2 * kDmaPerOperand, 0);   // direct loads
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
  for (int q = 0; q < kTI + kTJ; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}

template <int MODE>   // 0: gate/up with SwiGLU epilogue, 1: down projection
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(
    const uint16_t* __restrict__ A, int64_t n_rows, int K, const int32_t* __restrict__ offs,
    int n_experts, const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, int NB,
    uint16_t* __restrict__ C, int ldc, int max_m_tiles, int n_col_tiles) {
  // the four ring slots are distinct arrays, so the compiler can tell a slot
  // being loaded from the slot being read and adds no wait between them
  __shared__ __align__(1024) unsigned char slot0[kStageBytes];
  __shared__ __align__(1024) unsigned char slot1[kStageBytes];
  __shared__ __align__(1024) unsigned char slot2[kStageBytes];
  __shared__ __align__(1024) unsigned char slot3[kStageBytes];

  // XCD-aware placement: workgroup b runs on XCD b % 8; give each XCD a
  // contiguous range of tile ids.
  const int nb = gridDim.x;                // a multiple of kXcds
  const int b = blockIdx.x;
  const int tile = (b % kXcds) * (nb / kXcds) + b / kXcds;
  const TileInfo ti = find_tile(tile, max_m_tiles, n_col_tiles, offs, n_experts, n_rows);
  if (!ti.valid) return;

  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const int wm = w >> 2, wn = w & 3;

  // Direct-load assignment: run s of wave w fills LDS bytes
  // [(s * 8 + w) KB, +1 KB) of each operand tile, i.e. 16 rows of 64 bytes;
  // lane l writes the 16 bytes at l * 16, which hold logical chunk
  // pc ^ ((row >> 2) & 3) of its row.
  Operands op;
#pragma unroll
  for (int s = 0; s < kDmaPerOperand; ++s) {
    op.lds_off[s] = (s * (kThreads / kWave) + w) * 1024;
    const int p = op.lds_off[s] + lane * 16;
    const int row = p / kRowBytes, pc = (p % kRowBytes) / 16;
    const int c = pc ^ ((row >> 2) & 3);
    int64_t gr = ti.row0 + row;
    if (gr >= ti.row_end) gr = ti.row_end - 1;            // clamped rows are never stored
    op.a_src[s] = A + gr * K + c * 8;
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
    op.b_src[s] = bp + c * 8;
  }

  // operand rows of this lane: wave (wm, wn) owns rows wm*128.. and B rows
  //   gate/up: gate wn*32 (j = 0) and up kBN/2 + wn*32 (j = 1): one F column block
  //   down:    wn*64 + 32j
  op.a_row0 = wm * (kTI * 32) + (lane & 31);
#pragma unroll
  for (int j = 0; j < kTJ; ++j) {
    if (MODE == 0)
      op.b_row[j] = j * (kBN / 2) + wn * 32 + (lane & 31);
    else
      op.b_row[j] = wn * (kTJ * 32) + 32 * j + (lane & 31);
  }
  op.khalf = lane >> 5;

  f32x16 acc[kTI][kTJ];
#pragma unroll
  for (int i = 0; i < kTI; ++i)
#pragma unroll
    for (int j = 0; j < kTJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int kt_n = K / kBK;                // K % 64 == 0: an even number of stages
  Frag f0, f1;
  load_stage(slot0, op, 0);
  load_stage(slot1, op, min(1, kt_n - 1) * kBK);
  load_stage(slot2, op, min(2, kt_n - 1) * kBK);
  stage_barrier<wait_vm_lgkm0(2 * 2 * kDmaPerOperand)>();   // stage 0 landed
  read_frag(slot0, op, 0, f0);
  const int kq = kt_n & ~(kStages - 1);
  for (int kt = 0; kt < kq; kt += kStages) {
    stage_step(acc, f0, f1, slot0, slot1, slot3, op, kt, kt_n);
    stage_step(acc, f0, f1, slot1, slot2, slot0, op, kt + 1, kt_n);
    stage_step(acc, f0, f1, slot2, slot3, slot1, op, kt + 2, kt_n);
    stage_step(acc, f0, f1, slot3, slot0, slot2, op, kt + 3, kt_n);
  }
  if (kq < kt_n) {                         // two trailing stages
    stage_step(acc, f0, f1, slot0, slot1, slot3, op, kq, kt_n);
    stage_step(acc, f0, f1, slot1, slot2, slot0, op, kq + 1, kt_n);
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(0));  // no direct load may outlive the workgroup

  // epilogue: lane holds C[8*(v/4) + 4*(lane/32) + v%4][lane%32] of each 32x32 tile
  const int khalf = op.khalf;
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
