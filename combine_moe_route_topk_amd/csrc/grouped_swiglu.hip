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
//   gate/up:  A = rows [R, D], B = W_gate[e] and W_up[e] [F, D] in one B tile
//             (128 gate rows + 128 up rows of the same F columns); a lane holds
//             gate and up of the same output element, so the epilogue
//             h = bf16(silu(g) * u) is lane-local;  h -> workspace;
//   down:     A = h [R, F], B = W_down[e] [D, F];  y = bf16(A B^T).
//
// Tiles: 256 rows x 256 B-rows per workgroup of 4 waves (2 x 2); each wave owns
// a 128 x 128 block as 4 x 4 v_mfma_f32_32x32x16_bf16 tiles whose 256 fp32
// accumulators per lane live in the accumulation registers, one wave per SIMD.
//
// Operands: K advances in stages of 64, so each row of a stage is one whole
// 128-byte line.  Direct global->LDS loads (global_load_lds_dwordx4, no staging
// registers) fill two 64 KB LDS slots; stage d is multiplied from slot d % 2
// while stage d+1 lands in the other.  One barrier per stage, after the
// fragment reads of the stage's last 16-wide slice, both publishes stage d+1 and
// frees slot d % 2, so the loads of stage d+2 go out right after it.  Those 16
// loads per lane are spread over the next 32 MFMAs (half over the slice that
// follows the barrier, half over the next stage's first slice) instead of being
// issued in one burst: measured on MI355X this cut the mean L2 request latency
// and made the kernel 4-11% faster (depending on the data) than with the loads
// in one group.
// LDS rows are 128 bytes with their 16-byte chunks XOR-swizzled by
// ((row >> 1) & 7), so the 16 rows one 16-lane phase of a ds_read_b128 reads
// fall in distinct bank groups; the direct loads write whole 1 KB runs, so the
// swizzle sits in the global addresses they read.
//
// Tile scheduling is device-side: the grid is sized for the worst case
// (ceil(R/256) + E row tiles per column tile); each workgroup counts the real
// row tiles from expert_offsets and takes tile t of a grouped order: XCD x
// (workgroup b runs on XCD b % 8) owns a contiguous range of t, and within it
// 8 row tiles x all column tiles, row tiles fastest, so the 32 workgroups an
// XCD runs together share 8 row tiles and 4 weight tiles through its L2.
// Workgroups past the last unit exit.
//
// The last round: tiles that do not fill a whole round of workgroups (one per
// CU) are split into K parts (an even number of stages each, at most 8 parts)
// so that round keeps every CU busy.  Each part stores its fp32 partial tile in
// the workspace and counts itself on the tile's counter (zeroed by a small
// kernel at the start of every call); the part that arrives last sums the
// partials in part order, so the result does not depend on which part that
// was, and writes the tile.  Nothing waits on another workgroup.
#include <atomic>

#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;       // rows per tile
constexpr int kBN = 256;       // B rows per tile
constexpr int kBK = 64;        // K per stage
constexpr int kThreads = 256;  // 4 waves: 2 (rows) x 2 (B rows)
constexpr int kRowBytes = kBK * 2;                        // 128-byte LDS rows
constexpr int kTileBytes = kBM * kRowBytes;               // 32 KB per operand per stage
constexpr int kSlotBytes = 2 * kTileBytes;                // A tile then B tile
constexpr int kLd = kTileBytes / (kThreads * 16);         // 1 KB runs per lane per operand (8)
constexpr int kTI = 4;         // 32-row MFMA tiles per wave (128 rows)
constexpr int kTJ = 4;         // 32-column MFMA tiles per wave (128 B rows)
constexpr int kGroupM = 8;     // row tiles per group of the tile order
constexpr int kXcds = 8;
constexpr int kCuMax = 256;    // workgroups of the last round at most (one per CU)
constexpr int kMaxSplit = 8;   // K parts of a last-round tile at most
constexpr int kTileElems = kBM * kBN;   // fp32 partial of one tile

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8).
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

// Expert e owns rows [lo_e, hi_e): lo_0 = clamp(offs[0], 0, R), hi_e =
// clamp(offs[e+1], lo_e, R), lo_{e+1} = hi_e.  Offsets are thereby clamped into
// [0, R] and made non-decreasing, so no row outside the buffer is ever touched
// whatever the caller passed.

// Real row tile m (row tiles of expert 0 first) -> expert and row range.
__device__ TileInfo find_row_tile(int m, const int32_t* __restrict__ offs, int n_experts,
                                  int64_t n_rows) {
  TileInfo ti{};
  ti.valid = false;
  int cum = 0;
  int64_t lo = offs[0] < 0 ? 0 : (offs[0] > n_rows ? n_rows : offs[0]);
  for (int e = 0; e < n_experts; ++e) {
    int64_t hi = offs[e + 1];
    hi = hi < lo ? lo : (hi > n_rows ? n_rows : hi);
    const int nt = int((hi - lo + kBM - 1) / kBM);
    if (m < cum + nt) {
      ti.expert = e;
      ti.row0 = lo + int64_t(m - cum) * kBM;
      ti.row_end = hi;
      ti.valid = true;
      return ti;
    }
    cum += nt;
    lo = hi;
  }
  return ti;
}

// Number of real row tiles under the same ranges, 64 experts at a time: hi_e =
// min(R, max(lo_0, offs[1..e+1])) is a running maximum, so each chunk takes an
// inclusive max-scan across the wave (DPP row operations; the clamp into
// [lo_0, R] commutes with the running maximum, so it is applied first).
__device__ int count_row_tiles(const int32_t* __restrict__ offs, int n_experts, int64_t n_rows) {
  const int lane = lane_id();
  const int R = int(n_rows);                  // NK <= INT32_MAX rows
  int carry = offs[0] < 0 ? 0 : (offs[0] > R ? R : offs[0]);
  int total = 0;
  for (int c = 0; c < n_experts; c += kWave) {
    const int e = c + lane;
    int v = e < n_experts ? offs[e + 1] : carry;
    v = v > R ? R : v;
    v = v < carry ? carry : v;
    const int hi = wave_inclusive_max_nonneg(v);
    const int lo = wave_shift_up1(hi, carry);
    const int nt = e < n_experts ? (hi - lo + kBM - 1) / kBM : 0;
    total += lane_value(wave_inclusive_scan(nt), kWave - 1);
    carry = lane_value(hi, kWave - 1);
  }
  return __builtin_amdgcn_readfirstlane(total);
}

// Tile t of the grouped order (t < tiles): 8 row tiles x all column tiles,
// row tiles fastest.
__device__ TileInfo grouped_tile(int t, int m_real, int n_col_tiles,
                                 const int32_t* __restrict__ offs, int n_experts, int64_t n_rows) {
  const int g = t / (kGroupM * n_col_tiles);
  const int m0 = g * kGroupM;
  const int gm = m_real - m0 < kGroupM ? m_real - m0 : kGroupM;
  const int i = t - g * kGroupM * n_col_tiles;
  TileInfo ti = find_row_tile(m0 + i % gm, offs, n_experts, n_rows);
  ti.n_tile = i / gm;
  return ti;
}

// The work of one launch: `full` tiles fill whole rounds of n_cus workgroups;
// the `tail` tiles of the last, partial round are each split into `split` K
// parts so that round keeps every CU busy.  Part results are fp32 partial
// tiles in the workspace; the last part of a tile to finish (an atomic
// counter per tile) sums them in part order and writes the tile.
struct Unit {
  TileInfo ti;
  int part, n_parts;    // K part of the tile and the tile's number of parts
  int tail;             // index of the tile among the split ones (n_parts > 1)
  int unit;             // index of the part among all split parts
};

// Workgroup b (on XCD b % 8) -> unit.  Full tiles come first in dispatch
// order: XCD x takes a contiguous range of them; then the parts of the split
// tiles, round-robin over the XCDs.
__device__ Unit find_unit(int b, int n_col_tiles, int kt_n, int n_cus,
                          const int32_t* __restrict__ offs, int n_experts, int64_t n_rows) {
  Unit u{};
  u.ti.valid = false;
  const int m_real = count_row_tiles(offs, n_experts, n_rows);
  const int tiles = m_real * n_col_tiles;
  const int full = tiles / n_cus * n_cus;      // n_cus is a multiple of kXcds
  const int tail = tiles - full;
  int split = 1;
  if (tail > 0 && kt_n % 2 == 0) {
    split = n_cus / tail;
    split = split < kMaxSplit ? split : kMaxSplit;
    split = split < kt_n / 2 ? split : kt_n / 2;
    split = split > 1 ? split : 1;
  }
  const int j = b / kXcds, x = b % kXcds;
  const int full_per_xcd = full / kXcds;
  if (j < full_per_xcd) {
    u.ti = grouped_tile(x * full_per_xcd + j, m_real, n_col_tiles, offs, n_experts, n_rows);
    u.part = 0;
    u.n_parts = 1;
    return u;
  }
  const int v = (j - full_per_xcd) * kXcds + x;
  if (v >= tail * split) return u;
  u.tail = v / split;
  u.part = v % split;
  u.n_parts = split;
  u.unit = v;
  u.ti = grouped_tile(full + u.tail, m_real, n_col_tiles, offs, n_experts, n_rows);
  return u;
}

// Global sources of this lane's direct loads.  Run r = i*4 + w of an operand
// tile holds tile rows r*8 .. r*8+7: lane l fills row r*8 + l/8 at LDS chunk
// position l%8 and so reads global chunk (l%8) ^ ((row >> 1) & 7).
struct Src {
  const unsigned char* a_base;            // the tile's first A row
  const unsigned char* b_base[kLd];       // per run: gate or up rows (gate/up), B rows (down)
  int a_off[kLd], b_off[kLd];             // per-lane byte offsets from those bases
  int lds_run[kLd];                       // LDS byte offset of run i within an operand tile
};

// Direct loads [LO, HI) of one stage (0..7: A runs, 8..15: B runs).
template <int LO, int HI>
__device__ __forceinline__ void load_runs(unsigned char* slot, const Src& src, int kbyte) {
#pragma unroll
  for (int i = LO; i < HI; ++i) {
    if (i < kLd)
      __builtin_amdgcn_global_load_lds(src.a_base + kbyte + src.a_off[i],
                                       (lds_ptr)(slot + src.lds_run[i]), 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(src.b_base[i - kLd] + kbyte + src.b_off[i - kLd],
                                       (lds_ptr)(slot + kTileBytes + src.lds_run[i - kLd]), 16,
                                       0, 0);
  }
}

struct Frag {
  bf16x8 a[kTI];
  bf16x8 b[kTJ];
};

// Fragments of 16-wide slice kk: lane l reads row base + 32*i + l%32 at
// logical chunk 2*kk + l/32, stored at chunk ^ ((row >> 1) & 7); roff[kk] holds
// that swizzled byte offset (the same for every row of the lane).
struct Lds {
  int a_row;            // byte offset of this lane's first A row
  int b_row;            // byte offset of this lane's row within the B tile
  int b_rows[kTJ];      // B tile row of fragment j
  int roff[4];
};

__device__ __forceinline__ void read_frag(const unsigned char* slot, const Lds& l, int kk, Frag& f) {
#pragma unroll
  for (int i = 0; i < kTI; ++i)
    f.a[i] = *reinterpret_cast<const bf16x8*>(slot + l.a_row + i * 32 * kRowBytes + l.roff[kk]);
#pragma unroll
  for (int j = 0; j < kTJ; ++j)
    f.b[j] = *reinterpret_cast<const bf16x8*>(slot + kTileBytes + l.b_row +
                                              l.b_rows[j] * kRowBytes + l.roff[kk]);
}

__device__ __forceinline__ void mma(f32x16 (&acc)[kTI][kTJ], const Frag& f) {
#pragma unroll
  for (int i = 0; i < kTI; ++i)
#pragma unroll
    for (int j = 0; j < kTJ; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Issue order of one slice: 16 MFMAs, the first R each followed by an LDS
// read, and N direct loads spread evenly between them, each after its two
// 64-bit address adds (without the VALU group the scheduler let the loads
// bunch up behind their address arithmetic).
template <int R, int N>
__device__ __forceinline__ void slice_order() {
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                     // MFMA
    if (q < R) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);          // LDS read
    if ((q * N) / 16 != ((q + 1) * N) / 16) {
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);                   // its address adds
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                   // direct load
    }
  }
}

// Barrier that publishes the direct loads every wave has waited for; the
// empty asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Stage d, multiplied from `cur` (slot d % 2); on entry f0 holds its slice 0.
// kLoad1: the B half of stage d+1's loads goes out over slice 0 (its A half
// went out after the previous barrier).  kNext: slice 0 of stage d+1 is read
// after the barrier.  kLoad2: the A half of stage d+2 goes into `cur` after
// the barrier, spread over slice 3.
template <bool kLoad1, bool kNext, bool kLoad2>
__device__ __forceinline__ void stage(f32x16 (&acc)[kTI][kTJ], Frag& f0, Frag& f1,
                                      unsigned char* cur, unsigned char* nxt, const Src& src,
                                      const Lds& l, int d) {
  __builtin_amdgcn_sched_barrier(0);
  if (kLoad1) load_runs<kLd, 2 * kLd>(nxt, src, (d + 1) * kBK * 2);
  read_frag(cur, l, 1, f1);
  mma(acc, f0);
  slice_order<kTI + kTJ, kLoad1 ? kLd : 0>();
  __builtin_amdgcn_sched_barrier(0);
  read_frag(cur, l, 2, f0);
  mma(acc, f1);
  slice_order<kTI + kTJ, 0>();
  __builtin_amdgcn_sched_barrier(0);
  read_frag(cur, l, 3, f1);
  mma(acc, f0);
  slice_order<kTI + kTJ, 0>();
  __builtin_amdgcn_sched_barrier(0);
  stage_barrier();                          // stage d+1 landed everywhere; cur is free
  __builtin_amdgcn_sched_barrier(0);
  if (kLoad2) load_runs<0, kLd>(cur, src, (d + 2) * kBK * 2);
  if (kNext) read_frag(nxt, l, 0, f0);
  mma(acc, f1);
  slice_order<kNext ? kTI + kTJ : 0, kLoad2 ? kLd : 0>();
  __builtin_amdgcn_sched_barrier(0);
}

// MODE 0: gate/up with SwiGLU epilogue, 1: down projection.  TAIL: the number of
// K stages is 1 (TAIL 1), even (TAIL 2) or odd and at least 3 (TAIL 3); each
// case is its own straight-line sequence of stages.
template <int MODE, int TAIL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_kernel(const uint16_t* __restrict__ A, int64_t n_rows, int K,
                         const int32_t* __restrict__ offs, int n_experts,
                         const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, int NB,
                         uint16_t* __restrict__ C, int ldc, int n_col_tiles, int n_cus,
                         float* __restrict__ partials, int* __restrict__ counters) {
  // two distinct arrays, so the compiler can tell the slot being loaded from
  // the slot being read and adds no wait between them
  __shared__ __align__(1024) unsigned char slot0[kSlotBytes];
  __shared__ __align__(1024) unsigned char slot1[kSlotBytes];

  const Unit u = find_unit(blockIdx.x, n_col_tiles, K / kBK, n_cus, offs, n_experts, n_rows);
  if (!u.ti.valid) return;
  const TileInfo& ti = u.ti;
  // this part's K stages [k_lo, k_hi) (all of K unless the tile is split; parts
  // cover an even number of stages each, so the stage sequence stays the even one)
  int k_lo = 0, kt_n = K / kBK;
  if (u.n_parts > 1) {
    const int half = kt_n / 2;
    k_lo = 2 * (u.part * half / u.n_parts);
    kt_n = 2 * ((u.part + 1) * half / u.n_parts) - k_lo;
  }
  const int64_t k_byte = int64_t(k_lo) * kBK * 2;

  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const int wm = w >> 1, wn = w & 1;

  Src src;
  src.a_base = reinterpret_cast<const unsigned char*>(A + ti.row0 * K) + k_byte;
  const int q = lane >> 3, pos = lane & 7;
#pragma unroll
  for (int i = 0; i < kLd; ++i) {
    const int r = i * (kThreads / kWave) + w;
    const int row = r * 8 + q;
    const int chunk = pos ^ ((row >> 1) & 7);
    src.lds_run[i] = r * 1024;
    int64_t gr = ti.row0 + row;
    if (gr >= ti.row_end) gr = ti.row_end - 1;            // clamped rows are never stored
    src.a_off[i] = (int(gr - ti.row0) * K + chunk * 8) * 2;
    if (MODE == 0) {
      const int64_t c0 = int64_t(ti.n_tile) * (kBN / 2);
      int64_t f = c0 + (row & (kBN / 2 - 1));
      if (f >= NB) f = NB - 1;                              // partial last column tile
      src.b_base[i] = reinterpret_cast<const unsigned char*>(
          (row < kBN / 2 ? B0 : B1) + (int64_t(ti.expert) * NB + c0) * K) + k_byte;
      src.b_off[i] = (int(f - c0) * K + chunk * 8) * 2;
    } else {
      const int64_t c0 = int64_t(ti.n_tile) * kBN;
      int64_t n = c0 + row;
      if (n >= NB) n = NB - 1;                              // partial last column tile
      src.b_base[i] = reinterpret_cast<const unsigned char*>(B0 + (int64_t(ti.expert) * NB + c0) * K) + k_byte;
      src.b_off[i] = (int(n - c0) * K + chunk * 8) * 2;
    }
  }

  // fragment rows: wave (wm, wn) owns A rows wm*128.. and B rows
  //   gate/up: j = 0, 1 gate rows wn*64 + 32j, j = 2, 3 the up rows of the same columns
  //   down:    wn*128 + 32j
  Lds l;
  const int r32 = lane & 31;
  l.a_row = (wm * kTI * 32 + r32) * kRowBytes;
  l.b_row = r32 * kRowBytes;
#pragma unroll
  for (int j = 0; j < kTJ; ++j)
    l.b_rows[j] = MODE == 0 ? (j >> 1) * (kBN / 2) + wn * 64 + (j & 1) * 32 : wn * 128 + j * 32;
  const int sw = (r32 >> 1) & 7;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) l.roff[kk] = ((2 * kk + (lane >> 5)) ^ sw) << 4;

  f32x16 acc[kTI][kTJ];
#pragma unroll
  for (int i = 0; i < kTI; ++i)
#pragma unroll
    for (int j = 0; j < kTJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // stage d lives in slot d % 2; every wave runs the same barrier sequence
  // kt_n >= 1 stages from k_lo; its parity is the one TAIL says.  The main
  // loop runs four stages per iteration (at its head the first loads wait for
  // the loop-carried K offset, so fewer heads keep the loads better spread),
  // then pairs.
  Frag f0, f1;
  load_runs<0, 2 * kLd>(slot0, src, 0);
  stage_barrier();                          // stage 0 landed
  read_frag(slot0, l, 0, f0);
  if constexpr (TAIL == 1) {
    stage<false, false, false>(acc, f0, f1, slot0, slot1, src, l, 0);
  } else {
    load_runs<0, kLd>(slot1, src, kBK * 2);   // A half of stage 1
    constexpr int kLeft = TAIL == 2 ? 2 : 3;  // stages after the loop of pairs
    int d = 0;
    for (; d + 4 <= kt_n - kLeft; d += 4) {
      stage<true, true, true>(acc, f0, f1, slot0, slot1, src, l, d);
      stage<true, true, true>(acc, f0, f1, slot1, slot0, src, l, d + 1);
      stage<true, true, true>(acc, f0, f1, slot0, slot1, src, l, d + 2);
      stage<true, true, true>(acc, f0, f1, slot1, slot0, src, l, d + 3);
    }
    for (; d < kt_n - kLeft; d += 2) {
      stage<true, true, true>(acc, f0, f1, slot0, slot1, src, l, d);
      stage<true, true, true>(acc, f0, f1, slot1, slot0, src, l, d + 1);
    }
    if constexpr (TAIL == 3) {
      stage<true, true, true>(acc, f0, f1, slot0, slot1, src, l, d);
      stage<true, true, false>(acc, f0, f1, slot1, slot0, src, l, d + 1);
      stage<false, false, false>(acc, f0, f1, slot0, slot1, src, l, d + 2);
    } else {
      stage<true, true, false>(acc, f0, f1, slot0, slot1, src, l, d);
      stage<false, false, false>(acc, f0, f1, slot1, slot0, src, l, d + 1);
    }
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(0));  // no direct load may outlive the workgroup

  if (u.n_parts > 1) {
    // a part of a split tile: store the fp32 partial (element e of the lane's
    // 256 at e * kThreads + tid, coalesced), then count the part; the last
    // part to arrive sums all of them in part order and writes the tile
    const int tid = threadIdx.x;
    float* mine = partials + int64_t(u.unit) * kTileElems;
#pragma unroll
    for (int i = 0; i < kTI; ++i)
#pragma unroll
      for (int j = 0; j < kTJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) mine[((i * kTJ + j) * 16 + v) * kThreads + tid] = acc[i][j][v];
    __shared__ int s_last;
    __threadfence();                        // the partial is visible device-wide ...
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&counters[u.tail], 1) == u.n_parts - 1;   // ... before the count
    __syncthreads();
    if (!s_last) return;
    __threadfence();                        // every part's partial is visible here
    // sum in part order, one part at a time so each part's 256 loads per lane
    // are independent and go out together
    for (int p = 0; p < u.n_parts; ++p) {
      const float* part = partials + (int64_t(u.tail) * u.n_parts + p) * kTileElems + tid;
#pragma unroll
      for (int i = 0; i < kTI; ++i)
#pragma unroll
        for (int j = 0; j < kTJ; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float x = part[((i * kTJ + j) * 16 + v) * kThreads];
            acc[i][j][v] = p == 0 ? x : acc[i][j][v] + x;
          }
    }
  }

  // epilogue: lane holds C[8*(v/4) + 4*(lane/32) + v%4][lane%32] of each 32x32 tile
  const int khalf = lane >> 5;
#pragma unroll
  for (int i = 0; i < kTI; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * (kTI * 32) + 32 * i + 8 * (v >> 2) + 4 * khalf + (v & 3);
      const int64_t gr = ti.row0 + r;
      if (gr >= ti.row_end) continue;
      if (MODE == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t col = int64_t(ti.n_tile) * (kBN / 2) + wn * 64 + 32 * j + r32;
          const float h = silu(acc[i][j][v]) * acc[i][j + 2][v];
          if (col < NB) C[gr * ldc + col] = f32_to_bf16_rne(h);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kTJ; ++j) {
          const int64_t col = int64_t(ti.n_tile) * kBN + wn * 128 + 32 * j + r32;
          if (col < NB) C[gr * ldc + col] = f32_to_bf16_rne(acc[i][j][v]);
        }
      }
    }
  }
}

}  // namespace

int64_t grouped_swiglu_tiles(int64_t n_rows, int n_experts, int64_t hidden, int64_t ffn) {
  const int64_t m = (n_rows + kBM - 1) / kBM + n_experts;
  const int64_t c1 = (ffn + kBN / 2 - 1) / (kBN / 2), c2 = (hidden + kBN - 1) / kBN;
  return m * (c1 > c2 ? c1 : c2);
}

namespace {

// Workspace: h [R, F] bf16 | per-launch counters of the split tiles (2 x
// kCuMax int32) | fp32 partial tiles of the split parts (kCuMax at most).
struct SwigluLayout {
  size_t counters, partials, total;
};

SwigluLayout swiglu_layout(int64_t n_rows, int64_t ffn) {
  SwigluLayout L;
  L.counters = (size_t(n_rows) * size_t(ffn) * 2 + 255) / 256 * 256;
  L.partials = L.counters + 2 * kCuMax * sizeof(int32_t);
  L.total = L.partials + size_t(kCuMax) * kTileElems * sizeof(float);
  return L;
}

__global__ void zero_counters_kernel(int32_t* __restrict__ c, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) c[i] = 0;
}

// CUs of the current device, as a multiple of kXcds in [kXcds, kCuMax],
// queried once per device and kept (a racing first call stores the same value).
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = kCuMax;
  if (dev < 0 || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n = kCuMax;
  n = n / kXcds * kXcds;
  n = n < kXcds ? kXcds : (n > kCuMax ? kCuMax : n);
  if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace

size_t grouped_swiglu_workspace_bytes(int64_t n_rows, int n_experts, int64_t hidden, int64_t ffn) {
  (void)n_experts;
  (void)hidden;
  return swiglu_layout(n_rows, ffn).total + 256;
}

hipError_t launch_grouped_swiglu(const void* rows, int64_t n_rows, int64_t hidden,
                                 const int32_t* expert_offsets, int n_experts, const void* w_gate,
                                 const void* w_up, const void* w_down, int64_t ffn, void* y,
                                 void* workspace, hipStream_t stream) {
  const SwigluLayout L = swiglu_layout(n_rows, ffn);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws);
  int32_t* counters = reinterpret_cast<int32_t*>(ws + L.counters);
  float* partials = reinterpret_cast<float*>(ws + L.partials);
  const int n_cus = cu_count();
  // worst case of real row tiles: ceil(R / 256) plus one partial tile per expert;
  // the grid also holds the extra parts of the split tiles (fewer than n_cus)
  const int max_m_tiles = int((n_rows + kBM - 1) / kBM) + n_experts;
  auto grid_for = [&](int n_col_tiles) {
    const int64_t units = int64_t(max_m_tiles) * n_col_tiles + n_cus;
    return unsigned((units + kXcds - 1) / kXcds * kXcds);
  };
  auto kernel_for = [](int64_t k, auto k1, auto k2, auto k3) {
    const int64_t stages = k / kBK;
    return stages == 1 ? k1 : (stages % 2 == 0 ? k2 : k3);
  };
  zero_counters_kernel<<<1, 256, 0, stream>>>(counters, 2 * kCuMax);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // gate/up: F/(kBN/2) column tiles (kBN/2 gate + kBN/2 up rows per B tile), K = D
  const int nct1 = int((ffn + kBN / 2 - 1) / (kBN / 2));
  kernel_for(hidden, grouped_gemm_kernel<0, 1>, grouped_gemm_kernel<0, 2>,
             grouped_gemm_kernel<0, 3>)<<<grid_for(nct1), kThreads, 0, stream>>>(
      static_cast<const uint16_t*>(rows), n_rows, int(hidden), expert_offsets, n_experts,
      static_cast<const uint16_t*>(w_gate), static_cast<const uint16_t*>(w_up), int(ffn), h,
      int(ffn), nct1, n_cus, partials, counters);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  // down: ceil(D/kBN) column tiles, K = F
  const int nct2 = int((hidden + kBN - 1) / kBN);
  kernel_for(ffn, grouped_gemm_kernel<1, 1>, grouped_gemm_kernel<1, 2>,
             grouped_gemm_kernel<1, 3>)<<<grid_for(nct2), kThreads, 0, stream>>>(
      h, n_rows, int(ffn), expert_offsets, n_experts, static_cast<const uint16_t*>(w_down),
      nullptr, int(hidden), static_cast<uint16_t*>(y), int(hidden), nct2, n_cus, partials,
      counters + kCuMax);
  return hipGetLastError();
}

}  // namespace moe
