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
//   * a tile is 64 rows x 128 columns of one expert and K advances in blocks
//     of 128 (one scale block); its 8 waves each own 32 rows x 32 columns;
//   * weights and rows go from global memory straight into LDS
//     (global_load_lds_dwordx4), eight lanes per 128-byte line, so every load
//     instruction reads whole lines; the row tile is loaded once per
//     workgroup for its eight waves; each wave's 32 row scales ride along;
//   * a ring of three LDS slots keeps block kt+2 loading while block kt is
//     multiplied; one barrier per block publishes block kt+1 and retires the
//     reads of the slot block kt+2 overwrites.  Two workgroups fit per CU;
//   * each lane multiplies 64 contiguous bytes of its row and column per
//     block, 8-byte group g feeding MFMA g (v_mfma_f32_32x32x16_fp8_fp8),
//     which permutes K identically on both operands;
//   * each block's fp32 partial sum is scaled by sx * sw and added to the
//     accumulator;
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
constexpr int kThreads = 512;   // 8 waves: 2 row halves x 4 column groups of 32
constexpr int kXcds = 8;

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
    const int incl = wave_inclusive_scan(nt);         // DPP, no LDS round trips
    const int excl = incl - nt;
    const uint64_t own = ballot(nt > 0 && m_idx >= base + excl && m_idx < base + incl);
    if (own) {
      const int src = __ffsll((unsigned long long)own) - 1;
      const int lo_s = lane_value(lo, src), hi_s = lane_value(hi, src), ex_s = lane_value(excl, src);
      t.expert = c + src;
      t.row0 = lo_s + int64_t(m_idx - base - ex_s) * kTM;
      t.row_end = hi_s;
      t.valid = true;
      return t;
    }
    base += lane_value(incl, kWave - 1);
  }
  return t;
}

// LDS ring slot: the weight tile (128 columns x 128 bytes of K), the row tile
// (64 rows x 128 bytes) and, per wave, the scales of its 32 rows for one K
// block.  Rows of both
// tiles are 128 bytes with their 16-byte chunks XOR-swizzled by
// ((row >> 1) & 7): the 16 rows one 16-lane phase of a ds_read_b128 reads
// fall in 16 distinct 16-byte bank groups.
constexpr int kWaves = kThreads / 64;
constexpr int kSlotW = 0;
constexpr int kSlotA = kTN * kQB;                 // 16 KB
constexpr int kSlotS = kSlotA + kTM * kQB;        // + 8 KB
constexpr int kSlotBytes = kSlotS + kWaves * 256; // + each wave's copy of its 32 row scales
constexpr int kDmaW = kTN * kQB / (kThreads * 16);   // 1 KB runs per wave: weights (2)
constexpr int kDmaA = kTM * kQB / (kThreads * 16);   // rows (1)
constexpr int kDmaPerStage = kDmaW + kDmaA + 1;      // + one run of row scales
// Three 26 KB slots let two workgroups (16 waves) share a CU; deeper rings
// (4 or 6 slots, one workgroup per CU) measured slower.
constexpr int kRingSlots = 3;

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kQB + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8): at most n vector-memory operations of this wave
// outstanding and (lgkm0) all of its LDS operations returned.
constexpr unsigned wait_vm_lgkm0(int n) {
  return unsigned(n & 15) | (unsigned((n >> 4) & 3) << 14) | (0x7u << 4);
}
constexpr unsigned wait_vm(int n) {
  return unsigned(n & 15) | (unsigned((n >> 4) & 3) << 14) | (0x7u << 4) | (0xFu << 8);
}

struct Sources {
  const uint8_t* w[kDmaW];     // this lane's 16 bytes of each weight run (K block 0)
  const uint8_t* a[kDmaA];     // and of each row run
  const float* sx;             // the row scale of K block 0 this lane copies
  int w_lds[kDmaW], a_lds[kDmaA], s_lds;   // wave-uniform LDS offsets in a slot
};

// One direct global->LDS load: M0 holds the LDS byte address of the run and
// lane l's bytes land at M0 + l * size.  Issued from asm so that the
// compiler's own wait insertion does not track it (it would conservatively
// wait for every direct load in flight before reading any ring slot); the
// explicit vmcnt waits at the block barriers are what orders these loads.
// The instruction writes no register.
typedef const __attribute__((address_space(3))) unsigned char* lds_cptr;
__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
  return uint32_t(size_t((lds_cptr)p));
}
// M0 is saved and restored around the load, so the compiler's own use of it
// is undisturbed.
__device__ __forceinline__ void dma16(const uint8_t* g, const unsigned char* l) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\ts_nop 0\n\ts_mov_b32 m0, %0"
      : "=&s"(keep) : "s"(lds_addr(l)), "v"(g) : "memory");
}
__device__ __forceinline__ void dma4(const float* g, const unsigned char* l) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "global_load_lds_dword %2, off\n\ts_nop 0\n\ts_mov_b32 m0, %0"
      : "=&s"(keep) : "s"(lds_addr(l)), "v"(g) : "memory");
}

// Direct global->LDS loads of K block `blk` into one ring slot (kDmaPerStage
// operations per wave, every lane active).
__device__ __forceinline__ void load_block(unsigned char* slot, const Sources& src, int blk) {
  const int64_t o = int64_t(blk) * kQB;
#pragma unroll
  for (int i = 0; i < kDmaW; ++i) dma16(src.w[i] + o, slot + src.w_lds[i]);
#pragma unroll
  for (int i = 0; i < kDmaA; ++i) dma16(src.a[i] + o, slot + src.a_lds[i]);
  dma4(src.sx + blk, slot + src.s_lds);
}

template <unsigned kWait>
__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_s_waitcnt(kWait);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ long lo8(u32x4 q) {
  return long((unsigned long)q.x | ((unsigned long)q.y << 32));
}
__device__ __forceinline__ long hi8(u32x4 q) {
  return long((unsigned long)q.z | ((unsigned long)q.w << 32));
}

// acc += sx * sw * (K block partial products) for this wave's 32 rows and 32
// columns.  Lane l multiplies bytes [64 * (l / 32), +64) of its row and
// column; 8-byte group g feeds MFMA g, the same on both operands.
__device__ __forceinline__ void block_mma(f32x16& acc, const unsigned char* slot, int w_row,
                                          int a_row, int s_off, int half, float sw) {
  u32x4 wb[4], a[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    wb[i] = *reinterpret_cast<const u32x4*>(slot + kSlotW + swz(w_row, half * 4 + i));
    a[i] = *reinterpret_cast<const u32x4*>(slot + kSlotA + swz(a_row, half * 4 + i));
  }
  f32x16 p;
#pragma unroll
  for (int v = 0; v < 16; ++v) p[v] = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(lo8(a[i]), lo8(wb[i]), p, 0, 0, 0);
    p = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(hi8(a[i]), hi8(wb[i]), p, 0, 0, 0);
  }
  // lane holds rows 8*(v/4) + 4*half + v%4 of the wave's 32 rows
  // (read as an ext-vector type like the operands: the compiler then knows the
  // read cannot touch the slot being loaded and adds no wait for the loads)
  const unsigned char* sx = slot + s_off + 16 * half;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 s4 = *reinterpret_cast<const u32x4*>(sx + 32 * q);
    const float r[4] = {__uint_as_float(s4.x), __uint_as_float(s4.y), __uint_as_float(s4.z),
                        __uint_as_float(s4.w)};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[4 * q + i] = __builtin_fmaf(r[i] * sw, p[4 * q + i], acc[4 * q + i]);
  }
}

// One K block: wait for block kt (only block kt+1's loads may be in flight),
// then load block kt+2 into the slot block kt-1 used (every wave has passed
// this barrier, so all its reads of that slot are done), then multiply.
// One K block of a ring of NS slots: wait for block kt (the loads of blocks
// kt+1 .. kt+NS-2 may still be in flight), then load block kt+NS-1 into the
// slot block kt-1 used (every wave has passed this barrier, so all its reads
// of that slot are done), then multiply.
template <int NS>
__device__ __forceinline__ void block_step(f32x16& acc, unsigned char* ring, const Sources& src,
                                           int kt, int kb, const float* __restrict__ swp,
                                           int w_row, int a_row, int s_off, int half) {
  block_barrier<wait_vm_lgkm0((NS - 2) * kDmaPerStage)>();
  // past the last block the loads repeat it into a slot that is not multiplied
  load_block(ring + ((kt + NS - 1) % NS) * kSlotBytes, src, min(kt + NS - 1, kb - 1));
  block_mma(acc, ring + (kt % NS) * kSlotBytes, w_row, a_row, s_off, half, swp[kt]);
}

template <int NS>   // LDS ring slots
__global__ __launch_bounds__(kThreads) void grouped_gemm_fp8_kernel(
    const uint8_t* __restrict__ rows, const float* __restrict__ row_scales, int64_t n_rows,
    int K, const int32_t* __restrict__ offs, int n_experts, const uint8_t* __restrict__ w,
    const float* __restrict__ w_scales, int N, uint16_t* __restrict__ y, int max_m_tiles,
    int n_tiles) {
  __shared__ __align__(1024) unsigned char ring[NS * kSlotBytes];

  // workgroup b runs on XCD b % 8; XCD x takes row tiles x, x + 8, ..., each
  // with all its column tiles back to back (the tile's rows stay in that XCD's
  // L2).  The grid covers the worst-case row-tile count; interleaving the row
  // tiles over the XCDs spreads the unused ones evenly.
  const int b = blockIdx.x;
  const int slot = b / kXcds;
  const int m_idx = (slot / n_tiles) * kXcds + b % kXcds, n_tile = slot % n_tiles;
  if (m_idx >= max_m_tiles) return;
  Fp8Tile ti = find_fp8_tile(m_idx, offs, n_experts, n_rows);
  if (!ti.valid) return;
  // the lookup's results are wave-uniform; saying so keeps the tile's
  // addresses (and the weight-scale loads) in scalar registers
  ti.expert = __builtin_amdgcn_readfirstlane(ti.expert);
  ti.row0 = __builtin_amdgcn_readfirstlane(int(ti.row0));
  ti.row_end = __builtin_amdgcn_readfirstlane(int(ti.row_end));

  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const int hw = wv >> 2, cg = wv & 3;      // row half and column group of this wave
  const int half = lane >> 5;
  const int kb = K / kQB;
  const int64_t col0 = int64_t(n_tile) * kTN;

  // Direct-load assignment: run i of wave wv covers 8 rows of a tile (1 KB);
  // lane l writes LDS bytes l * 16 of the run, i.e. row l / 8, physical chunk
  // l % 8, which holds logical chunk (l % 8) ^ ((row >> 1) & 7).
  Sources src;
#pragma unroll
  for (int i = 0; i < kDmaW; ++i) {
    const int run = i * kWaves + wv;
    const int row = run * 8 + lane / 8;
    const int c = (lane % 8) ^ ((row >> 1) & 7);
    src.w[i] = w + (int64_t(ti.expert) * N + col0 + row) * K + c * 16;
    src.w_lds[i] = kSlotW + run * 1024;
  }
#pragma unroll
  for (int i = 0; i < kDmaA; ++i) {
    const int run = i * kWaves + wv;
    const int row = run * 8 + lane / 8;
    const int c = (lane % 8) ^ ((row >> 1) & 7);
    int64_t gr = ti.row0 + row;
    if (gr >= ti.row_end) gr = ti.row_end - 1;       // clamped rows are never stored
    src.a[i] = rows + gr * K + c * 16;
    src.a_lds[i] = kSlotA + run * 1024;
  }
  {
    // lane l copies the scale of the wave's row l % 32 (lanes 32..63 repeat it)
    int64_t gr = ti.row0 + hw * 32 + (lane & 31);
    if (gr >= ti.row_end) gr = ti.row_end - 1;
    src.sx = row_scales + gr * kb;
    src.s_lds = kSlotS + wv * 256;
  }
  const float* swp = w_scales + (int64_t(ti.expert) * (N / kQB) + n_tile) * kb;
  const int w_row = cg * 32 + (lane & 31);     // this wave's 32 weight columns
  const int a_row = hw * 32 + (lane & 31);     // and 32 rows
  const int s_off = src.s_lds;

  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) load_block(ring + i * kSlotBytes, src, min(i, kb - 1));
  for (int kt = 0; kt < kb; ++kt) block_step<NS>(acc, ring, src, kt, kb, swp, w_row, a_row, s_off, half);
  __builtin_amdgcn_s_waitcnt(wait_vm(0));   // no direct load may outlive the workgroup

  // acc[v] = C[8*(v/4) + 4*half + v%4][lane % 32] of the wave's 32 x 32 block
  const int64_t col = col0 + cg * 32 + (lane & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t g = ti.row0 + hw * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
    if (g < ti.row_end) y[g * N + col] = f32_to_bf16_rne(acc[v]);
  }
}

}  // namespace

hipError_t launch_grouped_gemm_fp8(const void* rows, const float* row_scales, int64_t n_rows,
                                   int64_t k_dim, const int32_t* expert_offsets, int n_experts,
                                   const void* w, const float* w_scales, int64_t n_dim, void* y,
                                   hipStream_t stream) {
  const int max_m_tiles = int((n_rows + kTM - 1) / kTM) + n_experts;
  const int n_tiles = int(n_dim / kTN);
  const int64_t m_slots = (int64_t(max_m_tiles) + kXcds - 1) / kXcds * kXcds;
  const unsigned grid = unsigned(m_slots * n_tiles);
  grouped_gemm_fp8_kernel<kRingSlots><<<grid, kThreads, 0, stream>>>(
      static_cast<const uint8_t*>(rows), row_scales, n_rows, int(k_dim), expert_offsets,
      n_experts, static_cast<const uint8_t*>(w), w_scales, int(n_dim),
      static_cast<uint16_t*>(y), max_m_tiles, n_tiles);
  return hipGetLastError();
}

}  // namespace moe
