// SwiGLU expert FFN over rows left in any order, each row naming its own
// expert: y[r] = FFN_{row_expert[r]}(rows[r]).
//
// "backends/mlx: runtime MoE expert-sort for decode (issue #20554)": decode
// keeps the rows in token order (no argsort) and hands the expert product a
// per-row expert id (gather_mm with unsorted right-hand indices); expert
// weights are laid out [E, out, in].  The result is defined row by row.
//
// A product that fetched an expert's weights once per row would read them as
// many times as the expert has rows.  Here a stable counting sort of the R
// expert ids (the same ranking as the sorted dispatch, on 4-byte ids only)
// lists the rows of each expert, and every active expert's weights stream from
// HBM once for all of its rows.  The rows themselves do not move: the row
// operand is gathered through that list and y is written back at each row's
// own position.
//
// At decode sizes an expert has a handful of rows (1024 rows over 256
// experts: 4 on average), so both products are bound by the weight stream:
// three [F, D] matrices per active expert against at most 16 rows.  Shape:
//   * a pass is up to 16 rows of one expert, one 16-row tile of
//     v_mfma_f32_16x16x32_bf16; an expert with more rows takes several passes;
//   * a wave owns 64 weight rows over the whole K (gate/up: 32 F columns of
//     W_gate and the same 32 of W_up, so h = silu(g) * u is lane-local; down:
//     64 D columns) and streams them straight into registers, 128 K-elements
//     per chunk with the next chunk in flight; no LDS, no barriers;
//   * the 16 rows of a pass are read through L2, where each of the pass's
//     column groups finds them; consecutive workgroups (one XCD) take the
//     column groups of one pass.
// Lane (n = l % 16, g = l / 16) holds row/column n and elements
// [32 s + 8 g, +8) of MFMA step s; A and B use the same assignment, so each
// step's 32-wide dot products cover their K slice exactly once.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPass = 16;           // rows per pass
constexpr int kKC = 128;            // K elements per chunk
constexpr int kSteps = kKC / 32;    // MFMA K steps per chunk
constexpr int kNT = 4;              // 16-wide weight tiles per wave
constexpr int kWaves = 4;           // waves per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr int kXcds = 8;
constexpr int kPlanThreads = 1024;  // one thread per expert (n_experts <= kMaxExperts)

__device__ __forceinline__ float silu(float a) { return a / (1.f + expf(-a)); }

struct Chunk {
  bf16x8 a[kSteps];
  bf16x8 b[kNT][kSteps];
};

__device__ __forceinline__ void load_chunk(Chunk& ch, const uint16_t* a,
                                           const uint16_t* const (&b)[kNT], int c) {
  const int k0 = c * kKC;
#pragma unroll
  for (int s = 0; s < kSteps; ++s) ch.a[s] = *reinterpret_cast<const bf16x8*>(a + k0 + 32 * s);
#pragma unroll
  for (int t = 0; t < kNT; ++t)
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
      ch.b[t][s] = *reinterpret_cast<const bf16x8*>(b[t] + k0 + 32 * s);
}

__device__ __forceinline__ void mma(f32x4 (&acc)[kNT], const Chunk& ch) {
#pragma unroll
  for (int s = 0; s < kSteps; ++s)
#pragma unroll
    for (int t = 0; t < kNT; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ch.a[s], ch.b[t][s], acc[t], 0, 0, 0);
}

// Pass list from the expert offsets: expert e owns ceil(count_e / 16) passes;
// pass i = {expert, first row, end of the expert's rows} in grouped order.
__global__ __launch_bounds__(kPlanThreads) void gather_plan_kernel(
    const int32_t* __restrict__ offs, int n_experts, int4* __restrict__ passes,
    int32_t* __restrict__ n_passes) {
  __shared__ int s_base[kMaxExperts + 1];
  __shared__ int s_wave[kPlanThreads / kWave + 1];
  const int e = threadIdx.x;
  int np = 0;
  if (e < n_experts) {
    const int c = offs[e + 1] - offs[e];
    np = c > 0 ? (c + kPass - 1) / kPass : 0;
  }
  int total;
  const int base = block_exclusive_scan(np, s_wave, &total);
  if (e < n_experts) s_base[e] = base;
  if (e == 0) {
    s_base[n_experts] = total;
    n_passes[0] = total;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < total; i += kPlanThreads) {
    // the last expert whose first pass is <= i owns pass i (an expert with
    // no passes shares its base with the next one, which then wins)
    int lo = 0, hi = n_experts - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_base[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    passes[i] = make_int4(lo, offs[lo] + (i - s_base[lo]) * kPass, offs[lo + 1], 0);
  }
}

// MODE 0: A = rows [R, D] gathered through order, B = W_gate / W_up [E, F, D],
//         C = h [R, F] in grouped order, h = bf16(silu(g) * u).
// MODE 1: A = h [R, F] in grouped order, B = W_down [E, D, F],
//         C = y [R, D] at the rows' own positions order[p].
template <int MODE>
__global__ __launch_bounds__(kThreads) void gather_gemm_kernel(
    const uint16_t* __restrict__ A, int K, const int32_t* __restrict__ order,
    const int4* __restrict__ passes, const int32_t* __restrict__ n_passes, int n_groups,
    int n_tiles, const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, int NB,
    uint16_t* __restrict__ C, int ldc) {
  // XCD-aware placement: workgroup b runs on XCD b % 8; each XCD takes a
  // contiguous range of tile ids, tile = pass * n_groups + column group
  const int nb = gridDim.x;                 // a multiple of kXcds
  const int b = blockIdx.x;
  const int tile = (b % kXcds) * (nb / kXcds) + b / kXcds;
  if (tile >= n_tiles) return;
  const int pass = tile / n_groups, grp = tile % n_groups;
  if (pass >= __builtin_amdgcn_readfirstlane(n_passes[0])) return;
  const int4 ps = passes[pass];
  const int expert = __builtin_amdgcn_readfirstlane(ps.x);
  const int row0 = __builtin_amdgcn_readfirstlane(ps.y);
  const int row_end = __builtin_amdgcn_readfirstlane(ps.z);

  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  const int n = lane & 15, g = lane >> 4;
  constexpr int kCols = MODE == 0 ? 32 : 64;           // output columns per wave
  const int col0 = (grp * kWaves + w) * kCols;
  if (col0 >= NB) return;                               // past the last column; no barriers follow

  // rows past the end of the pass repeat its first row; they are never stored
  const int p = row0 + n < row_end ? row0 + n : row0;
  const int64_t arow = MODE == 0 ? int64_t(order[p]) : int64_t(p);
  const uint16_t* a_ptr = A + arow * K + 8 * g;
  const uint16_t* b_ptr[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    // gate/up: tiles 0, 1 = gate columns col0 + 16t, tiles 2, 3 = the same columns of up
    int col = MODE == 0 ? col0 + 16 * (t & 1) + n : col0 + 16 * t + n;
    if (col >= NB) col = NB - 1;                        // partial last group; never stored
    const uint16_t* base = (MODE == 0 && t >= 2) ? B1 : B0;
    b_ptr[t] = base + (int64_t(expert) * NB + col) * K + 8 * g;
  }

  f32x4 acc[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // two chunks in registers: chunk c is multiplied while chunk c + 1 loads
  const int nc = K / kKC;
  Chunk c0, c1;
  load_chunk(c0, a_ptr, b_ptr, 0);
  if (nc > 1) load_chunk(c1, a_ptr, b_ptr, 1);
  int c = 0;
  for (; c + 3 < nc; c += 2) {
    mma(acc, c0);
    load_chunk(c0, a_ptr, b_ptr, c + 2);
    mma(acc, c1);
    load_chunk(c1, a_ptr, b_ptr, c + 3);
  }
  if (c + 2 < nc) {                                     // three chunks left
    mma(acc, c0);
    load_chunk(c0, a_ptr, b_ptr, c + 2);
    mma(acc, c1);
    mma(acc, c0);
  } else if (c + 1 < nc) {                              // two left
    mma(acc, c0);
    mma(acc, c1);
  } else {
    mma(acc, c0);
  }

  // lane holds C[4 g + i][n] of each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pr = row0 + 4 * g + i;
    if (pr >= row_end) continue;
    if (MODE == 0) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int col = col0 + 16 * hh + n;
        if (col < NB)
          C[int64_t(pr) * ldc + col] = f32_to_bf16_rne(silu(acc[hh][i]) * acc[2 + hh][i]);
      }
    } else {
      const int64_t dst = order[pr];
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        const int col = col0 + 16 * t + n;
        if (col < NB) C[dst * ldc + col] = f32_to_bf16_rne(acc[t][i]);
      }
    }
  }
}

// Workspace: grouping maps, the pass list, then h.
struct GatherLayout {
  size_t counts, offsets, seg_offsets, dst_pos, order, n_passes, passes, dispatch_ws, h, total;
  int max_passes;
};

size_t round256(size_t v) { return (v + 255) / 256 * 256; }

GatherLayout gather_layout(int64_t n_rows, int n_experts, int64_t ffn) {
  GatherLayout L{};
  L.max_passes = int((n_rows + kPass - 1) / kPass) + n_experts;
  size_t o = 0;
  L.counts = o;      o += round256(size_t(n_experts) * 4);
  L.offsets = o;     o += round256(size_t(n_experts + 1) * 4);
  L.seg_offsets = o; o += round256(2 * 4);
  L.dst_pos = o;     o += round256(size_t(n_rows) * 4);
  L.order = o;       o += round256(size_t(n_rows) * 4);
  L.n_passes = o;    o += 256;
  L.passes = o;      o += round256(size_t(L.max_passes) * 16);
  L.dispatch_ws = o; o += round256(dispatch_workspace_bytes(n_rows, n_experts, 1, 1));
  L.h = o;           o += round256(size_t(n_rows) * size_t(ffn) * 2);
  L.total = o;
  return L;
}

}  // namespace

size_t gather_swiglu_workspace_bytes(int64_t n_rows, int n_experts, int64_t hidden, int64_t ffn) {
  (void)hidden;
  return gather_layout(n_rows, n_experts, ffn).total;
}

int64_t gather_swiglu_tiles(int64_t n_rows, int n_experts, int64_t hidden, int64_t ffn) {
  const int64_t passes = (n_rows + kPass - 1) / kPass + n_experts;
  const int64_t g1 = (ffn + kWaves * 32 - 1) / (kWaves * 32);
  const int64_t g2 = (hidden + kWaves * 64 - 1) / (kWaves * 64);
  return passes * (g1 > g2 ? g1 : g2);
}

hipError_t launch_gather_swiglu(const void* rows, int64_t n_rows, int64_t hidden,
                                const int32_t* row_expert, int n_experts, const void* w_gate,
                                const void* w_up, const void* w_down, int64_t ffn, void* y,
                                void* workspace, hipStream_t stream) {
  const GatherLayout L = gather_layout(n_rows, n_experts, ffn);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* order = reinterpret_cast<int32_t*>(ws + L.order);
  int32_t* n_passes = reinterpret_cast<int32_t*>(ws + L.n_passes);
  int4* passes = reinterpret_cast<int4*>(ws + L.passes);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h);

  // 1. rows of each expert, ascending: the sorted ranking of the ids with top_k = 1
  DispatchArgs d{};
  d.n_tokens = n_rows;
  d.topk_idx = row_expert;
  d.n_experts = n_experts;
  d.k = 1;
  d.n_segments = 1;
  d.sorted = 1;
  d.expert_counts = reinterpret_cast<int32_t*>(ws + L.counts);
  d.expert_offsets = offsets;
  d.segment_offsets = reinterpret_cast<int32_t*>(ws + L.seg_offsets);
  d.dst_pos = reinterpret_cast<int32_t*>(ws + L.dst_pos);
  d.src_pair = order;
  d.workspace = ws + L.dispatch_ws;
  hipError_t err = launch_dispatch(d, stream);
  if (err != hipSuccess) return err;

  // 2. pass list
  gather_plan_kernel<<<1, kPlanThreads, 0, stream>>>(offsets, n_experts, passes, n_passes);
  err = hipGetLastError();
  if (err != hipSuccess) return err;

  auto grid_for = [](int64_t tiles) { return unsigned((tiles + kXcds - 1) / kXcds * kXcds); };
  // 3. gate/up: 128 F columns per workgroup, K = D
  const int g1 = int((ffn + kWaves * 32 - 1) / (kWaves * 32));
  const int64_t t1 = int64_t(L.max_passes) * g1;
  gather_gemm_kernel<0><<<grid_for(t1), kThreads, 0, stream>>>(
      static_cast<const uint16_t*>(rows), int(hidden), order, passes, n_passes, g1, int(t1),
      static_cast<const uint16_t*>(w_gate), static_cast<const uint16_t*>(w_up), int(ffn), h,
      int(ffn));
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  // 4. down: 256 D columns per workgroup, K = F
  const int g2 = int((hidden + kWaves * 64 - 1) / (kWaves * 64));
  const int64_t t2 = int64_t(L.max_passes) * g2;
  gather_gemm_kernel<1><<<grid_for(t2), kThreads, 0, stream>>>(
      h, int(ffn), order, passes, n_passes, g2, int(t2), static_cast<const uint16_t*>(w_down),
      nullptr, int(hidden), static_cast<uint16_t*>(y), int(hidden));
  return hipGetLastError();
}

}  // namespace moe
