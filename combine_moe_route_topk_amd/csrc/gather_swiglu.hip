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
//   * a workgroup of 8 waves takes one pass and a group of columns; a wave
//     owns 32 weight rows over the whole K (gate/up: 16 F columns of W_gate
//     and the same 16 of W_up, so h = silu(g) * u is lane-local; down: 32 D
//     columns) and streams them straight into registers, 512 K-elements of
//     each weight row in flight;
//   * the pass's 16 rows are staged through LDS 1024 K-elements at a time,
//     double-buffered, one barrier per stage: each row byte is fetched once per
//     workgroup instead of once per wave, which keeps the weight stream alone
//     on the memory queues;
//   * the pass count is only known on the device, so the grid is sized for the
//     worst case; workgroup b runs on XCD b % 8 and XCD x takes passes
//     x, x + 8, x + 16, ... (all column groups of one pass back to back, so its
//     rows stay in that XCD's L2), which spreads the unused tail of the grid
//     evenly over the XCDs.
// Lane (n = l % 16, g = l / 16) holds row/column n and elements
// [32 s + 8 g, +8) of MFMA step s; A and B use the same assignment, so each
// step's 32-wide dot products cover their K slice exactly once.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPass = 16;           // rows per pass
constexpr int kNT = 2;              // 16-wide weight tiles per wave
constexpr int kWaves = 8;           // waves per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr int kSK = 1024;           // K elements per LDS stage
constexpr int kPitch = kSK * 2 + 16;   // LDS row pitch: rows land 4 banks apart
constexpr int kPieces = kPass * kSK / 8 / kThreads;   // 16-byte staging loads per thread
constexpr int kXcds = 8;
constexpr int kPlanThreads = 1024;  // one thread per expert (n_experts <= kMaxExperts)

__device__ __forceinline__ float silu(float a) { return a / (1.f + expf(-a)); }

// One chunk (KC K-elements) of this lane's weight fragments: tile t, MFMA step s.
template <int KC>
struct BChunk {
  bf16x8 b[kNT][KC / 32];
};

template <int KC>
__device__ __forceinline__ void load_chunk(BChunk<KC>& ch, const uint16_t* const (&b)[kNT], int c) {
#pragma unroll
  for (int t = 0; t < kNT; ++t)
#pragma unroll
    for (int s = 0; s < KC / 32; ++s)
      ch.b[t][s] = *reinterpret_cast<const bf16x8*>(b[t] + c * KC + 32 * s);
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
// MODE 2: as MODE 1, but y is not stored: the fp32 result of row r, which
//         holds pair q = fc.row_pair[r] (q = r without the map), is weighted
//         by topk_w[q] and added into out[q / k] (the combine, fused).
// The weights stream in chunks of KC K-elements with DEPTH chunks in flight
// (KC = 256, DEPTH = 2 when K is a multiple of 256, else 128 and 4: the same
// bytes in flight and the same order of accumulation).
template <int MODE, int KC, int DEPTH>
__global__ __launch_bounds__(kThreads) void gather_gemm_kernel(
    const uint16_t* __restrict__ A, int K, const int32_t* __restrict__ order,
    const int4* __restrict__ passes, const int32_t* __restrict__ n_passes, int n_groups,
    const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, int NB,
    uint16_t* __restrict__ C, int ldc, FusedCombine fc) {
  __shared__ __align__(16) unsigned char sa[2][kPass * kPitch];
  const int b = blockIdx.x;
  const int slot = b / kXcds;
  const int pass = (slot / n_groups) * kXcds + b % kXcds, grp = slot % n_groups;
  if (pass >= __builtin_amdgcn_readfirstlane(n_passes[0])) return;   // whole workgroup
  const int4 ps = passes[pass];
  const int expert = __builtin_amdgcn_readfirstlane(ps.x);
  const int row0 = __builtin_amdgcn_readfirstlane(ps.y);
  const int row_end = __builtin_amdgcn_readfirstlane(ps.z);

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 15, g = lane >> 4;
  constexpr int kCols = MODE == 0 ? kNT * 8 : kNT * 16;   // output columns per wave
  const int col0 = (grp * kWaves + w) * kCols;
  // a wave past the last column still stages rows and meets every barrier
  const bool active = col0 < NB;

  // staging: piece q = tid + kThreads * j is row q / (kSK / 8), 16-byte column
  // q % (kSK / 8) of the stage; rows past the end of the pass repeat its first
  // row (never stored)
  const uint16_t* a_src[kPieces];
  int a_lds[kPieces], a_col[kPieces];
#pragma unroll
  for (int j = 0; j < kPieces; ++j) {
    const int q = tid + kThreads * j;
    const int row = q / (kSK / 8);
    a_col[j] = 8 * (q % (kSK / 8));
    const int p = row0 + row < row_end ? row0 + row : row0;
    const int64_t arow = MODE == 0 ? int64_t(order[p]) : int64_t(p);
    a_src[j] = A + arow * K + a_col[j];
    a_lds[j] = row * kPitch + 2 * a_col[j];
  }
  const uint16_t* b_ptr[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    // gate/up: tile 0 = gate columns, tile 1 = the same columns of up
    int col = MODE == 0 ? col0 + n : col0 + 16 * t + n;
    if (col >= NB) col = NB - 1;                        // partial last group; never stored
    const uint16_t* base = (MODE == 0 && t == 1) ? B1 : B0;
    b_ptr[t] = base + (int64_t(expert) * NB + col) * K + 8 * g;
  }

  f32x4 acc[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int kCPS = kSK / KC;                        // chunks per stage, a multiple of DEPTH
  const int nc = K / KC;
  const int n_st = (K + kSK - 1) / kSK;
  BChunk<KC> ring[DEPTH];                               // chunk c lives in ring[c % DEPTH]
  if (active) {
#pragma unroll
    for (int r = 0; r < DEPTH; ++r)
      if (r < nc) load_chunk(ring[r], b_ptr, r);
  }
  u32x4 stg[kPieces];
#pragma unroll
  for (int j = 0; j < kPieces; ++j)
    if (a_col[j] < K) stg[j] = *reinterpret_cast<const u32x4*>(a_src[j]);
#pragma unroll
  for (int j = 0; j < kPieces; ++j)
    if (a_col[j] < K) *reinterpret_cast<u32x4*>(&sa[0][a_lds[j]]) = stg[j];
  __syncthreads();

  for (int st = 0; st < n_st; ++st) {
    const int k1 = (st + 1) * kSK;                      // first element of the next stage
    if (k1 < K) {
#pragma unroll
      for (int j = 0; j < kPieces; ++j)
        if (k1 + a_col[j] < K) stg[j] = *reinterpret_cast<const u32x4*>(a_src[j] + k1);
    }
    if (active) {
      const unsigned char* arow = sa[st & 1] + n * kPitch + 16 * g;
#pragma unroll
      for (int cc = 0; cc < kCPS; ++cc) {
        const int c = st * kCPS + cc;
        if (c < nc) {                                   // partial last stage (uniform)
          BChunk<KC>& ch = ring[cc % DEPTH];
#pragma unroll
          for (int s = 0; s < KC / 32; ++s) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + (cc * KC + 32 * s) * 2);
#pragma unroll
            for (int t = 0; t < kNT; ++t)
              acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ch.b[t][s], acc[t], 0, 0, 0);
          }
          if (c + DEPTH < nc) load_chunk(ch, b_ptr, c + DEPTH);
        }
      }
    }
    if (k1 < K) {
      // the other buffer was last read in stage st - 1, which every wave has left
#pragma unroll
      for (int j = 0; j < kPieces; ++j)
        if (k1 + a_col[j] < K) *reinterpret_cast<u32x4*>(&sa[(st + 1) & 1][a_lds[j]]) = stg[j];
    }
    __syncthreads();
  }
  if (!active) return;

  // lane holds C[4 g + i][n] of each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pr = row0 + 4 * g + i;
    if (pr >= row_end) continue;
    if (MODE == 0) {
      const int col = col0 + n;
      if (col < NB) C[int64_t(pr) * ldc + col] = f32_to_bf16_rne(silu(acc[0][i]) * acc[1][i]);
    } else if (MODE == 1) {
      const int64_t dst = order[pr];
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        const int col = col0 + 16 * t + n;
        if (col < NB) C[dst * ldc + col] = f32_to_bf16_rne(acc[t][i]);
      }
    } else {
      const int r = order[pr];
      const int q = fc.row_pair ? fc.row_pair[r] : r;
      if (unsigned(q) >= unsigned(fc.n_pairs)) continue;   // a row that holds no pair
      const float wq = fc.topk_w[q];
      float* o = fc.out + int64_t(q / fc.k) * ldc;
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        const int col = col0 + 16 * t + n;
        if (col < NB) unsafeAtomicAdd(o + col, wq * acc[t][i]);
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

namespace {
// column groups of the two products and the worst-case pass count, rounded up
// to a multiple of the XCD count
int64_t groups_gate_up(int64_t ffn) { return (ffn + kWaves * kNT * 8 - 1) / (kWaves * kNT * 8); }
int64_t groups_down(int64_t hidden) { return (hidden + kWaves * kNT * 16 - 1) / (kWaves * kNT * 16); }
int64_t pass_slots(int64_t n_rows, int n_experts) {
  return ((n_rows + kPass - 1) / kPass + n_experts + kXcds - 1) / kXcds * kXcds;
}
}  // namespace

int64_t gather_swiglu_tiles(int64_t n_rows, int n_experts, int64_t hidden, int64_t ffn) {
  const int64_t g1 = groups_gate_up(ffn), g2 = groups_down(hidden);
  return pass_slots(n_rows, n_experts) * (g1 > g2 ? g1 : g2);
}

hipError_t launch_gather_swiglu(const void* rows, int64_t n_rows, int64_t hidden,
                                const int32_t* row_expert, int n_experts, const void* w_gate,
                                const void* w_up, const void* w_down, int64_t ffn, void* y,
                                void* workspace, hipStream_t stream, const FusedCombine* fused) {
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

  const int64_t slots = pass_slots(n_rows, n_experts);
  const FusedCombine none{};
  // 3. gate/up: 128 F columns per workgroup, K = D
  const int g1 = int(groups_gate_up(ffn));
  const dim3 grid1(unsigned(slots * g1));
  const uint16_t* r16 = static_cast<const uint16_t*>(rows);
  const uint16_t* wg = static_cast<const uint16_t*>(w_gate);
  const uint16_t* wu = static_cast<const uint16_t*>(w_up);
  if (hidden % 256 == 0)
    gather_gemm_kernel<0, 256, 2><<<grid1, kThreads, 0, stream>>>(
        r16, int(hidden), order, passes, n_passes, g1, wg, wu, int(ffn), h, int(ffn), none);
  else
    gather_gemm_kernel<0, 128, 4><<<grid1, kThreads, 0, stream>>>(
        r16, int(hidden), order, passes, n_passes, g1, wg, wu, int(ffn), h, int(ffn), none);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  // 4. down: 256 D columns per workgroup, K = F; y stored, or the combine fused
  const int g2 = int(groups_down(hidden));
  const dim3 grid2(unsigned(slots * g2));
  const uint16_t* wd = static_cast<const uint16_t*>(w_down);
  uint16_t* y16 = static_cast<uint16_t*>(y);
  const bool k256 = ffn % 256 == 0;
  if (fused) {
    if (k256)
      gather_gemm_kernel<2, 256, 2><<<grid2, kThreads, 0, stream>>>(
          h, int(ffn), order, passes, n_passes, g2, wd, nullptr, int(hidden), nullptr,
          int(hidden), *fused);
    else
      gather_gemm_kernel<2, 128, 4><<<grid2, kThreads, 0, stream>>>(
          h, int(ffn), order, passes, n_passes, g2, wd, nullptr, int(hidden), nullptr,
          int(hidden), *fused);
  } else if (k256) {
    gather_gemm_kernel<1, 256, 2><<<grid2, kThreads, 0, stream>>>(
        h, int(ffn), order, passes, n_passes, g2, wd, nullptr, int(hidden), y16, int(hidden),
        none);
  } else {
    gather_gemm_kernel<1, 128, 4><<<grid2, kThreads, 0, stream>>>(
        h, int(ffn), order, passes, n_passes, g2, wd, nullptr, int(hidden), y16, int(hidden),
        none);
  }
  return hipGetLastError();
}

}  // namespace moe
