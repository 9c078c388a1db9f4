// Dispatch: per-expert counts, prefix sums, stable position assignment and the
// row copy into expert-major (or segment-major) buffers.
//
// Semantics ("backends/mlx: runtime MoE expert-sort for decode (issue
// #20554)", author's follow-up "Handler fixes" and CI write-up): the routed
// pairs q = t*k + j are the flattened [N, top_k] expert ids; the sorted layout
// is a stable sort of those keys (token = order / top_k), the unsorted layout
// with one segment is the identity (x repeated top_k times).  Segments
// ("One-Sided Expert-Parallel All-to-All ... over NVLink", abstract:
// rank-major blocks) bucket pairs by expert group instead of by expert.
//
// A stable counting sort without global atomics, so positions are
// deterministic:
//   count  -- each chunk of C pairs builds its expert histogram in LDS;
//   rank   -- each chunk reads all [P, E] histograms (L2-resident), scans the
//             expert totals into offsets and forms its starting position in
//             every bucket (bucket-major, chunk-minor order); it recounts per
//             wave, then each wave walks its pairs in order, 64 at a time:
//             ballots over the key bits give every lane the set of lanes with
//             the same bucket, so its rank among earlier equal keys is a
//             popcount (wave multisplit, after Ashkiani et al., "GPU
//             Multisplit", PPoPP 2016);
//   copy   -- scatter form: one wave reads a slice of token t's row once and
//             writes it to the k destination rows dst_pos[t*k + j].
// With a 16-byte payload, rank and copy share one launch: the rank workgroups
// come first in the grid, the copy waves load their slice of x at once and
// then wait only for their own token's k positions.  Each position is its own
// flag: the count launch sets it to a not-ready value, the rank workgroup
// replaces it with an atomic store and the copy wave polls it with atomic
// loads, all relaxed at device scope.  No fence is involved, so no wave
// invalidates or writes back its L2 (the copy's rows stay cached), and the
// copy starts without waiting for the slowest rank workgroup.  Waves are
// dispatched in grid order, so every rank workgroup is resident before any
// copy wave can wait on it; the wait is bounded all the same (a wave that
// gives up flags the status word and skips its stores).
// Small problems (NK <= 4096, at most 256 buckets) run count, scan and rank
// in one workgroup.  Nothing is read back to the host: NK rows is always the
// output size.
#include <mutex>

#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kBlock = 256;
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / kWave;
constexpr int64_t kSmallMaxPairs = 4096;
constexpr int kSmallMaxBuckets = 256;
// dst_pos value of a pair whose position is not yet known (valid values are
// -1 and [0, NK)).
constexpr int32_t kNotReady = INT32_MIN;
// Polls of a copy wave before it gives up by default (each after ~128 cycles
// of sleep and a memory round trip: milliseconds, three orders of magnitude
// above a rank workgroup's run time).
constexpr int kSpinMax = 1 << 18;

__device__ __forceinline__ int bucket_of(int e, int sorted, int per_segment) {
  return sorted ? e : e / per_segment;
}

// Peer mask of this lane: active lanes whose key equals this lane's key.
__device__ __forceinline__ uint64_t peer_mask(int key, bool active, int nbits) {
  uint64_t peers = ballot(active);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool b = (key >> bit) & 1;
    const uint64_t m = ballot(b);
    peers &= b ? m : ~m;
  }
  return peers;
}

// Walk pairs [s0, s1) in order, 64 at a time, assigning positions from the
// per-bucket running counters run[] (LDS, private to this wave).  Keys are
// fetched four steps ahead so their loads overlap.  kPublish: dst_pos is
// written with device-scope atomic stores, for copy waves of the same launch.
template <bool kPublish>
__device__ __forceinline__ void ordered_walk(const int32_t* __restrict__ idx, int64_t s0,
                                             int64_t s1, int n_experts, int sorted,
                                             int per_segment, int nbits, int* run,
                                             int32_t* __restrict__ dst_pos,
                                             int32_t* __restrict__ src_pair,
                                             int32_t* __restrict__ row_expert) {
  constexpr int kAhead = 4;
  const int lane = lane_id();
  for (int64_t qa = s0; qa < s1; qa += kAhead * kWave) {
    int ev[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      const int64_t q = qa + i * kWave + lane;
      ev[i] = q < s1 ? idx[q] : -1;
    }
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      const int64_t q = qa + i * kWave + lane;
      if (qa + i * kWave >= s1) break;                  // uniform
      const bool in = q < s1;
      const int e = ev[i];
      const bool ok = in && unsigned(e) < unsigned(n_experts);
      const int key = ok ? bucket_of(e, sorted, per_segment) : 0;
      const uint64_t peers = peer_mask(key, ok, nbits);
      int pos = 0;
      if (ok) {
        const int rank = __popcll(peers & lanemask_lt());
        pos = run[key] + rank;
        __builtin_amdgcn_wave_barrier();
        if (rank == 0) run[key] = pos + __popcll(peers);
      }
      __builtin_amdgcn_wave_barrier();
      if (in) {
        const int32_t d = ok ? pos : -1;
        if (kPublish) __hip_atomic_store(dst_pos + q, d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else dst_pos[q] = d;
      }
      if (ok) {
        src_pair[pos] = int32_t(q);
        if (row_expert) row_expert[pos] = e;
      }
    }
  }
}

// Per-wave counts of pairs [s0, s1) into cnt[] by bucket (if cnt) and exp[] by
// expert (if exp), with LDS atomics (counts do not depend on order); out-of-
// range ids set *bad.  Ids are fetched four steps ahead.
__device__ __forceinline__ void wave_count(const int32_t* __restrict__ idx, int64_t s0, int64_t s1,
                                           int n_experts, int sorted, int per_segment, int* cnt,
                                           int* exp, bool* bad) {
  constexpr int kAhead = 4;
  const int lane = lane_id();
  for (int64_t qa = s0; qa < s1; qa += kAhead * kWave) {
    int ev[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      const int64_t q = qa + i * kWave + lane;
      ev[i] = q < s1 ? idx[q] : -1;
    }
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      const int64_t q = qa + i * kWave + lane;
      if (q >= s1) continue;
      const int e = ev[i];
      if (unsigned(e) < unsigned(n_experts)) {
        if (cnt) atomicAdd(&cnt[bucket_of(e, sorted, per_segment)], 1);
        if (exp) atomicAdd(&exp[e], 1);
      } else if (bad) {
        *bad = true;
      }
    }
  }
}

// ------------------------------------------------------------------ count
__global__ __launch_bounds__(kBlock) void count_kernel(const int32_t* __restrict__ idx, int64_t nk,
                                                       int n_experts, int chunk,
                                                       int32_t* __restrict__ hist,
                                                       int32_t* status, int identity,
                                                       int32_t* __restrict__ dst_pos,
                                                       int32_t* __restrict__ src_pair,
                                                       int32_t* __restrict__ row_expert,
                                                       int32_t* __restrict__ clear_pos) {
  __shared__ int h[kMaxExperts];
  for (int i = threadIdx.x; i < n_experts; i += kBlock) h[i] = 0;
  __syncthreads();
  const int64_t q0 = int64_t(blockIdx.x) * chunk;
  const int64_t q1 = q0 + chunk < nk ? q0 + chunk : nk;
  bool bad = false;
  constexpr int kAhead = 4;
  for (int64_t qa = q0; qa < q1; qa += kAhead * kBlock) {
    int ev[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      const int64_t q = qa + i * kBlock + threadIdx.x;
      ev[i] = q < q1 ? idx[q] : 0;
    }
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      const int64_t q = qa + i * kBlock + threadIdx.x;
      if (q >= q1) continue;
      const int e = ev[i];
      if (unsigned(e) < unsigned(n_experts)) atomicAdd(&h[e], 1);
      else bad = true;
      if (identity == 1) {                // 2: the routing launch wrote the maps
        dst_pos[q] = int32_t(q);
        src_pair[q] = int32_t(q);
        if (row_expert) row_expert[q] = e;
      }
      if (clear_pos) clear_pos[q] = kNotReady;   // published by the rank+copy launch
    }
  }
  if (bad && status) atomicOr(status, 1);
  __syncthreads();
  int32_t* out = hist + int64_t(blockIdx.x) * n_experts;
  for (int i = threadIdx.x; i < n_experts; i += kBlock) out[i] = h[i];
}

// ------------------------------------------------------------------ row loads
// Token rows are read once per dispatch: non-temporal loads for the 16-byte
// path, plain loads for the narrow fallback types.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_once(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <typename V>
__device__ __forceinline__ V load_once(const V* p) { return *p; }

// An empty asm statement that reads and writes the value's registers: the
// compiler must have the value in registers (its load waited for) at this point.
__device__ __forceinline__ void consume(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}
__device__ __forceinline__ void consume(uint2& v) { asm volatile("" : "+v"(v.x), "+v"(v.y)); }
__device__ __forceinline__ void consume(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void consume(uint16_t& v) {
  uint32_t t = v;
  asm volatile("" : "+v"(t));
  v = uint16_t(t);
}
__device__ __forceinline__ void consume(uint8_t& v) {
  uint32_t t = v;
  asm volatile("" : "+v"(t));
  v = uint8_t(t);
}

// ------------------------------------------------------------------ rank
// Rank of one chunk.  From the [P, E] chunk histograms (L2-resident) it
// derives every expert's total and the count in chunks before its own, scans
// the totals into expert offsets (chunk 0 also writes counts and offsets),
// forms its per-bucket starting positions, recounts per wave and walks its
// pairs in order.
struct RankArgs {
  const int32_t* idx;
  int64_t nk;
  int n_experts, n_segments, chunk, n_chunks, sorted, identity, nbits;
  const int32_t* hist;
  int32_t* counts;
  int32_t* offsets;
  int32_t* seg_offsets;
  int32_t* dst_pos;
  int32_t* src_pair;
  int32_t* row_expert;
};

// LDS of the rank part, carved from dynamic shared memory sized by E and the
// bucket count (7 KB at E = 256, 28 KB at E = 1024).
struct RankLds {
  int* tot;     // [E]
  int* bef;     // [E]
  int* off;     // [E + 1]
  int* wh;      // [waves * buckets]
  int* wave;    // [waves + 1]
};

__host__ __device__ constexpr size_t rank_lds_ints(int n_experts, int n_buckets) {
  return size_t(3) * n_experts + 1 + size_t(kBlock / kWave) * n_buckets + (kBlock / kWave + 1);
}

__device__ __forceinline__ RankLds rank_lds(int* base, int n_experts, int n_buckets) {
  RankLds L;
  L.tot = base;
  L.bef = L.tot + n_experts;
  L.off = L.bef + n_experts;
  L.wh = L.off + n_experts + 1;
  L.wave = L.wh + (kBlock / kWave) * n_buckets;
  return L;
}

template <bool kPublish>
__device__ __forceinline__ void rank_chunk(const RankArgs& r, int me, const RankLds& L) {
  constexpr int kWaves = kBlock / kWave;
  constexpr int kPer = kMaxExperts / kBlock;           // experts per thread in the scan
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int n_experts = r.n_experts, n_chunks = r.n_chunks;
  const int32_t* __restrict__ hist = r.hist;
  const int per = n_experts / r.n_segments;
  const int n_buckets = r.sorted ? n_experts : r.n_segments;

  // 1. totals and before-counts per expert
  for (int e = tid; e < n_experts; e += kBlock) {
    int tot = 0, bef = 0;
    int c = 0;
    for (; c + 32 <= n_chunks; c += 32) {          // 32 loads in flight per thread
      int v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = hist[int64_t(c + i) * n_experts + e];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        tot += v[i];
        bef += (c + i < me) ? v[i] : 0;
      }
    }
    for (; c + 8 <= n_chunks; c += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = hist[int64_t(c + i) * n_experts + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        tot += v[i];
        bef += (c + i < me) ? v[i] : 0;
      }
    }
    for (; c < n_chunks; ++c) {
      const int v = hist[int64_t(c) * n_experts + e];
      tot += v;
      bef += (c < me) ? v : 0;
    }
    L.tot[e] = tot;
    L.bef[e] = bef;
  }
  for (int i = tid; i < kWaves * n_buckets; i += kBlock) L.wh[i] = 0;
  __syncthreads();

  // 2. exclusive scan of the totals: thread i takes experts [i*kPer, i*kPer + kPer)
  int local[kPer];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid * kPer + i;
    local[i] = e < n_experts ? L.tot[e] : 0;
    sum += local[i];
  }
  int total;
  int run = block_exclusive_scan(sum, L.wave, &total);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid * kPer + i;
    if (e < n_experts) L.off[e] = run;
    run += local[i];
  }
  if (tid == 0) L.off[n_experts] = total;
  __syncthreads();
  if (me == 0) {
    for (int e = tid; e < n_experts; e += kBlock) {
      r.counts[e] = L.tot[e];
      r.offsets[e] = L.off[e];
    }
    if (tid == 0) r.offsets[n_experts] = total;
    for (int g = tid; g <= r.n_segments; g += kBlock) r.seg_offsets[g] = L.off[g * per];
  }
  if (r.identity) return;   // the count kernel already wrote the identity maps

  // 3. this chunk's bucket starts (kept in tot, no longer needed)
  if (r.sorted) {
    for (int e = tid; e < n_experts; e += kBlock) L.tot[e] = L.off[e] + L.bef[e];
  } else {
    for (int g = tid; g < r.n_segments; g += kBlock) {
      int b = L.off[g * per];
      for (int e = g * per; e < (g + 1) * per; ++e) b += L.bef[e];
      L.tot[g] = b;
    }
  }

  // 4. per-wave counts of this chunk, then per-wave starts
  const int64_t q0 = int64_t(me) * r.chunk;
  const int64_t q1 = q0 + r.chunk < r.nk ? q0 + r.chunk : r.nk;
  const int sub = (r.chunk + kWaves - 1) / kWaves;
  const int64_t s0 = q0 + int64_t(w) * sub < q1 ? q0 + int64_t(w) * sub : q1;
  const int64_t s1 = s0 + sub < q1 ? s0 + sub : q1;
  int* mine = L.wh + w * n_buckets;
  wave_count(r.idx, s0, s1, n_experts, r.sorted, per, mine, nullptr, nullptr);
  __syncthreads();
  for (int b = tid; b < n_buckets; b += kBlock) {
    int rr = L.tot[b];
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const int c = L.wh[ww * n_buckets + b];
      L.wh[ww * n_buckets + b] = rr;
      rr += c;
    }
  }
  __syncthreads();
  ordered_walk<kPublish>(r.idx, s0, s1, n_experts, r.sorted, per, r.nbits, mine, r.dst_pos,
                         r.src_pair, r.row_expert);
}

// Block p ranks chunk p.
__global__ __launch_bounds__(kBlock) void rank_kernel(RankArgs r) {
  extern __shared__ int lds[];
  rank_chunk<false>(r, blockIdx.x, rank_lds(lds, r.n_experts, r.sorted ? r.n_experts : r.n_segments));
}

// ------------------------------------------------------------------ small problems
__global__ __launch_bounds__(kSmallThreads) void small_meta_kernel(
    const int32_t* __restrict__ idx, int64_t nk, int n_experts, int n_segments, int sorted,
    int nbits, int identity, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ seg_offsets, int32_t* __restrict__ dst_pos,
    int32_t* __restrict__ src_pair, int32_t* __restrict__ row_expert, int32_t* status) {
  __shared__ int h[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int wh[kSmallWaves * kSmallMaxBuckets];
  __shared__ int s_wave[17];
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int lane = lane_id();
  const int per = n_experts / n_segments;
  const int n_buckets = sorted ? n_experts : n_segments;
  for (int i = tid; i < n_experts; i += kSmallThreads) h[i] = 0;
  if (!identity)
    for (int i = tid; i < kSmallWaves * n_buckets; i += kSmallThreads) wh[i] = 0;
  __syncthreads();

  // wave w owns pairs [s0, s1), a multiple of 64 long
  const int64_t sub = ((nk + kSmallWaves - 1) / kSmallWaves + kWave - 1) / kWave * kWave;
  const int64_t s0 = int64_t(w) * sub < nk ? int64_t(w) * sub : nk;
  const int64_t s1 = s0 + sub < nk ? s0 + sub : nk;
  int* mine = wh + w * n_buckets;
  bool bad = false;
  if (identity == 1) {                  // 2: the routing launch wrote the maps
    for (int64_t q = s0 + lane; q < s1; q += kWave) {
      dst_pos[q] = int32_t(q);
      src_pair[q] = int32_t(q);
      if (row_expert) row_expert[q] = idx[q];
    }
  }
  wave_count(idx, s0, s1, n_experts, sorted, per, identity ? nullptr : mine, h, &bad);
  if (bad && status) atomicOr(status, 1);
  __syncthreads();

  const int c = tid < n_experts ? h[tid] : 0;
  int total;
  const int excl = block_exclusive_scan(c, s_wave, &total);
  if (tid < n_experts) {
    counts[tid] = c;
    offsets[tid] = excl;
    s_off[tid] = excl;
  }
  if (tid == 0) {
    offsets[n_experts] = total;
    s_off[n_experts] = total;
  }
  __syncthreads();
  for (int i = tid; i <= n_segments; i += blockDim.x) seg_offsets[i] = s_off[i * per];
  if (identity) return;

  for (int b = tid; b < n_buckets; b += kSmallThreads) {
    int run = s_off[sorted ? b : b * per];
    for (int ww = 0; ww < kSmallWaves; ++ww) {
      const int cc = wh[ww * n_buckets + b];
      wh[ww * n_buckets + b] = run;
      run += cc;
    }
  }
  __syncthreads();
  ordered_walk<false>(idx, s0, s1, n_experts, sorted, per, nbits, mine, dst_pos, src_pair,
                      row_expert);
}

// ------------------------------------------------------------------ N == 0
__global__ void zero_offsets_kernel(int n_experts, int n_segments, int32_t* counts,
                                    int32_t* offsets, int32_t* seg_offsets) {
  for (int i = threadIdx.x; i <= n_experts; i += blockDim.x) {
    if (i < n_experts) counts[i] = 0;
    offsets[i] = 0;
    if (i <= n_segments) seg_offsets[i] = 0;
  }
}

// ------------------------------------------------------------------ row copy
// One wave per (token, slice) item; each lane moves U vectors of type V.  The
// loads use clamped (always valid) indices so they issue back to back.  Lane
// j < k holds destination j (read with readlane).
template <typename V, int U>
__global__ __launch_bounds__(kBlock) void scatter_rows_kernel(const V* __restrict__ x,
                                                              int64_t n_tokens, int64_t nvec,
                                                              int k, int n_slices,
                                                              const int32_t* __restrict__ dst_pos,
                                                              int64_t nk, V* __restrict__ rows) {
  const int lane = lane_id();
  const int64_t item = __builtin_amdgcn_readfirstlane(int(blockIdx.x)) * int64_t(kBlock / kWave) +
                       __builtin_amdgcn_readfirstlane(int(threadIdx.x / kWave));
  const int64_t t = item / n_slices;
  if (t >= n_tokens) return;
  const int64_t v0 = (item - t * n_slices) * int64_t(kWave * U) + lane;
  const int my_p = lane < k ? dst_pos[t * k + lane] : -1;
  const V* src = x + t * nvec;
  // Lanes past the end of the row take index nvec - 1: they load and store the
  // same value as the lane that owns it, so no store needs a predicate.
  V buf[U];
  int64_t vi[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    vi[u] = v0 + u * kWave < nvec ? v0 + u * kWave : nvec - 1;
    buf[u] = load_once(src + vi[u]);
  }
  // Consume the loaded registers once here so the loads are waited for before
  // the store loop; otherwise the wait lands inside the loop, where it would
  // also wait for the previous destination's stores (vmcnt counts both).
#pragma unroll
  for (int u = 0; u < U; ++u) consume(buf[u]);
  for (int j = 0; j < k; ++j) {
    const int p = __builtin_amdgcn_readlane(my_p, j);
    if (unsigned(p) >= uint64_t(nk)) continue;
    V* dst = rows + int64_t(p) * nvec;
#pragma unroll
    for (int u = 0; u < U; ++u) dst[vi[u]] = buf[u];
  }
}

// 16-byte payload rows and, for fp8 workloads, their block-scale rows: items
// [0, n_tokens * n_slices_a) copy payload slices, the rest (n_slices_b per
// token, 0 without scales) copy scale rows.
struct PairCopy {
  const uint4* xa;
  int64_t nvec_a;
  int n_slices_a;
  uint4* rows_a;
  const uint4* xb;
  int64_t nvec_b;
  int n_slices_b;
  uint4* rows_b;
  int64_t n_tokens;
  int k;
  int64_t nk;
  int spin_max;          // polls before a waiting copy wave gives up
};

// Lane j < k: dst_pos[t*k + j] read with a device-scope atomic load (other
// lanes -1).
__device__ __forceinline__ int32_t poll_position(const int32_t* dst_pos, int64_t t, int k) {
  const int lane = lane_id();
  return lane < k ? __hip_atomic_load(dst_pos + t * k + lane, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT)
                  : -1;
}

// Poll until no lane holds kNotReady, sleeping between polls; after spin_max
// polls the lanes still waiting give -1 (their rows are skipped) and the
// status word, if any, gets bit 2.  The loop condition is a ballot, so the
// wave leaves it together.
__device__ __forceinline__ int32_t wait_position(int32_t p, const int32_t* dst_pos, int64_t t,
                                                 int k, int32_t* status, int spin_max) {
  for (int it = 0; ballot(p == kNotReady) != 0; ++it) {
    if (it >= spin_max) {
      if (status && lane_id() == 0) atomicOr(status, 2);
      return p == kNotReady ? -1 : p;
    }
    __builtin_amdgcn_s_sleep(2);
    if (p == kNotReady) p = poll_position(dst_pos, t, k);
  }
  return p;
}

// One (token, slice) item.  kWait: the positions are published by rank
// workgroups of the same launch.
template <int U, bool kWait>
__device__ __forceinline__ void pair_copy(const PairCopy& c, int64_t item,
                                          const int32_t* __restrict__ dst_pos, int32_t* status) {
  const int lane = lane_id();
  const int64_t items_a = c.n_tokens * c.n_slices_a;
  const bool second = item >= items_a;       // wave-uniform
  if (second && c.n_slices_b == 0) return;
  const uint4* x = second ? c.xb : c.xa;
  uint4* rows = second ? c.rows_b : c.rows_a;
  const int64_t nvec = second ? c.nvec_b : c.nvec_a;
  const int n_slices = second ? c.n_slices_b : c.n_slices_a;
  if (second) item -= items_a;
  const int64_t t = item / n_slices;
  if (t >= c.n_tokens) return;
  const int k = c.k;
  const int64_t v0 = (item - t * n_slices) * int64_t(kWave * U) + lane;
  int32_t my_p = kWait ? poll_position(dst_pos, t, k) : (lane < k ? dst_pos[t * k + lane] : -1);
  const uint4* src = x + t * nvec;
  uint4 buf[U];
  int64_t vi[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    vi[u] = v0 + u * kWave < nvec ? v0 + u * kWave : nvec - 1;
    buf[u] = load_once(src + vi[u]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) consume(buf[u]);
  if (kWait) my_p = wait_position(my_p, dst_pos, t, k, status, c.spin_max);
  for (int j = 0; j < k; ++j) {
    const int p = __builtin_amdgcn_readlane(my_p, j);
    if (unsigned(p) >= uint64_t(c.nk)) continue;
    uint4* dst = rows + int64_t(p) * nvec;
#pragma unroll
    for (int u = 0; u < U; ++u) dst[vi[u]] = buf[u];
  }
}

template <int U>
__global__ __launch_bounds__(kBlock) void scatter_pair_kernel(PairCopy c,
                                                              const int32_t* __restrict__ dst_pos) {
  const int64_t item = __builtin_amdgcn_readfirstlane(int(blockIdx.x)) * int64_t(kBlock / kWave) +
                       __builtin_amdgcn_readfirstlane(int(threadIdx.x / kWave));
  pair_copy<U, false>(c, item, dst_pos, nullptr);
}

// Rank and copy in one launch: blocks [0, P) rank chunk blockIdx.x and
// publish its positions; the blocks after them copy (token, slice) items.
template <int U>
__global__ __launch_bounds__(kBlock) void rank_scatter_kernel(RankArgs r, PairCopy c,
                                                              int32_t* status) {
  extern __shared__ int lds[];
  const int b = __builtin_amdgcn_readfirstlane(int(blockIdx.x));
  if (b < r.n_chunks) {
    rank_chunk<true>(r, b, rank_lds(lds, r.n_experts, r.sorted ? r.n_experts : r.n_segments));
    return;
  }
  const int64_t item = int64_t(b - r.n_chunks) * (kBlock / kWave) +
                       __builtin_amdgcn_readfirstlane(int(threadIdx.x / kWave));
  pair_copy<U, true>(c, item, r.dst_pos, status);
}

template <typename V>
hipError_t launch_scatter_typed(const void* x, int64_t n_tokens, int64_t row_bytes, int k,
                                const int32_t* dst_pos, int64_t nk, void* rows,
                                hipStream_t stream) {
  constexpr int U = 2;
  const int64_t nvec = row_bytes / int64_t(sizeof(V));
  const int n_slices = int((nvec + kWave * U - 1) / (kWave * U));
  const int64_t items = n_tokens * n_slices;
  const int per_block = kBlock / kWave;
  const dim3 grid(unsigned((items + per_block - 1) / per_block));
  scatter_rows_kernel<V, U><<<grid, kBlock, 0, stream>>>(
      static_cast<const V*>(x), n_tokens, nvec, k, n_slices, dst_pos, nk, static_cast<V*>(rows));
  return hipGetLastError();
}

hipError_t launch_scatter(const void* x, int64_t n_tokens, int64_t row_bytes, int k,
                          const int32_t* dst_pos, int64_t nk, void* rows, hipStream_t stream) {
  // widest access that divides the row size and both base addresses
  const uint64_t align = uint64_t(row_bytes) | reinterpret_cast<uintptr_t>(x) |
                         reinterpret_cast<uintptr_t>(rows);
  if ((align & 15) == 0) return launch_scatter_typed<uint4>(x, n_tokens, row_bytes, k, dst_pos, nk, rows, stream);
  if ((align & 7) == 0) return launch_scatter_typed<uint2>(x, n_tokens, row_bytes, k, dst_pos, nk, rows, stream);
  if ((align & 3) == 0) return launch_scatter_typed<uint32_t>(x, n_tokens, row_bytes, k, dst_pos, nk, rows, stream);
  if ((align & 1) == 0) return launch_scatter_typed<uint16_t>(x, n_tokens, row_bytes, k, dst_pos, nk, rows, stream);
  return launch_scatter_typed<uint8_t>(x, n_tokens, row_bytes, k, dst_pos, nk, rows, stream);
}

// Gather form: one wave per (row, slice) item, rows[p] = x[src_pair[p] / k].
template <typename V, int U>
__global__ __launch_bounds__(kBlock) void gather_rows_kernel(const V* __restrict__ x,
                                                             int64_t n_tokens, int64_t nvec,
                                                             int k, int n_slices,
                                                             const int32_t* __restrict__ src_pair,
                                                             int64_t n_rows, V* __restrict__ rows) {
  const int lane = lane_id();
  const int64_t item = __builtin_amdgcn_readfirstlane(int(blockIdx.x)) * int64_t(kBlock / kWave) +
                       __builtin_amdgcn_readfirstlane(int(threadIdx.x / kWave));
  const int64_t p = item / n_slices;
  if (p >= n_rows) return;
  const int64_t v0 = (item - p * n_slices) * int64_t(kWave * U) + lane;
  const int q = src_pair[p];
  if (q < 0 || int64_t(q) / k >= n_tokens) return;
  const V* src = x + (int64_t(q) / k) * nvec;
  V* dst = rows + p * nvec;
  V buf[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (v0 + u * kWave < nvec) buf[u] = src[v0 + u * kWave];
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (v0 + u * kWave < nvec) dst[v0 + u * kWave] = buf[u];
}

template <typename V>
hipError_t launch_gather_typed(const void* x, int64_t n_tokens, int64_t row_bytes, int k,
                               const int32_t* src_pair, int64_t n_rows, void* rows,
                               hipStream_t stream) {
  constexpr int U = 2;
  const int64_t nvec = row_bytes / int64_t(sizeof(V));
  const int n_slices = int((nvec + kWave * U - 1) / (kWave * U));
  const int64_t items = n_rows * n_slices;
  const int per_block = kBlock / kWave;
  const dim3 grid(unsigned((items + per_block - 1) / per_block));
  gather_rows_kernel<V, U><<<grid, kBlock, 0, stream>>>(
      static_cast<const V*>(x), n_tokens, nvec, k, n_slices, src_pair, n_rows, static_cast<V*>(rows));
  return hipGetLastError();
}

int bits_for(int n) {
  int b = 0;
  while ((1 << b) < n) ++b;
  return b;
}

}  // namespace

DispatchPlan plan_dispatch(int64_t n_tokens, int n_experts, int k, int n_segments) {
  DispatchPlan p{};
  p.nk = n_tokens * k;
  // about 64 chunks (more rank workgroups, shorter in-order walks), 256 to 1024
  // pairs each; beyond a million pairs, about 1024 chunks
  int64_t chunk = ((p.nk + 63) / 64 + 255) / 256 * 256;
  if (chunk > 1024) chunk = 1024;
  if (chunk < 256) chunk = 256;
  if (p.nk > int64_t(1024) * 1024) chunk = ((p.nk + 1023) / 1024 + 255) / 256 * 256;
  p.chunk = int(chunk);
  p.n_chunks = int((p.nk + chunk - 1) / chunk);
  p.small = p.nk <= kSmallMaxPairs && n_experts <= kSmallMaxBuckets ? 1 : 0;
  (void)n_segments;
  return p;
}

size_t dispatch_workspace_bytes(int64_t n_tokens, int n_experts, int k, int n_segments) {
  const DispatchPlan p = plan_dispatch(n_tokens, n_experts, k, n_segments);
  const size_t cells = size_t(p.n_chunks > 0 ? p.n_chunks : 1) * size_t(n_experts);
  return cells * sizeof(int32_t) + 256;
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream) {
  const DispatchPlan p = plan_dispatch(a.n_tokens, a.n_experts, a.k, a.n_segments);
  if (p.nk == 0) {
    zero_offsets_kernel<<<1, 256, 0, stream>>>(a.n_experts, a.n_segments, a.expert_counts,
                                               a.expert_offsets, a.segment_offsets);
    return hipGetLastError();
  }
  // identity layout: 1, or 2 when the routing launch already wrote its maps
  const int identity = (!a.sorted && a.n_segments == 1) ? (a.maps_done ? 2 : 1) : 0;
  const int n_buckets = a.sorted ? a.n_experts : a.n_segments;
  const int nbits = bits_for(n_buckets);
  const size_t rank_lds = rank_lds_ints(a.n_experts, n_buckets) * sizeof(int);

  // 16-byte payload (and scale) rows: the copy can share the rank launch
  constexpr int U = 2;
  PairCopy c{};
  bool wide = false;
  if (a.x) {
    uint64_t align = uint64_t(a.row_bytes) | reinterpret_cast<uintptr_t>(a.x) |
                     reinterpret_cast<uintptr_t>(a.rows);
    if (a.x_scales)
      align |= uint64_t(a.scale_bytes) | reinterpret_cast<uintptr_t>(a.x_scales) |
               reinterpret_cast<uintptr_t>(a.row_scales);
    wide = (align & 15) == 0;
    if (wide) {
      c.xa = static_cast<const uint4*>(a.x);
      c.nvec_a = a.row_bytes / 16;
      c.n_slices_a = int((c.nvec_a + kWave * U - 1) / (kWave * U));
      c.rows_a = static_cast<uint4*>(a.rows);
      if (a.x_scales) {
        c.xb = reinterpret_cast<const uint4*>(a.x_scales);
        c.nvec_b = a.scale_bytes / 16;
        c.n_slices_b = int((c.nvec_b + kWave * U - 1) / (kWave * U));
        c.rows_b = reinterpret_cast<uint4*>(a.row_scales);
      }
      c.n_tokens = a.n_tokens;
      c.k = a.k;
      c.nk = p.nk;
      c.spin_max = a.spin_limit >= 0 ? a.spin_limit : kSpinMax;
    }
  }
  const int per_block = kBlock / kWave;
  const int64_t copy_blocks =
      wide ? (a.n_tokens * (c.n_slices_a + c.n_slices_b) + per_block - 1) / per_block : 0;
  // rank + copy in one launch: general layouts, rank LDS small enough not to
  // limit the copy's occupancy
  const bool fused = wide && !identity && !p.small && rank_lds <= 16384 &&
                     p.n_chunks + copy_blocks <= int64_t(INT32_MAX);

  if (p.small) {
    small_meta_kernel<<<1, kSmallThreads, 0, stream>>>(
        a.topk_idx, p.nk, a.n_experts, a.n_segments, a.sorted, nbits, identity, a.expert_counts,
        a.expert_offsets, a.segment_offsets, a.dst_pos, a.src_pair, a.row_expert, a.status);
  } else {
    int32_t* hist = static_cast<int32_t*>(a.workspace);
    count_kernel<<<p.n_chunks, kBlock, 0, stream>>>(a.topk_idx, p.nk, a.n_experts, p.chunk, hist,
                                                    a.status, identity, a.dst_pos, a.src_pair,
                                                    a.row_expert, fused ? a.dst_pos : nullptr);
    // identity layout: only block 0's offsets are needed
    const RankArgs r{a.topk_idx, p.nk, a.n_experts, a.n_segments, p.chunk, p.n_chunks, a.sorted,
                     identity, nbits, hist, a.expert_counts, a.expert_offsets, a.segment_offsets,
                     a.dst_pos, a.src_pair, a.row_expert};
    if (fused) {
      rank_scatter_kernel<U><<<unsigned(p.n_chunks + copy_blocks), kBlock, rank_lds, stream>>>(
          r, c, a.status);
      return hipGetLastError();
    }
    rank_kernel<<<identity ? 1 : p.n_chunks, kBlock, rank_lds, stream>>>(r);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (wide) {                      // payload and scales in one launch
    scatter_pair_kernel<U><<<unsigned(copy_blocks), kBlock, 0, stream>>>(c, a.dst_pos);
    return hipGetLastError();
  }
  if (a.x) {
    err = launch_scatter(a.x, a.n_tokens, a.row_bytes, a.k, a.dst_pos, p.nk, a.rows, stream);
    if (err != hipSuccess) return err;
  }
  if (a.x_scales) {
    err = launch_scatter(a.x_scales, a.n_tokens, a.scale_bytes, a.k, a.dst_pos, p.nk,
                         a.row_scales, stream);
  }
  return err;
}

size_t route_dispatch_workspace_bytes(int64_t n_tokens, int n_experts, int k, int n_segments) {
  return dispatch_workspace_bytes(n_tokens, n_experts, k, n_segments);
}

// ------------------------------------------------------------------ allocation-free scratch
// The workspace of moe_route_dispatch_noalloc: one copy of this array per GPU,
// alive until the process ends.  Host code never passes `scratch` itself to a
// kernel (on the host it names a stand-in, not the device copy): the device
// address is looked up once per device with hipGetSymbolAddress and kept.
namespace {
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
  *ptr = nullptr;
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream) {                      // the kernels run on the stream's device
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess) return e;
    dev = int(sd);
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_route_dispatch(const RouteArgs& r, const DispatchArgs& a, hipStream_t stream) {
  if (a.n_tokens > 0) {
    // identity layout (unsorted, one segment): the row copy needs nothing from
    // the routing, so both run in one launch and only the maps follow
    const bool identity = !a.sorted && a.n_segments == 1;
    const uint64_t align = uint64_t(a.row_bytes) | reinterpret_cast<uintptr_t>(a.x) |
                           reinterpret_cast<uintptr_t>(a.rows);
    if (identity && a.x && !a.x_scales && (align & 15) == 0) {
      hipError_t err = launch_route_copy_identity(r.logits, a.n_tokens, a.n_experts, a.k,
                                                  r.renormalize, const_cast<int32_t*>(a.topk_idx),
                                                  r.topk_w, a.x, a.row_bytes, a.rows, a.dst_pos,
                                                  a.src_pair, a.row_expert, stream);
      if (err != hipSuccess) return err;
      DispatchArgs maps = a;
      maps.x = nullptr;                     // rows and maps are already in place
      maps.maps_done = 1;
      return launch_dispatch(maps, stream);
    }
    hipError_t err = launch_route_topk(r.logits, a.n_tokens, a.n_experts, a.k, r.renormalize,
                                       const_cast<int32_t*>(a.topk_idx), r.topk_w, stream);
    if (err != hipSuccess) return err;
  }
  return launch_dispatch(a, stream);
}

hipError_t launch_scatter_rows(const void* x, int64_t n_tokens, int64_t row_bytes, int k,
                               const int32_t* dst_pos, void* rows, hipStream_t stream) {
  return launch_scatter(x, n_tokens, row_bytes, k, dst_pos, n_tokens * k, rows, stream);
}

hipError_t launch_gather_rows(const void* x, int64_t n_tokens, int64_t row_bytes, int k,
                              const int32_t* src_pair, int64_t n_rows, void* rows,
                              hipStream_t stream) {
  const uint64_t align = uint64_t(row_bytes) | reinterpret_cast<uintptr_t>(x) |
                         reinterpret_cast<uintptr_t>(rows);
  if ((align & 15) == 0) return launch_gather_typed<uint4>(x, n_tokens, row_bytes, k, src_pair, n_rows, rows, stream);
  if ((align & 7) == 0) return launch_gather_typed<uint2>(x, n_tokens, row_bytes, k, src_pair, n_rows, rows, stream);
  if ((align & 3) == 0) return launch_gather_typed<uint32_t>(x, n_tokens, row_bytes, k, src_pair, n_rows, rows, stream);
  if ((align & 1) == 0) return launch_gather_typed<uint16_t>(x, n_tokens, row_bytes, k, src_pair, n_rows, rows, stream);
  return launch_gather_typed<uint8_t>(x, n_tokens, row_bytes, k, src_pair, n_rows, rows, stream);
}

}  // namespace moe
