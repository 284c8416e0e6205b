// Routing metadata: the stable by-expert sort of the routed (token, slot) pairs.
//
// The pages describe the GPU sorting tokens before expert compute (Prime Mega
// MoE news item, "Why is MoE training communication-bound?").  Here that sort
// is a counting sort of the flat pair index p = t*K + k, in three launches:
//   1. count:   each block takes a chunk of 2048 pairs and counts them per
//               expert with LDS atomics (counting only; ranks come later), and
//               flags the chunk if it holds an index outside [0, E).
//   2. scan:    one block turns the per-chunk counts into per-chunk bases (an
//               exclusive scan over chunks for every expert), per-expert totals,
//               the expert offsets (exclusive scan over experts) and the
//               per-expert m-tile prefix sums used by the grouped GEMMs.  It
//               also starts the device error word afresh from the chunk flags
//               (the caller's scratch may hold anything).
//   3. scatter: each block re-reads its chunk in order; inside a wavefront the
//               lanes holding the same expert are found with one ballot per
//               expert-id bit, the in-wave rank is the popcount of that match
//               mask below the lane, and the wave's per-expert counts go to LDS
//               so later waves (and later rounds) of the chunk add them.  The
//               result is stable in p and bit-exact.
#include "moe_common.h"

namespace moe {

__global__ void __launch_bounds__(kRouteThreads) route_count_kernel(
    const int32_t* __restrict__ idx, int N, int E, int32_t* __restrict__ chunk_cnt,
    int32_t* __restrict__ chunk_bad) {
  __shared__ int hist[1024];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kRouteChunk;
  bool bad = false;
  for (int i = threadIdx.x; i < kRouteChunk; i += blockDim.x) {
    const int p = base + i;
    if (p < N) {
      const int e = idx[p];
      if (e >= 0 && e < E)
        atomicAdd(&hist[e], 1);
      else
        bad = true;
    }
  }
  const int any_bad = __syncthreads_or(bad);
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    chunk_cnt[size_t(blockIdx.x) * E + e] = hist[e];
  if (threadIdx.x == 0) chunk_bad[blockIdx.x] = any_bad ? 1 : 0;
}

// One block of 1024 threads; thread e owns expert e.  Besides the offsets and
// tile prefixes it writes eorder: the experts by descending token count (ties
// to the lower index), the longest-first order in which the weight-gradient
// GEMMs take their experts, and in eorder[E] a skew flag (the largest count
// above twice the mean) that makes them spread each expert's tiles over all
// XCDs instead of grouping them on one.
__global__ void __launch_bounds__(1024) route_scan_kernel(
    int E, int nchunks, int32_t* __restrict__ chunk_cnt, const int32_t* __restrict__ chunk_bad,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ tiles64,
    int32_t* __restrict__ tiles128, int32_t* __restrict__ tiles256, int32_t* __restrict__ eorder,
    uint32_t* __restrict__ err) {
  __shared__ int sc[4][1024];
  __shared__ int cnt[1024];
  const int e = threadIdx.x;
  int bad = 0;
  for (int b = e; b < nchunks; b += blockDim.x) bad |= chunk_bad[b];
  int total = 0;
  if (e < E) {
    // the chunk counts of expert e, 32 independent loads at a time, the first batch in
    // flight together with the bad-index flags above
    constexpr int kB = 32;
    for (int b0 = 0; b0 < nchunks; b0 += kB) {
      int c[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j) c[j] = b0 + j < nchunks ? chunk_cnt[size_t(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        if (b0 + j < nchunks) chunk_cnt[size_t(b0 + j) * E + e] = total;  // the chunk's base within e
        total += c[j];
      }
    }
    counts[e] = total;
  }
  bad = __syncthreads_or(bad);
  if (e == 0) err[0] = bad ? kErrIndex : 0u;
  // inclusive scans over experts of: count, tiles of 64, 128 and 256 rows
  int v[4];
  v[0] = e < E ? total : 0;
  v[1] = e < E ? (total + 63) / 64 : 0;
  v[2] = e < E ? (total + 127) / 128 : 0;
  v[3] = e < E ? (total + 255) / 256 : 0;
  for (int q = 0; q < 4; ++q) sc[q][e] = v[q];
  cnt[e] = v[0];
  __syncthreads();
  int mx = 0;  // the largest count (every thread, in the ranking loop)
  if (e < E) {
    int rank = 0;
    for (int f = 0; f < E; ++f) {
      const int cf = cnt[f];
      rank += (cf > total || (cf == total && f < e)) ? 1 : 0;
      mx = max(mx, cf);
    }
    eorder[rank] = e;
  }
  for (int step = 1; step < E; step <<= 1) {
    int add[4];
    for (int q = 0; q < 4; ++q) add[q] = e >= step ? sc[q][e - step] : 0;
    __syncthreads();
    for (int q = 0; q < 4; ++q) sc[q][e] += add[q];
    __syncthreads();
  }
  if (e < E) {
    // exclusive value for e is inclusive value minus own
    offsets[e] = sc[0][e] - v[0];
    tiles64[e] = sc[1][e] - v[1];
    tiles128[e] = sc[2][e] - v[2];
    tiles256[e] = sc[3][e] - v[3];
    if (e == E - 1) {
      eorder[E] = (long long)mx * E > 2LL * sc[0][e] ? 1 : 0;
      offsets[E] = sc[0][e];
      tiles64[E] = sc[1][e];
      tiles128[E] = sc[2][e];
      tiles256[E] = sc[3][e];
    }
  }
}

__global__ void __launch_bounds__(kRouteThreads) route_scatter_kernel(
    const int32_t* __restrict__ idx, int N, int E, int nbits,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ pos, int32_t* __restrict__ src, const float* __restrict__ topk_w,
    float* __restrict__ wperm) {
  constexpr int kWaves = kRouteThreads / 64;
  __shared__ int base[1024];
  __shared__ int wcnt[kWaves][1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += kRouteThreads) {
    base[e] = offsets[e] + chunk_base[size_t(blockIdx.x) * E + e];
    for (int w = 0; w < kWaves; ++w) wcnt[w][e] = 0;
  }
  __syncthreads();
  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  for (int round = 0; round < kRouteChunk / kRouteThreads; ++round) {
    const int p = blockIdx.x * kRouteChunk + round * kRouteThreads + tid;
    const int e = p < N ? idx[p] : -1;
    const bool valid = e >= 0 && e < E;
    // lanes holding the same expert id: intersect one ballot per id bit
    uint64_t match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      match &= bit ? m : ~m;
    }
    const int rank = __popcll(match & lt_mask);
    if (valid && rank == 0) wcnt[wave][e] = __popcll(match);
    __syncthreads();
    if (valid) {
      int q = base[e] + rank;
      for (int w = 0; w < wave; ++w) q += wcnt[w][e];
      pos[p] = q;
      src[q] = p;
      if (topk_w != nullptr) wperm[q] = topk_w[p];
    } else if (p < N) {
      pos[p] = -1;
    }
    __syncthreads();
    for (int x = tid; x < E; x += kRouteThreads) {
      int s = 0;
      for (int w = 0; w < kWaves; ++w) {
        s += wcnt[w][x];
        wcnt[w][x] = 0;
      }
      base[x] += s;
    }
    __syncthreads();
  }
}

__global__ void clear_err_kernel(uint32_t* err) {
  if (threadIdx.x == 0) err[0] = 0;
}

int launch_clear_err(char* scratch, const Layout& L, hipStream_t s) {
  prof_begin("clear_err", s);
  clear_err_kernel<<<1, 64, 0, s>>>(reinterpret_cast<uint32_t*>(scratch + L.err));
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int launch_route(const moe_desc& d, const Layout& L, const int32_t* idx, char* scratch,
                 hipStream_t s, const float* topk_w) {
  const int N = d.T * d.K, E = d.E;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  auto* err = reinterpret_cast<uint32_t*>(scratch + L.err);
  auto* chunk = reinterpret_cast<int32_t*>(scratch + L.chunk_cnt);
  auto* bad = reinterpret_cast<int32_t*>(scratch + L.chunk_bad);
  // with no pairs (T = 0) only the scan runs: zero counts and offsets, a clear error word
  if (L.nchunks > 0) {
    prof_begin("route_count", s);
    route_count_kernel<<<L.nchunks, kRouteThreads, 0, s>>>(idx, N, E, chunk, bad);
    prof_end(s);
  }
  prof_begin("route_scan", s);
  route_scan_kernel<<<1, 1024, 0, s>>>(
      E, L.nchunks, chunk, bad, reinterpret_cast<int32_t*>(scratch + L.counts),
      reinterpret_cast<int32_t*>(scratch + L.offsets),
      reinterpret_cast<int32_t*>(scratch + L.tiles[0]),
      reinterpret_cast<int32_t*>(scratch + L.tiles[1]),
      reinterpret_cast<int32_t*>(scratch + L.tiles[2]),
      reinterpret_cast<int32_t*>(scratch + L.eorder), err);
  prof_end(s);
  if (L.nchunks > 0) {
    prof_begin("route_scatter", s);
    route_scatter_kernel<<<L.nchunks, kRouteThreads, 0, s>>>(
        idx, N, E, nbits, chunk, reinterpret_cast<const int32_t*>(scratch + L.offsets),
        reinterpret_cast<int32_t*>(scratch + L.pos), reinterpret_cast<int32_t*>(scratch + L.src),
        topk_w, reinterpret_cast<float*>(scratch + L.wperm));
    prof_end(s);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
