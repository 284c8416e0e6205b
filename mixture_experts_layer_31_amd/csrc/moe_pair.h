// Two independent GEMMs of the backward in one launch: a token-grouped GEMM
// (its "A items" are the output tiles of one expert's rows) and a per-expert
// weight gradient ("B items": the tiles of dW[e]).  W2 dgrad + SwiGLU-backward
// runs beside the W2 weight gradient, and the W1 dgrad beside the W1 weight
// gradient.  Neither GEMM reads what the other writes, so no item ever waits:
// the point is that tiles of both kinds share the chip, so the HBM-heavy
// epilogues of one overlap the matrix-core main loops of the other instead of
// running in lock-step phases, and one tail replaces two.
//
// Schedule.  The items form one list in the experts' longest-first order
// (routing's eorder): for each expert its B tiles, then its A tiles (the dgrad
// then finds the token rows both read, dY or dH, in the caches: W2 pair -1.5%
// and W1 pair -0.4% at the 30B shape, both -0.4% at 235B, against A tiles
// first; spreading the A tiles evenly among the B tiles measured 1-2% slower:
// it splits the expert's A tiles, which share the weight slices, over more of
// the XCD's workgroup slots).  The list
// is cut into 8 contiguous ranges of about equal estimated cost (an A tile
// costs its contraction length, a B tile its expert's token count, both plus
// an epilogue share), one per XCD queue; workgroup b takes tickets from queue
// b % 8 (where round-robin dispatch places it, so an expert's items share that
// XCD's L2) through an atomic counter, and when its queue is exhausted it takes
// tickets from the next queues in turn, so no queue's tail waits for its own
// workgroups.  Every workgroup computes the cost prefix and the cut points
// itself (a block scan over the experts) at the start.  A workgroup that finds
// every queue exhausted exits; since no item waits, every item that has been
// ticketed completes whether or not all workgroups are resident.
#pragma once

#include "moe_gemm_common.h"

namespace moe {
namespace gemm {

constexpr int kPairQueues = 8;
constexpr int kPairMaxE = 256;  // experts of a paired launch (its schedule lives in LDS)
constexpr int kPairEpilogueCost = 256;  // cost units (contraction elements) of one epilogue

struct PairSched {
  const int32_t* offsets;  // [E+1] first permuted row of each expert
  const int32_t* tstart;   // [E+1] prefix of the A GEMM's m-tiles per expert
  const int32_t* eorder;   // [E+1] experts longest first
  int E;
  int ntn;                 // n-tiles of the A GEMM per m-tile
  int per_b;               // B tiles per expert
  int cost_a;              // contraction length of an A tile
  int* ctr;                // [kPairQueues] ticket counters, zero at launch
};

// LDS of the schedule (placed after the tiles' pipeline LDS).
struct PairLds {
  int items[kPairMaxE + 1];   // exclusive prefix of items per rank
  float cost[kPairMaxE + 1];  // exclusive prefix of cost per rank
  int bound[kPairQueues + 1]; // first item of each queue
  int wsum_i[16], slot;
  float wsum_c[16];
};

// Items and cost of the expert of rank r.
__device__ __forceinline__ void pair_rank(const PairSched& s, int r, int& n_items, float& cost) {
  const int e = s.eorder[r];
  const int na = (s.tstart[e + 1] - s.tstart[e]) * s.ntn;
  const int ne = s.offsets[e + 1] - s.offsets[e];
  n_items = na + s.per_b;
  cost = float(na) * float(s.cost_a + kPairEpilogueCost) +
         float(s.per_b) * float(ne + kPairEpilogueCost);
}

// Builds the item and cost prefixes and the queue bounds in LDS (whole workgroup).
template <int THREADS>
__device__ __forceinline__ void pair_setup(const PairSched& s, PairLds& L) {
  static_assert(THREADS % 64 == 0 && THREADS * 2 >= kPairMaxE && THREADS / 64 <= 16,
                "two ranks per thread, at most 16 waves");
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  // ranks 2t and 2t + 1
  int i0 = 0, i1 = 0;
  float c0 = 0.f, c1 = 0.f;
  if (2 * t < s.E) pair_rank(s, 2 * t, i0, c0);
  if (2 * t + 1 < s.E) pair_rank(s, 2 * t + 1, i1, c1);
  // inclusive scan of the pair sums over the wave, then over the waves
  int si = i0 + i1;
  float sc = c0 + c1;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int oi = __shfl_up(si, d, 64);
    const float oc = __shfl_up(sc, d, 64);
    if (lane >= d) {
      si += oi;
      sc += oc;
    }
  }
  if (lane == 63) {
    L.wsum_i[w] = si;
    L.wsum_c[w] = sc;
  }
  __syncthreads();
  int bi = 0;
  float bc = 0.f;
  for (int v = 0; v < w; ++v) {
    bi += L.wsum_i[v];
    bc += L.wsum_c[v];
  }
  const int ex_i = bi + si - (i0 + i1);  // exclusive prefix before rank 2t
  const float ex_c = bc + sc - (c0 + c1);
  if (2 * t < s.E) {
    L.items[2 * t] = ex_i;
    L.cost[2 * t] = ex_c;
  }
  if (2 * t + 1 < s.E) {
    L.items[2 * t + 1] = ex_i + i0;
    L.cost[2 * t + 1] = ex_c + c0;
  }
  if (t == 0) {  // the totals
    int ti = 0;
    float tc = 0.f;
    for (int v = 0; v < THREADS / 64; ++v) {
      ti += L.wsum_i[v];
      tc += L.wsum_c[v];
    }
    L.items[s.E] = ti;
    L.cost[s.E] = tc;
  }
  __syncthreads();
  // queue q's first item: where the cost prefix reaches q / 8 of the total
  if (t <= kPairQueues) {
    const int total = L.items[s.E];
    int b = 0;
    if (t == kPairQueues) {
      b = total;
    } else if (t > 0) {
      const float target = L.cost[s.E] * float(t) / float(kPairQueues);
      int lo = 0, hi = s.E;  // last rank whose prefix is <= target
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (L.cost[mid] <= target) lo = mid; else hi = mid;
      }
      const int e = s.eorder[lo];
      const int ne = s.offsets[e + 1] - s.offsets[e];
      const float ca = float(s.cost_a + kPairEpilogueCost), cb = float(ne + kPairEpilogueCost);
      const float rem = target - L.cost[lo];
      int i;
      if (rem <= float(s.per_b) * cb) i = int(ceilf(rem / cb));
      else i = s.per_b + int(ceilf((rem - float(s.per_b) * cb) / ca));
      b = min(L.items[lo] + max(i, 0), L.items[lo + 1]);
    }
    L.bound[t] = b;
  }
  __syncthreads();
  // the bounds must not decrease (rounding of the float prefix aside)
  if (t == 0)
    for (int q = 1; q <= kPairQueues; ++q) L.bound[q] = max(L.bound[q], L.bound[q - 1]);
  __syncthreads();
}

// Next item of this workgroup (or -1 when every queue is exhausted), starting
// at queue *q and moving on to the following queues when one runs dry.  *q is
// thread 0's state (only thread 0 takes tickets).
__device__ __forceinline__ int pair_next(const PairSched& s, PairLds& L, int* q) {
  if (threadIdx.x == 0) {
    int item = -1;
    for (int k = 0; k < kPairQueues && item < 0; ++k) {
      const int qq = (*q + k) % kPairQueues;
      const int n = L.bound[qq + 1] - L.bound[qq];
      if (n <= 0) continue;
      const int t = __hip_atomic_fetch_add(s.ctr + qq, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (t < n) {
        item = L.bound[qq] + t;
        *q = qq;
      }
    }
    L.slot = item;
  }
  __syncthreads();
  const int item = __builtin_amdgcn_readfirstlane(L.slot);
  __syncthreads();  // the slot is rewritten by the next call
  return item;
}

// Which GEMM and which of its flat tile indices item g is: item i of the
// expert of rank r is, for i < per_b, tile r * per_b + i of the weight gradient
// (which maps rank r back to its expert through eorder), else flat tile
// tstart[e] * ntn + (i - per_b) of the token-grouped GEMM.
struct PairItem { bool is_a; int l; };
__device__ __forceinline__ PairItem pair_decode(const PairSched& s, const PairLds& L, int g) {
  int lo = 0, hi = s.E;  // last rank whose first item is <= g
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (L.items[mid] <= g) lo = mid; else hi = mid;
  }
  const int e = s.eorder[lo];
  const int i = g - L.items[lo];
  PairItem it;
  it.is_a = i >= s.per_b;
  it.l = it.is_a ? s.tstart[e] * s.ntn + (i - s.per_b) : lo * s.per_b + i;
  it.is_a = __builtin_amdgcn_readfirstlane(it.is_a ? 1 : 0) != 0;
  it.l = __builtin_amdgcn_readfirstlane(it.l);
  return it;
}

}  // namespace gemm
}  // namespace moe
