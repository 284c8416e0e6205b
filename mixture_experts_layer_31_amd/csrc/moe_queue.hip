// Overlapped forward: dispatch, W1 + SwiGLU and W2 in one launch, ordered by
// per-XCD ticket queues.
//
// The pages overlap the arrival of tokens with expert compute: the kernel
// computes on a group of tokens as soon as that group has arrived, keeping
// intermediates in GPU scratch buffers (Prime Mega MoE news item, "How does the
// fused kernel work?").  On one GPU the "arrival" is the local permute, so the
// same schedule here overlaps the (HBM-bound) dispatch with the (matrix-core-
// bound) expert GEMMs, and lets the W2 tiles of early experts fill the tail of
// the W1 GEMM.
//
// Partition: the expert-major list of 256-row m-tiles is cut into 8 contiguous
// ranges, one per XCD (workgroup b takes its tickets from queue b % 8, and
// round-robin dispatch places it on XCD b % 8, so an expert's tiles share one
// L2).  XCD x owns the x_perm rows [R_x, R_x+1) of its m-tiles and the items
//   * dispatch item: 256 of those rows gathered from x (with their routing
//     weights), then flag[item] = 1;
//   * W1 tile: waits until the dispatch items holding its rows are flagged,
//     computes H and A = silu(gate) * up, then f2done[m-tile] += 1;
//   * W2 tile: waits until f2done[m-tile] equals the number of W1 tiles of that
//     m-tile, then computes O.
// Its ticket order merges the dispatch items into the W1 tiles so that each W1
// tile comes kLead items after the last dispatch item it needs, then lists the
// W2 tiles.  Every workgroup takes one ticket, runs that one item and exits.
// An item waits only on items of its own queue with smaller tickets, which
// were taken by workgroups already running (dispatch items never wait), so the
// schedule cannot deadlock whether or not all workgroups are resident.  Each
// wait is bounded in time and reports MOE_ETIMEOUT through the error word.
//
// Selected with MOE_FLAG_OVERLAP.  On MI355X at the Qwen3 shapes it is slower
// than one kernel per step (30B forward 2.4 ms against 1.9 ms): each workgroup
// pays a ticket round trip before its tile starts, the rows crossing
// workgroups are written through, and the L2 hit rate drops (67% against 76%
// for the separate GEMMs), which outweighs the overlap it buys.
//
// Coherence: the XCDs' L2 caches are not coherent with each other.  Rows that
// cross workgroups inside the launch (x_perm, A) are written with device-
// coherent stores (written through to the coherence point), each producer waits
// for its stores to complete before its flag is raised, and a consumer touches
// no line of those rows before their flag is up (rows are whole 128-byte lines
// and a tile reads only its own rows), so no XCD holds a stale copy and
// consumers need no cache invalidation.
#include <algorithm>

#include "moe_grouped.h"

namespace moe {

namespace {

using namespace gemm;

// A dispatch item copies its rows on one CU, so it takes much longer than its
// share of a whole-GPU copy; items are therefore small and placed far ahead of
// the tiles that need them (measured at the 30B shape: 256-row items two ahead
// took the forward from 1.9 to 3.8 ms, 64-row items 160 ahead to 2.4 ms).
constexpr int kChunkRows = 64;  // x_perm rows per dispatch item
constexpr int kLead = 160;      // dispatch items placed ahead of the W1 tiles needing them
constexpr int kXcds = 8;
constexpr uint64_t kWaitTicks = 2000000;  // 20 ms of the 100 MHz real-time counter per wait
constexpr uint64_t kTestWaitTicks = 100;  // 1 us
enum : int { kItemChunk = 0, kItemW1 = 1, kItemW2 = 2 };
// the wide two-stage 128-byte-row loop of the per-step forward GEMMs
using TileQ = Tile<256, 256, 2, 4, 2, true>;

// ctrl words: tickets [8], totals [8], table bases [8], row bounds R [9],
// dispatch-item bases CB [9]
enum : int { kTickets = 0, kTotals = 8, kBases = 16, kRows = 24, kChunkBase = 33, kCtrlWords = 42 };

struct QLayout {
  size_t ctrl, flags, f2done, table, total;  // byte offsets inside the queue region
  int nc, mt, ntn2, ntn3;                    // capacities: dispatch items, m-tiles; n-tiles
};

inline int max_mtiles256(const moe_desc& d) {
  const long long N = (long long)d.T * d.K;
  return int((N + (long long)d.E * 255) / 256);
}

inline QLayout qlayout(const moe_desc& d) {
  QLayout q{};
  const long long N = (long long)d.T * d.K;
  q.nc = int((N + kChunkRows - 1) / kChunkRows) + kXcds;
  q.mt = max_mtiles256(d);
  q.ntn2 = (2 * d.F) / 256;
  q.ntn3 = d.D / 256;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
  q.ctrl = take(kCtrlWords * 4);
  q.flags = take(size_t(q.nc) * 4);
  q.f2done = take(size_t(q.mt) * 4);
  q.table = take((size_t(q.nc) + size_t(q.mt) * (q.ntn2 + q.ntn3)) * 4);
  q.total = o;
  return q;
}

struct BuildArgs {
  const int32_t* offsets;
  const int32_t* tile256;  // [E+1] prefix sum of ceil(count / 256)
  int E, ntn2, ntn3;
  int* ctrl;
  int* flags;
  int* f2done;
  int* table;
};

__device__ __forceinline__ int part(int n, int x) { return int((long long)n * x / kXcds); }

// Expert of global 256-row m-tile mt (largest e with tile256[e] <= mt).
__device__ __forceinline__ int expert_of(const int32_t* tile256, int E, int mt) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile256[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

// Builds the per-XCD ticket tables and clears the counters for one forward.
__global__ void __launch_bounds__(256) queue_build_kernel(BuildArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int E = a.E, MT = a.tile256[E], nvalid = a.offsets[E];
  // first x_perm row of m-tile mt (nvalid past the last one)
  auto first_row = [&](int mt) {
    if (mt >= MT) return nvalid;
    const int e = expert_of(a.tile256, E, mt);
    return a.offsets[e] + (mt - a.tile256[e]) * 256;
  };
  int R[kXcds + 1], CB[kXcds + 1], BASE[kXcds + 1];
  CB[0] = 0;
  BASE[0] = 0;
  for (int x = 0; x <= kXcds; ++x) R[x] = first_row(part(MT, x));
  for (int x = 0; x < kXcds; ++x) {
    const int nc = (R[x + 1] - R[x] + kChunkRows - 1) / kChunkRows;
    const int nm = part(MT, x + 1) - part(MT, x);
    CB[x + 1] = CB[x] + nc;
    BASE[x + 1] = BASE[x] + nc + nm * (a.ntn2 + a.ntn3);
  }
  const int G2 = MT * a.ntn2, G3 = MT * a.ntn3, NC = CB[kXcds];
  // XCD owning global m-tile mt
  auto xcd_of_mtile = [&](int mt) {
    int x = 0;
    while (x + 1 < kXcds && part(MT, x + 1) <= mt) ++x;
    return x;
  };
  // local dispatch items of XCD x placed before its W1 tile g
  auto before = [&](int g, int x) {
    const int mt = g / a.ntn2;
    const int e = expert_of(a.tile256, E, mt);
    const int e0 = a.offsets[e], ne = a.offsets[e + 1] - e0, m0 = (mt - a.tile256[e]) * 256;
    const int last = e0 + m0 + min(256, ne - m0) - 1;
    return min((last - R[x]) / kChunkRows + 1 + kLead, CB[x + 1] - CB[x]);
  };
  if (i < G2) {
    const int x = xcd_of_mtile(i / a.ntn2);
    a.table[BASE[x] + (i - part(MT, x) * a.ntn2) + before(i, x)] = (kItemW1 << 28) | i;
  }
  if (i < NC) {
    int x = 0;
    while (x + 1 < kXcds && CB[x + 1] <= i) ++x;
    const int cl = i - CB[x];
    int lo = part(MT, x) * a.ntn2, hi = part(MT, x + 1) * a.ntn2;  // first W1 tile after it
    const int g0 = lo;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (before(mid, x) <= cl) lo = mid + 1; else hi = mid;
    }
    a.table[BASE[x] + cl + (lo - g0)] = (kItemChunk << 28) | i;
    a.flags[i] = 0;
  }
  if (i < G3) {
    const int x = xcd_of_mtile(i / a.ntn3);
    const int nm = part(MT, x + 1) - part(MT, x);
    a.table[BASE[x] + (CB[x + 1] - CB[x]) + nm * a.ntn2 + (i - part(MT, x) * a.ntn3)] =
        (kItemW2 << 28) | i;
  }
  if (i < MT) a.f2done[i] = 0;
  if (i < kXcds) {
    a.ctrl[kTickets + i] = 0;
    a.ctrl[kTotals + i] = BASE[i + 1] - BASE[i];
    a.ctrl[kBases + i] = BASE[i];
  }
  if (i <= kXcds) {
    a.ctrl[kRows + i] = R[i];
    a.ctrl[kChunkBase + i] = CB[i];
  }
}

struct QueueArgs {
  GroupedArgs w1, w2;      // tile_start = 256-row m-tile prefix
  const void* x;           // [T, D] bf16, or fp32 when in_f32
  int in_f32, K, D;
  const int32_t* src;      // [N] pair of each permuted row
  uint16_t* xperm;         // [N, D]
  int* ctrl;
  int* flags;
  int* f2done;
  const int* table;
  uint32_t* err;
  uint64_t wait_ticks;
  int unreachable;         // test hook: waits target +unreachable
};

// Polls *p until it reaches target, for at most limit_ticks of the 100 MHz
// real-time counter; on expiry sets the timeout bit of the error word.
__device__ __forceinline__ void wait_at_least(const int* p, int target, uint64_t limit_ticks,
                                              uint32_t* err) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return;
    if (__builtin_amdgcn_s_memrealtime() - t0 > limit_ticks) break;
    __builtin_amdgcn_s_sleep(2);
  }
  atomicOr(err, kErrTimeout);
}

// Gathers x_perm rows [r0, r1): row r is token src[r] / K.
template <int THREADS>
__device__ __forceinline__ void dispatch_rows(const QueueArgs& q, int r0, int r1) {
  const int cpr = q.D / 8;  // 16-byte chunks per bf16 row
  const int total = (r1 - r0) * cpr;
  constexpr int U = 4;
  for (int i0 = threadIdx.x; i0 < total; i0 += U * THREADS) {
    uint4 v[U];
    int rr[U], cc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * THREADS;
      rr[u] = -1;
      if (i < total) {
        rr[u] = r0 + i / cpr;
        cc[u] = i % cpr;
        const int t = q.src[rr[u]] / q.K;
        if (q.in_f32) {
          const float4* s = reinterpret_cast<const float4*>(q.x) + (size_t(t) * q.D + cc[u] * 8) / 4;
          const float4 a = s[0], b = s[1];
          v[u] = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                            pack_bf16x2(b.z, b.w));
        } else {
          v[u] = reinterpret_cast<const uint4*>(q.x)[(size_t(t) * q.D) / 8 + cc[u]];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (rr[u] >= 0) {
        store16_coherent(reinterpret_cast<char*>(q.xperm + size_t(rr[u]) * q.D + cc[u] * 8), v[u]);
      }
  }
}

// One work item per workgroup, in per-XCD ticket order.
template <class TL>
__global__ void __launch_bounds__(TL::THREADS, 1) fwd_queue_kernel(QueueArgs q) {
  __shared__ __attribute__((aligned(1024))) char smem[TL::LDS];
  typedef volatile __attribute__((address_space(3))) int lds_int;
  lds_int* slot = static_cast<lds_int*>(AS3(smem));
  const int x = blockIdx.x % kXcds;
  if (threadIdx.x == 0) {
    const int t = __hip_atomic_fetch_add(q.ctrl + kTickets + x, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    *slot = t < q.ctrl[kTotals + x] ? q.table[q.ctrl[kBases + x] + t] : -1;
  }
  __syncthreads();
  // broadcast through LDS, then made wave-uniform so that the branches below
  // (which hold workgroup barriers) are scalar branches
  const int item = __builtin_amdgcn_readfirstlane(*slot);
  __syncthreads();  // the slot is pipeline LDS: read before the item reuses it
  if (item < 0) return;
  const int kind = item >> 28, idx = item & 0x0fffffff;
  const int mtiles = q.w1.tile_start[q.w1.E];
  const int r_lo = q.ctrl[kRows + x], r_hi = q.ctrl[kRows + x + 1], cb = q.ctrl[kChunkBase + x];
  // every table entry is rewritten by the build step; the range checks only
  // keep a corrupted table from turning into out-of-bounds accesses
  if (kind == kItemChunk && idx >= cb && idx < q.ctrl[kChunkBase + x + 1]) {
    const int r0 = r_lo + (idx - cb) * kChunkRows;
    dispatch_rows<TL::THREADS>(q, r0, min(r0 + kChunkRows, r_hi));
    wait_vmcnt<0>();
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(q.flags + idx, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (kind == kItemW1 && idx < mtiles * q.w1.ntn) {
    const TileCoord c = decode_tile<TL::BM>(q.w1, idx);
    if (threadIdx.x == 0) {
      const int first = c.e0 + c.m0, last = first + c.rows_valid - 1;
      for (int ch = (first - r_lo) / kChunkRows; ch <= (last - r_lo) / kChunkRows; ++ch)
        wait_at_least(q.flags + cb + ch, 1 + q.unreachable, q.wait_ticks, q.err);
    }
    __syncthreads();
    grouped_tile<TL, false, EPI_SWIGLU, true>(q.w1, c, smem);
    wait_vmcnt<0>();
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(q.f2done + c.mt_g, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (kind == kItemW2 && idx < mtiles * q.w2.ntn) {
    const TileCoord c = decode_tile<TL::BM>(q.w2, idx);
    if (threadIdx.x == 0)
      wait_at_least(q.f2done + c.mt_g, q.w1.ntn + q.unreachable, q.wait_ticks, q.err);
    __syncthreads();
    grouped_tile<TL, false, EPI_STORE>(q.w2, c, smem);
  }
}

}  // namespace

size_t queue_scratch_bytes(const moe_desc& d) { return qlayout(d).total; }

bool queue_capable(const moe_desc& d) {
  const bool bf16_fwd = d.mode == MOE_FP32_BF16GEMM || d.mode == MOE_BF16 || d.mode == MOE_FP8_BWD;
  return bf16_fwd && (2 * d.F) % 256 == 0 && d.D % 256 == 0 && (d.flags & MOE_FLAG_OVERLAP);
}

int launch_fwd_queue(const moe_desc& d, const Layout& L, const void* x, bool in_f32,
                     const uint16_t* w1, const uint16_t* w2, char* scratch, hipStream_t s) {
  const QLayout Q = qlayout(d);
  char* qbase = scratch + L.queue;
  BuildArgs b{};
  b.offsets = reinterpret_cast<const int32_t*>(scratch + L.offsets);
  b.tile256 = reinterpret_cast<const int32_t*>(scratch + L.tiles[2]);
  b.E = d.E;
  b.ntn2 = Q.ntn2;
  b.ntn3 = Q.ntn3;
  b.ctrl = reinterpret_cast<int*>(qbase + Q.ctrl);
  b.flags = reinterpret_cast<int*>(qbase + Q.flags);
  b.f2done = reinterpret_cast<int*>(qbase + Q.f2done);
  b.table = reinterpret_cast<int*>(qbase + Q.table);
  const long long items = std::max<long long>(
      {(long long)Q.nc, (long long)Q.mt * std::max(Q.ntn2, Q.ntn3), (long long)Q.mt,
       (long long)kXcds + 1});
  prof_begin("queue_build", s);
  queue_build_kernel<<<unsigned((items + 255) / 256), 256, 0, s>>>(b);
  prof_end(s);
  if (hipGetLastError() != hipSuccess) return MOE_EHIP;

  QueueArgs q{};
  q.w1.offsets = b.offsets;
  q.w1.tile_start = b.tile256;
  q.w1.E = d.E;
  q.w1.K = d.D;
  q.w1.ntn = Q.ntn2;
  q.w1.F = d.F;
  q.w1.A = reinterpret_cast<const uint16_t*>(scratch + L.xperm);
  q.w1.lda = d.D;
  q.w1.B = w1;
  q.w1.bstride = int64_t(2) * d.F * d.D;
  q.w1.ldb = d.D;
  q.w1.brows = 2 * d.F;
  q.w1.out = L.recompute ? nullptr : reinterpret_cast<uint16_t*>(scratch + L.h);
  q.w1.out2 = reinterpret_cast<uint16_t*>(scratch + L.a);
  if (bf16_wide(d))  // A_w = w A, as the per-step forward stores it (routing wrote w_perm)
    q.w1.rw = reinterpret_cast<const float*>(scratch + L.wperm);
  q.w2.offsets = b.offsets;
  q.w2.tile_start = b.tile256;
  q.w2.E = d.E;
  q.w2.K = d.F;
  q.w2.ntn = Q.ntn3;
  q.w2.F = d.F;
  q.w2.A = reinterpret_cast<const uint16_t*>(scratch + L.a);
  q.w2.lda = d.F;
  q.w2.B = w2;
  q.w2.bstride = int64_t(d.D) * d.F;
  q.w2.ldb = d.F;
  q.w2.brows = d.D;
  q.w2.out = reinterpret_cast<uint16_t*>(scratch + L.o);
  q.w2.ldo = d.D;
  q.x = x;
  q.in_f32 = in_f32 ? 1 : 0;
  q.K = d.K;
  q.D = d.D;
  q.src = reinterpret_cast<const int32_t*>(scratch + L.src);
  q.xperm = reinterpret_cast<uint16_t*>(scratch + L.xperm);
  q.ctrl = b.ctrl;
  q.flags = b.flags;
  q.f2done = b.f2done;
  q.table = b.table;
  q.err = reinterpret_cast<uint32_t*>(scratch + L.err);
  const bool test = (d.flags & MOE_FLAG_QUEUE_TIMEOUT_TEST) != 0;
  q.wait_ticks = test ? kTestWaitTicks : kWaitTicks;
  q.unreachable = test ? (1 << 28) : 0;
  // per XCD at most ceil(mt/8) m-tiles, with their W1 and W2 tiles and the
  // dispatch items of their rows (at most 256 / kChunkRows per m-tile), plus one
  const long long per_xcd = (long long)(Q.mt + kXcds - 1) / kXcds *
                                ((256 + kChunkRows - 1) / kChunkRows + Q.ntn2 + Q.ntn3) + 1;
  const long long grid = per_xcd * kXcds;
  prof_begin("fwd_queue", s);
  fwd_queue_kernel<TileQ><<<unsigned(grid), TileQ::THREADS, 0, s>>>(q);
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
