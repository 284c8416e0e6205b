// Building blocks shared by the MFMA GEMM kernels (bf16 and fp8): buffer
// resources, direct-to-LDS loads, swizzled LDS tiles, operand stagers, the
// pipelined main loop and the accumulator layout.  See moe_gemm.hip for the
// design notes.
#pragma once

#include <type_traits>

#include "moe_common.h"
#include "moe_fp8_codec.h"

namespace moe {
namespace gemm {

constexpr int kBK = 32;  // contraction step of the bf16 GEMMs (elements)

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
#define AS3(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ int xcd_remap(int b, int G) {
  const int xcd = b & 7, local = b >> 3;
  const int q = G >> 3, r = G & 7;
  return xcd * q + (xcd < r ? xcd : r) + local;
}

// Workgroups of KERNEL that fit on the current device at once (CUs times the
// occupancy per CU), queried once per kernel and device.
template <auto KERNEL>
int resident_grid(int threads, int* out) {
  static int cached[64] = {};
  int dev;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_EHIP;
  if (cached[dev] == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, KERNEL, threads, 0) != hipSuccess ||
        cus <= 0 || per <= 0)
      return MOE_EHIP;
    cached[dev] = cus * per;
  }
  *out = cached[dev];
  return MOE_OK;
}

// Tiles of a per-expert (weight-gradient) GEMM with `per` tiles per expert,
// one workgroup per tile: experts are taken longest first (eorder, written by
// the routing step).  Workgroup b takes tile expert_tile_start: when the
// routing is skewed (eorder[E] set) b itself, keeping the hardware's
// round-robin over the XCDs so the longest tiles start first on every XCD,
// otherwise its XCD's contiguous run, so consecutive tiles of an expert share
// that XCD's L2.
__device__ __forceinline__ int expert_tile_start(const int32_t* eorder, int E) {
  return eorder[E] ? int(blockIdx.x) : xcd_remap(blockIdx.x, gridDim.x);
}
struct ExpertTile { int e, rem; };
__device__ __forceinline__ ExpertTile expert_tile(const int32_t* eorder, int l, int per) {
  const int rank = l / per;
  return {eorder[rank], l - rank * per};
}

// Output tile (mt, nt) of the rem-th of one expert's tm x tn weight-gradient
// tiles: blocks of up to 4 m-tiles x 8 n-tiles, m-tiles fastest, so the run of
// 32 consecutive tiles an XCD holds at once reads 4 + 8 operand slices (in row
// order with tn = 16 it read 2 + 16, the whole second operand: the 235B W1
// wgrad fetched 7.45 GB, now 4.83 GB, and runs 1.8% faster in bf16 and 3.7% in
// blockwise FP8; row order for rows of at most 8 tiles made the 30B MXFP8 W2
// wgrad 7% slower).
__device__ __forceinline__ void wgrad_mn(int rem, int tm, int tn, int& mt, int& nt) {
  constexpr int GM = 4, GN = 8;
  const int sr = rem / (GM * tn), gm = min(GM, tm - sr * GM);
  const int in_sr = rem - sr * GM * tn;
  const int nb = in_sr / (gm * GN), in_nb = in_sr - nb * gm * GN;
  mt = sr * GM + in_nb % gm;
  nt = nb * GN + in_nb / gm;
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// The expert of flat tile l is the last e in [0, E) with tile_start[e] * u <= key
// (u = ntn, key = l for n-tiles outer; u = 1, key = the m-tile otherwise):
// tile_start is non-decreasing from 0, so e = #{e : tile_start[e] * u <= key} - 1.
// With E < 192 every lane loads its three entries at once and the wave counts
// them with ballots: one memory round trip at each tile's start instead of a
// chain of log2(E) dependent loads (30B W2 -2%, W1 dgrad -1%).  Called by whole
// waves in uniform control flow.
__device__ __forceinline__ int tile_expert(const int32_t* ts, int E, int u, int key) {
  if (E < 192) {
    const int lane = threadIdx.x & 63;
    const int v0 = ts[min(lane, E)], v1 = ts[min(lane + 64, E)], v2 = ts[min(lane + 128, E)];
    const int n = __popcll(__ballot(lane < E && v0 * u <= key)) +
                  __popcll(__ballot(lane + 64 < E && v1 * u <= key)) +
                  __popcll(__ballot(lane + 128 < E && v2 * u <= key));
    return n - 1;
  }
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ts[mid] * u <= key) lo = mid; else hi = mid;
  }
  return lo;
}

// Raw buffer resource over [base, base + bytes): loads at byte offsets >= bytes return 0.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(int(uint32_t(a)));
  r[1] = __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(int(bytes));
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from the buffer at `voff` into LDS at lds_base + 16 * lane.
// Issued as inline asm so the compiler does not serialise on it; completion is
// awaited explicitly with wait_vmcnt before the barrier that publishes a stage.
// NT: with the nontemporal cache policy, for data read once.
template <bool NT = false>
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_base, int voff) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "s"(lds_base), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_base), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(AS3(p)));
}

// Chunk swizzles (chunk = 16 bytes).  A k-contiguous tile row holds ROWB bytes
// of one row's k-run; the chunk index is XORed with bits of the row so that the
// 16 lanes of a fragment read (16 rows, same logical chunk) land on 16 distinct
// 16-byte bank groups of a 256-byte LDS line.
template <int ROWB>
__device__ __forceinline__ int swz_row(int row) {
  static_assert(ROWB == 64 || ROWB == 128, "k-contiguous rows are 64 or 128 bytes");
  if constexpr (ROWB == 128) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}
__device__ __forceinline__ int swz_k(int row) { return swz_row<128>(row); }
template <int R>
__device__ __forceinline__ int swz_t(int krow) {
  if constexpr (R >= 128) return (krow & 3) << 2;
  else return ((krow >> 1) & 1) << 2;
}

// ---------------------------------------------------------------------------
// Operand stagers.  Each knows, per lane, the byte offset (relative to its
// buffer resource, at k-step 0) of the 16-byte chunk that lane fetches for each
// of the wave's DMA instructions, and how far that offset moves per k-step.

// k-contiguous operand, R rows of ROWB bytes per k-step: row r of the tile is
// at rowoff(r) bytes (negative: the row does not exist and reads as zeros).
template <int R, int WAVES, int ROWB>
struct KStager {
  static constexpr int LPR = ROWB / 16;               // lanes per row
  static constexpr int RPI = 64 / LPR;                // rows per DMA instruction
  static constexpr int NI = R * ROWB / (1024 * WAVES);  // DMA instructions per wave per k-step
  static_assert(NI >= 1 && NI * 1024 * WAVES == R * ROWB, "tile rows must split evenly over waves");
  i32x4 rsrc;
  int vb[NI];
  template <class RowOff>
  __device__ __forceinline__ void init(i32x4 r, RowOff rowoff, int wave, int lane) {
    rsrc = r;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int q = wave * NI + j;
      const int row = q * RPI + lane / LPR;
      const int logical = (lane % LPR) ^ swz_row<ROWB>(row);
      const int ro = rowoff(row);
      vb[j] = ro < 0 ? int(0x80000000u) : ro + logical * 16;
    }
  }
  // DMA instructions [j0, j1) of this operand for k-step kt into the stage at lds.
  __device__ __forceinline__ void issue(uint32_t lds, int wave, int kt, int j0 = 0, int j1 = NI) const {
#pragma unroll
    for (int j = 0; j < NI; ++j)
      if (j >= j0 && j < j1) dma16(rsrc, lds + uint32_t(wave * NI + j) * 1024u, vb[j] + kt * ROWB);
  }
};

// k-outer operand, R output columns, kBK k-rows per k-step: k-row k of the
// tile is at k * ld_bytes, column c at c * 2 (relative to the resource base,
// which includes the tile's first column).
template <int R, int WAVES>
struct TStager {
  static constexpr int NI = R * kBK * 2 / (1024 * WAVES);
  static constexpr int LPR = R / 8;      // lanes per k-row
  static constexpr int RPI = 64 / LPR;   // k-rows per DMA instruction
  static_assert(NI >= 1 && NI * 1024 * WAVES == R * kBK * 2, "tile k-rows must split evenly over waves");
  i32x4 rsrc;
  int vb[NI];
  int step;  // bytes per k-step
  __device__ __forceinline__ void init(i32x4 r, int ld_bytes, int wave, int lane) {
    rsrc = r;
    step = ld_bytes * kBK;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int q = wave * NI + j;
      const int krow = q * RPI + lane / LPR;
      const int logical = (lane % LPR) ^ swz_t<R>(krow);
      vb[j] = krow * ld_bytes + logical * 16;
    }
  }
  __device__ __forceinline__ void issue(uint32_t lds, int wave, int kt, int j0 = 0, int j1 = NI) const {
#pragma unroll
    for (int j = 0; j < NI; ++j)
      if (j >= j0 && j < j1) dma16(rsrc, lds + uint32_t(wave * NI + j) * 1024u, vb[j] + kt * step);
  }
};

// Fragment reads (8 consecutive k of one row/column, k-step sub-block kk).
__device__ __forceinline__ bf16x8 frag_k(const char* tile, int row, int kk, int lane) {
  constexpr int ROWB = kBK * 2;
  const int chunk = kk * 2 + (lane >> 5);
  return *reinterpret_cast<const bf16x8*>(tile + row * ROWB + ((chunk ^ swz_row<ROWB>(row)) << 4));
}

template <int R>
__device__ __forceinline__ bf16x8 frag_t(const char* tile, int col0, int kk, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int col = col0 + 16 * (g & 1) + 4 * (s & 3);
  i16x4 h[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int krow = kk * 16 + 8 * (g >> 1) + 4 * half + (s >> 2);
    const char* p = tile + krow * (2 * R) + (((col >> 3) ^ swz_t<R>(krow)) << 4) + (col & 7) * 2;
    h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)AS3(p));
  }
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
  return __builtin_bit_cast(bf16x8, v);
}

// s_waitcnt vmcnt(n * per) for a runtime n in [0, 3].
template <int PER>
__device__ __forceinline__ void wait_vmcnt_n(int n) {
  if (n >= 3) wait_vmcnt<3 * PER>();
  else if (n == 2) wait_vmcnt<2 * PER>();
  else if (n == 1) wait_vmcnt<PER>();
  else wait_vmcnt<0>();
}

__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// threadIdx.x through an empty volatile asm: values derived from it are
// recomputed where they are used instead of being hoisted out of an enclosing
// loop (a persistent kernel would otherwise keep every per-thread address of
// every work item's code live across the whole loop).
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Scheduling pattern for one sub-step: NMF MFMAs with the NDS LDS reads of the
// next fragments spread between them (group masks: 0x8 MFMA, 0x100 DS read).
template <int NMF, int NDS, int M = 0>
__device__ __forceinline__ void interleave_mfma_ds() {
  if constexpr (M < NMF) {
    constexpr int PER = (NDS + NMF - 1) / NMF;
    constexpr int D0 = M * PER < NDS ? M * PER : NDS;
    constexpr int D1 = D0 + PER < NDS ? D0 + PER : NDS;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (D1 > D0) __builtin_amdgcn_sched_group_barrier(0x100, D1 - D0, 0);
    interleave_mfma_ds<NMF, NDS, M + 1>();
  }
}

// The pipelined main loop: acc += A_tile * B_tile^T over ktiles k-steps.  The
// workgroup's WGM x WGN waves each own a (BM/WGM) x (BN/WGN) sub-tile.  The
// MFMA takes the B fragment as its first operand, so an accumulator register
// block holds C^T: lane l owns output row (l & 31) of a 32 x 32 block and four
// consecutive output columns per group of four registers (see acc_col).
//
// STAGES k-steps of kBK sit in an LDS ring, filled by
// direct-to-LDS loads that run STAGES-1 k-steps ahead.  One barrier per k-step,
// placed before the last 16-deep sub-step: it publishes k-step kt+1 (each wave
// has waited for its own loads of it) and certifies that every wave has read
// its fragments of k-step kt-1's slot, which the loads issued from then on
// overwrite.  The first fragments of k-step kt+1 are read across the barrier
// while the MFMAs of k-step kt's last sub-step run, and the DMA instructions of
// a k-step are spread over its sub-steps instead of issued in one burst.  The
// steady-state body has no branches; the last STAGES-1 k-steps run a copy
// without loads.
// Calls f(std::integral_constant<int, A>) for the largest A <= TOP with A <= act
// (act is wave-uniform, so this is a chain of scalar branches).
template <int TOP, class F>
__device__ __forceinline__ void with_active(int act, F&& f) {
  if constexpr (TOP == 0) {
    f(std::integral_constant<int, 0>{});
  } else {
    if (act >= TOP) f(std::integral_constant<int, TOP>{});
    else with_active<TOP - 1>(act, f);
  }
}

// ACT: how many of this wave's 32-row blocks of A hold rows (the rest of a
// ragged last tile are past the expert's end): only those are read and
// multiplied.  Every variant issues the same loads and barriers.
template <int BM, int BN, int WGM, int WGN, int STAGES, bool A_T, bool B_T, int ACT, class SA,
          class SB>
__device__ __forceinline__ void mainloop(char* smem, const SA& sa, const SB& sb, int ktiles,
                                         f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32], int wave,
                                         int lane) {
  constexpr int WM = BM / WGM, WN = BN / WGN, WMT = WM / 32, WNT = WN / 32, KK = kBK / 16;
  static_assert(ACT >= 0 && ACT <= WMT, "active blocks within the wave tile");
  constexpr int A_BYTES = BM * kBK * 2, STAGE = (BM + BN) * kBK * 2;
  constexpr int NI = SA::NI + SB::NI;  // DMA instructions per wave per k-step
  static_assert(STAGES >= 3 && STAGES - 2 <= 3, "ring of 3 to 5 k-steps");
  static_assert(KK == 2, "two 16-deep sub-steps per k-step");
  const int wm = wave / WGN, wn = wave % WGN;
  const uint32_t base = lds_addr(smem);

  struct Frags { bf16x8 a[WMT], b[WNT]; };
  auto load = [&](int kt, int kk, Frags& f) {
    if constexpr (ACT == 0) return;
    const char* ta = smem + (kt % STAGES) * STAGE;
    const char* tb = ta + A_BYTES;
#pragma unroll
    for (int i = 0; i < ACT; ++i) {
      const int r0 = wm * WM + i * 32;
      if constexpr (A_T) f.a[i] = frag_t<BM>(ta, r0, kk, lane);
      else f.a[i] = frag_k(ta, r0 + (lane & 31), kk, lane);
    }
#pragma unroll
    for (int j = 0; j < WNT; ++j) {
      const int c0 = wn * WN + j * 32;
      if constexpr (B_T) f.b[j] = frag_t<BN>(tb, c0, kk, lane);
      else f.b[j] = frag_k(tb, c0 + (lane & 31), kk, lane);
    }
  };
  auto mma = [&](const Frags& f, int m0, int m1) {
#pragma unroll
    for (int m = 0; m < ACT * WNT; ++m)
      if (m >= m0 && m < m1) {
        const int i = m / WNT, j = m % WNT;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
      }
  };
  // DMA instructions [j0, j1) (over both operands) of k-step kt
  auto issue = [&](int kt, int j0, int j1) {
    const uint32_t st = base + uint32_t(kt % STAGES) * STAGE;
    sa.issue(st, wave, kt, j0, j1);
    sb.issue(st + A_BYTES, wave, kt, j0 - SA::NI, j1 - SA::NI);
  };
  constexpr int NH = NI / 2;  // instructions issued in the first sub-step

  const int pre = min(STAGES - 1, ktiles);
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < pre) issue(s, 0, NI);
  wait_vmcnt_n<NI>(pre - 1);
  __builtin_amdgcn_s_barrier();
  Frags f0, f1;
  load(0, 0, f0);

  // LDS read instructions per fragment set (a transposed fragment takes two)
  constexpr int NDS = ACT == 0 ? 0 : ACT * (A_T ? 2 : 1) + WNT * (B_T ? 2 : 1);
  constexpr int NMF = ACT * WNT;
  auto step = [&](int kt, auto dma_on) {
    constexpr bool DMA = decltype(dma_on)::value;
    const int kn = kt + STAGES - 1;
    // sub-step 0: fragments of sub-step 1 are read while its MFMAs run
    load(kt, 1, f1);
    if constexpr (DMA) issue(kn, 0, NH);
    mma(f0, 0, NMF);
    interleave_mfma_ds<NMF, NDS>();
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 1
    if constexpr (DMA) issue(kn, NH, NI);
    const bool more = DMA || kt + 1 < ktiles;
    if (more) {
      wait_vmcnt_n<NI>(DMA ? STAGES - 2 : ktiles - 2 - kt);
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      load(kt + 1, 0, f0);
    }
    mma(f1, 0, NMF);
    if constexpr (DMA) interleave_mfma_ds<NMF, NDS>();
    __builtin_amdgcn_sched_barrier(0);
  };
  const int kmain = ktiles - (STAGES - 1);
  int kt = 0;
  for (; kt < kmain; ++kt) step(kt, std::true_type{});
  for (; kt < ktiles; ++kt) step(kt, std::false_type{});
}

// Fragment of a 128-byte (64-k) row for 16-deep sub-step kk (0..3).
__device__ __forceinline__ bf16x8 frag_w(const char* tile, int row, int kk, int lane) {
  const int chunk = kk * 2 + (lane >> 5);
  return *reinterpret_cast<const bf16x8*>(tile + row * 128 + ((chunk ^ swz_row<128>(row)) << 4));
}

// Sub-steps of the wide loop over which the next k-step's loads are issued:
// half in the first, half in the second, so the last of them still has three
// sub-steps to arrive.  Measured at the 30B and 235B shapes against a quarter
// in each sub-step (the last quarter had one sub-step: W1+SwiGLU 0.97 -> 0.89
// ms and 3.22 -> 2.96 ms, W2 -3 to -6%), against all of them in the first
// sub-step (-2 to -3% only) and against thirds, or halves in the first and third.
constexpr int kWideIssueSub = 2;

// Wide-row main loop: bf16 operands in 128-byte rows (64 k per step), two
// stages.  Each step waits for its own loads and meets every wave at the
// barrier (after which the other stage is free); its four 16-deep sub-steps
// then each run their MFMAs while the next sub-step's fragments are read, and
// the first kWideIssueSub of them also issue a share of the next step's loads
// into the free stage.  A and B are both k-contiguous.
struct NoStepHook {
  __device__ void operator()(int, const char*) const {}
};

// hook(kt, a) runs once per k-step after the barrier, with a pointing at the
// stage's A rows (BM rows of 128 bytes, chunks swizzled as swz_row<128>).
template <int BM, int BN, int WGM, int WGN, int ACT, class SA, class SB, class Hook = NoStepHook>
__device__ __forceinline__ void mainloop_w(char* smem, const SA& sa, const SB& sb, int ktiles,
                                           f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32], int wave,
                                           int lane, Hook hook = {}) {
  constexpr int WM = BM / WGM, WN = BN / WGN, WMT = WM / 32, WNT = WN / 32;
  constexpr int A_BYTES = BM * 128, STAGE = (BM + BN) * 128;
  constexpr int NI = SA::NI + SB::NI;
  constexpr int NQW = (NI + kWideIssueSub - 1) / kWideIssueSub;  // DMA instructions per issuing sub-step
  static_assert(ACT >= 0 && ACT <= WMT, "active blocks within the wave tile");
  const int wm = wave / WGN, wn = wave % WGN;
  const uint32_t base = lds_addr(smem);
  // DMA instructions [j0, j1) (over both operands) of k-step kt into stage s
  auto issue = [&](int s, int kt, int j0, int j1) {
    sa.issue(base + uint32_t(s * STAGE), wave, kt, j0, j1);
    sb.issue(base + uint32_t(s * STAGE + A_BYTES), wave, kt, j0 - SA::NI, j1 - SA::NI);
  };
  struct Frags { bf16x8 a[WMT], b[WNT]; };
  auto load = [&](const char* ta, int kk, Frags& f) {
#pragma unroll
    for (int i = 0; i < ACT; ++i) f.a[i] = frag_w(ta, wm * WM + i * 32 + (lane & 31), kk, lane);
#pragma unroll
    for (int j = 0; j < WNT; ++j) f.b[j] = frag_w(ta + A_BYTES, wn * WN + j * 32 + (lane & 31), kk, lane);
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < ACT; ++i)
#pragma unroll
      for (int j = 0; j < WNT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
  };
  constexpr int NMF = ACT * WNT, NDS = ACT == 0 ? 0 : ACT + WNT;
  if (ktiles > 0) issue(0, 0, 0, NI);
  for (int kt = 0; kt < ktiles; ++kt) {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    const bool next = kt + 1 < ktiles;
    const char* ta = smem + (kt & 1) * STAGE;
    Frags f[2];
    load(ta, 0, f[0]);
    hook(kt, ta);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (next && kk < kWideIssueSub)
        issue((kt + 1) & 1, kt + 1, kk * NQW, kk + 1 == kWideIssueSub ? NI : (kk + 1) * NQW);
      if (kk < 3) load(ta, kk + 1, f[(kk + 1) & 1]);
      mma(f[kk & 1]);
      if (kk < 3) interleave_mfma_ds<NMF, NDS>();
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Column (within a 32x32 block) of accumulator register 4*g (the first of four
// consecutive columns); the row is lane & 31.
__device__ __forceinline__ int acc_col(int g, int lane) { return 8 * g + 4 * (lane >> 5); }

template <int A, int B>
__device__ __forceinline__ void zero(f32x16 (&acc)[A][B]) {
#pragma unroll
  for (int i = 0; i < A; ++i)
#pragma unroll
    for (int j = 0; j < B; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// The logistic function with the hardware reciprocal (v_rcp_f32, within 1 ulp):
// an IEEE division here compiles to about ten instructions (scale, reciprocal,
// Newton steps, fix-up) per value, in epilogues that run while the matrix
// cores wait.  exp(-x) = inf gives 0 and exp(-x) = 0 gives 1, as the division.
__device__ __forceinline__ float sigmoid(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  return make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

__device__ __forceinline__ void unpack4(uint2 v, float (&f)[4]) {
  f[0] = __uint_as_float(v.x << 16);
  f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16);
  f[3] = __uint_as_float(v.y & 0xffff0000u);
}

// Tile shape of a GEMM kernel: BM x BN outputs per workgroup of WGM x WGN waves.
// WIDE: the two-stage main loop on 128-byte rows (mainloop_w) instead of the
// STAGES-deep ring on 64-byte rows.
template <int BM_, int BN_, int WGM_, int WGN_, int STAGES_, bool WIDE_ = false>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, STAGES = STAGES_;
  static constexpr bool WIDE = WIDE_;
  static constexpr int WAVES = WGM * WGN, THREADS = 64 * WAVES;
  static constexpr int WM = BM / WGM, WN = BN / WGN, WMT = WM / 32, WNT = WN / 32;
  static constexpr int LDS = WIDE ? 2 * (BM + BN) * 128 : STAGES * (BM + BN) * kBK * 2;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32x32");
  static_assert(!WIDE || STAGES == 2, "the wide-row loop has two stages");
};

enum Epi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2 };

struct EpiArgs {
  uint16_t* out;          // STORE: [rows, ldo]; SWIGLU: H [rows, 2F] or null; DSWIGLU: dH [rows, 2F]
  int ldo;
  uint16_t* out2;         // SWIGLU: A [rows, F] or null
  const uint16_t* hsave;  // DSWIGLU: H [rows, 2F]; may equal out (each tile reads its H band
                          // into LDS before it stores the same band's dH)
  int F;
  // Routing weights carried by the GEMMs (epilogues instantiated with WS):
  // SWIGLU stores A_w = w * A, with wrow[i] the weight of the lane's row in
  // 32-row block i of its wave's share (loaded ahead of the main loop; 1
  // without weights); DSWIGLU takes dA = w * G, loading row r's weight wp[r]
  // itself, and writes dProb partials.  Null wp: no weights.
  float wrow[4];
  const float* wp;        // DSWIGLU: [rows] routing weight of each permuted row
  float* dpart;           // DSWIGLU: dProb partials [rows, F / 64], the wave's 64 columns of
                          // sum_f G[r, f] * A[r, f] (A recomputed from the saved H)
};

// Epilogues stage the output through LDS, one band of 32-row blocks (one per
// wave row, WGM * 32 rows) at a time: each wave writes its accumulators into a
// row-major LDS tile whose 16-byte chunks are XOR-swizzled by row, then the
// whole workgroup writes complete rows with 16-byte stores, so every store
// instruction covers whole 128-byte lines.  A band tile has `cols` elements of
// `ES` bytes per row.
template <int ES>
struct BandTile {
  char* base;
  int cols;
  __device__ __forceinline__ int chunks() const { return cols * ES / 16; }
  __device__ __forceinline__ char* at(int row, int col) const {
    const int byte = col * ES, ch = byte >> 4, sw = ch ^ (row & (min(chunks(), 32) - 1));
    return base + row * cols * ES + (sw << 4) + (byte & 15);
  }
};

// 16-byte global store that is written through to the device-coherent level
// (two agent-scope relaxed 8-byte stores), for data another workgroup of the
// same launch reads after a flag handshake.
__device__ __forceinline__ void store16_coherent(char* dst, uint4 v) {
  uint64_t* d = reinterpret_cast<uint64_t*>(dst);
  __hip_atomic_store(d, uint64_t(v.x) | (uint64_t(v.y) << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(d + 1, uint64_t(v.z) | (uint64_t(v.w) << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Cooperative copy of `rows` band rows (of which the first `valid` exist) from
// LDS to global rows dst(row) (16 bytes per thread per step); COH: device-coherent
// stores, NT: streaming stores.
template <int THREADS, int ES, bool COH = false, bool NT = false, class Dst>
__device__ __forceinline__ void band_store(const BandTile<ES>& t, int rows, int valid, int tid, Dst dst) {
  const int per_row = t.chunks();
  for (int i = tid; i < rows * per_row; i += THREADS) {
    const int r = i / per_row, c = i - r * per_row;
    if (r < valid) {
      const uint4 v = *reinterpret_cast<const uint4*>(t.base + r * per_row * 16 + ((c ^ (r & (min(per_row, 32) - 1))) << 4));
      if constexpr (COH) store16_coherent(dst(r) + c * 16, v);
      else if constexpr (NT) store16_nt(dst(r) + c * 16, v);
      else *reinterpret_cast<uint4*>(dst(r) + c * 16) = v;
    }
  }
}

// Whole-tile form of band_store: ROWS staged rows of CH 16-byte chunks (row
// stride CH * 16 bytes, chunks XOR-swizzled by row as in BandTile) to global
// rows dst(row), the first `valid` of them.  Every thread reads all of its
// chunks from LDS before it issues any store, so its stores leave back to back
// instead of each behind its own LDS round trip.
template <int THREADS, int ROWS, int CH, bool NT = false, class Dst>
__device__ __forceinline__ void tile_store(const char* base, int valid, Dst dst) {
  constexpr int N = ROWS * CH / THREADS;
  constexpr int SW = (CH < 32 ? CH : 32) - 1;
  static_assert(N * THREADS == ROWS * CH, "chunks split evenly over the threads");
  // per-thread offsets recomputed here, not hoisted out of a persistent tile loop
  const int tid = opaque_tid();
  uint4 v[N];
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int i = tid + k * THREADS, r = i / CH, c = i % CH;
    v[k] = *reinterpret_cast<const uint4*>(base + r * CH * 16 + ((c ^ (r & SW)) << 4));
  }
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int i = tid + k * THREADS, r = i / CH, c = i % CH;
    if (r < valid) {
      if constexpr (NT) store16_nt(dst(r) + c * 16, v[k]);
      else *reinterpret_cast<uint4*>(dst(r) + c * 16) = v[k];
    }
  }
}

// Cooperative copy of global rows src(row) into a band tile (zeros for rows >= valid).
template <int THREADS, int ES, class Src>
__device__ __forceinline__ void band_load(const BandTile<ES>& t, int rows, int valid, int tid, Src src) {
  const int per_row = t.chunks();
  for (int i = tid; i < rows * per_row; i += THREADS) {
    const int r = i / per_row, c = i - r * per_row;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < valid) v = *reinterpret_cast<const uint4*>(src(r) + c * 16);
    *reinterpret_cast<uint4*>(t.base + r * per_row * 16 + ((c ^ (r & (min(per_row, 32) - 1))) << 4)) = v;
  }
}

// Rows [0, n) of a 32-row slice of a band tile of CH 16-byte chunks per row to
// the bf16 rows out + (row0 + r) * ld + col0.  (Reading all of a thread's
// chunks before storing any made the SwiGLU-backward epilogue slower.)
template <int THREADS, int CH>
__device__ __forceinline__ void slice_store(const BandTile<2>& t, int n, size_t row0, int col0,
                                            uint16_t* out, int ld, int tid) {
  static_assert(CH <= 32, "one swizzle period per row");
  uint16_t* o = out + row0 * ld + col0;  // wave-uniform: scalar 64-bit arithmetic once
  for (int k = tid; k < 32 * CH; k += THREADS) {
    const int r = k / CH, c = k - r * CH;
    const uint4 v = *reinterpret_cast<const uint4*>(t.base + r * CH * 16 + ((c ^ (r & (CH - 1))) << 4));
    if (r < n) *reinterpret_cast<uint4*>(o + r * ld + 8 * c) = v;
  }
}

// LDS bytes the epilogues stage through (the kernels assert that their
// pipeline buffer is at least this large): one band of output for a store,
// gate + up + A for SwiGLU, two bands of H (gate + up) for the SwiGLU backward.
template <class TL, int EPI>
constexpr int grouped_epi_lds() {
  constexpr int RB = TL::WGM * 32;
  return EPI == EPI_STORE ? RB * TL::BN * 2 : EPI == EPI_SWIGLU ? 3 * RB * TL::BN : 8 * RB * TL::BN;
}
template <class TL, bool OUT_F32>
constexpr int wgrad_epi_lds() { return TL::WGM * 32 * TL::BN * (OUT_F32 ? 4 : 2); }

// SwiGLU-backward epilogue: acc holds dA = (w dy) W2[e] for the tile's
// F-columns; dH = [dg; du] from the saved H (gate, up).  The tile goes out one
// band of WGM x 32 rows at a time through two LDS band buffers: band i+1's H
// arrives by direct-to-LDS loads (into the XOR-swizzled band layout) while
// band i is computed in place and stored, so the H loads overlap the previous
// band's work instead of preceding it.
template <class TL, bool WS>
__device__ __forceinline__ void dswiglu_epilogue(const EpiArgs& p,
                                                 f32x16 (&acc)[TL::WMT][TL::WNT], size_t grow0,
                                                 int rows_valid, int nt, int wm, int wn, int lane,
                                                 char* smem) {
  constexpr int BN = TL::BN, WM = TL::WM, WN = TL::WN, WMT = TL::WMT, WNT = TL::WNT;
  constexpr int RB = TL::WGM * 32;       // rows per band
  constexpr int TILE = RB * BN * 2;      // one band's gate (or up) columns, bytes
  constexpr int BUF = 2 * TILE;          // gate + up
  constexpr int NQ = BUF / 1024;         // 1 KB direct-to-LDS loads per band
  constexpr int CH = BN * 2 / 16;        // 16-byte chunks per band row
  // (callers assert that their LDS holds grouped_epi_lds<TL, EPI_DSWIGLU>() = 2 * BUF bytes)
  static_assert(NQ % TL::WAVES == 0 && CH <= 32, "band loads split over the waves");
  const int F = p.F, f0 = nt * BN;
  const int wave = wm * TL::WGN + wn;
  const int rr = wm * 32 + (lane & 31);
  const i32x4 hr = make_rsrc(p.hsave + grow0 * 2 * F, uint32_t(rows_valid) * 2 * F * 2);
  const uint32_t base = lds_addr(smem);
  // band i's H into buffer b: load q fills bytes [1024 q, 1024 q + 1024) of the buffer
  auto issue = [&](int i, int b) {
#pragma unroll
    for (int k = 0; k < NQ / TL::WAVES; ++k) {
      const int q = wave + k * TL::WAVES;
      const int half = q / (TILE / 1024);                       // 0 gate, 1 up
      const int o = (q % (TILE / 1024)) * 1024 + lane * 16;     // byte in the band tile
      const int brow = o / (BN * 2), pch = (o % (BN * 2)) / 16;
      const int lch = pch ^ (brow & (CH - 1));                  // BandTile swizzle
      const int trow = (brow / 32) * WM + i * 32 + (brow % 32);  // tile row
      const int voff = trow < rows_valid ? (trow * 2 * F + half * F + f0 + lch * 8) * 2
                                         : int(0x80000000u);   // past the expert: zeros
      // read once: nontemporal, so it displaces less of the main loop's operands in the
      // caches (W2 pair -0.4% at 30B, -1.2% at 235B; MXFP8 W2 dgrad -1.4%)
      dma16<true>(hr, base + uint32_t(b * BUF + q * 1024), voff);
    }
  };
  const int tid = wave * 64 + lane;
  issue(0, 0);
  // the lane's rows' routing weights arrive with band 0's H
  float wr[WMT];
  const bool ws = WS && p.wp != nullptr;
  if constexpr (WS) {
#pragma unroll
    for (int i = 0; i < WMT; ++i) {
      const int trow = wm * WM + i * 32 + (lane & 31);
      wr[i] = ws && trow < rows_valid ? p.wp[grow0 + trow] : 1.f;
    }
  }
#pragma unroll
  for (int i = 0; i < WMT; ++i) {
    float part = 0.f;
    const int b = i & 1;
    wait_vmcnt<0>();   // band i's H (and the previous band's stores)
    __syncthreads();   // ... for every wave; buffer b ^ 1 is free again
    if (i + 1 < WMT) issue(i + 1, b ^ 1);
    char* buf = smem + b * BUF;
    BandTile<2> tg{buf, BN}, tu{buf + TILE, BN};
#pragma unroll
    for (int j = 0; j < WNT; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = wn * WN + j * 32 + acc_col(g, lane);
        uint2* pg = reinterpret_cast<uint2*>(tg.at(rr, c));
        uint2* pu = reinterpret_cast<uint2*>(tu.at(rr, c));
        float gv[4], uv[4], dg[4], du[4];
        unpack4(*pg, gv);
        unpack4(*pu, uv);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float G = acc[i][j][4 * g + q];
          // silu(g) = g sg and silu'(g) = sg + silu(g) (1 - sg), with sg the logistic
          // function: dH_gate = dA u silu'(g), dH_up = dA silu(g)
          const float sg = sigmoid(gv[q]);
          const float s = gv[q] * sg, ds = __builtin_fmaf(s, 1.f - sg, sg), Gu = G * uv[q];
          if constexpr (WS) {  // dA = w G; the dProb partial takes G A = G u silu(g)
            part = __builtin_fmaf(Gu, s, part);
            asm volatile("" : "+v"(part));  // keeps the compiler from spilling here
            dg[q] = Gu * wr[i] * ds;
            du[q] = G * wr[i] * s;
          } else {
            dg[q] = Gu * ds;
            du[q] = G * s;
          }
        }
        *pg = pack4(dg[0], dg[1], dg[2], dg[3]);
        *pu = pack4(du[0], du[1], du[2], du[3]);
      }
    if constexpr (WS) {
      if (ws && p.dpart != nullptr) {  // the row's other 32 columns of this wave sit in lane ^ 32
        part += __shfl_xor(part, 32);
        const int trow = wm * WM + i * 32 + (lane & 31);
        if (lane < 32 && trow < rows_valid)
          p.dpart[(grow0 + trow) * (F / 64) + (f0 + wn * WN) / 64] = part;
      }
    }
    __syncthreads();
    for (int w = 0; w < TL::WGM; ++w) {
      const int first = w * WM + i * 32, n = min(32, rows_valid - first);
      if (n <= 0) continue;
      // dH (its FP8 codes come from a pass over the stored rows)
      slice_store<TL::THREADS, CH>(BandTile<2>{buf + w * 32 * BN * 2, BN}, n, grow0 + first, f0,
                                   p.out, 2 * F, tid);
      slice_store<TL::THREADS, CH>(BandTile<2>{buf + TILE + w * 32 * BN * 2, BN}, n, grow0 + first,
                                   F + f0, p.out, 2 * F, tid);
    }
  }
}

// Epilogue of a token-grouped GEMM.  Lane owns row (lane & 31) of each 32-row
// block and, per group g of four registers, four consecutive columns starting
// at acc_col(g).  grow0 is the tile's first row in the permuted buffers; smem is
// the (now free) pipeline LDS, AVAIL bytes of it.  A plain store stages the
// whole bf16 tile at once when AVAIL holds it (one barrier, every store of a
// thread issued back to back; NT: with streaming stores), else one band at a
// time.
template <class TL, int EPI, bool COH2 = false, int AVAIL = 0, bool WS = false, bool NT = false>
__device__ __forceinline__ void grouped_epilogue(const EpiArgs& p,
                                                 f32x16 (&acc)[TL::WMT][TL::WNT], size_t grow0,
                                                 int rows_valid, int nt, int wm, int wn, int lane,
                                                 char* smem, int tid) {
  constexpr int BN = TL::BN, WM = TL::WM, WN = TL::WN, WMT = TL::WMT, WNT = TL::WNT;
  constexpr int RB = TL::WGM * 32;  // rows per band
  const int rr = wm * 32 + (lane & 31);
  __syncthreads();  // every wave is done reading the pipeline stages
  if constexpr (EPI == EPI_DSWIGLU) {
    dswiglu_epilogue<TL, WS>(p, acc, grow0, rows_valid, nt, wm, wn, lane, smem);
    return;
  }
  if constexpr (EPI == EPI_STORE && AVAIL >= TL::BM * BN * 2) {
    BandTile<2> t{smem, BN};
#pragma unroll
    for (int i = 0; i < WMT; ++i)
#pragma unroll
      for (int j = 0; j < WNT; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& a = acc[i][j];
          *reinterpret_cast<uint2*>(t.at(wm * WM + i * 32 + (lane & 31), wn * WN + j * 32 + acc_col(g, lane))) =
              pack4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
        }
    __syncthreads();
    // the tile's first row once in 64 bits (wave-uniform), each row's offset in 32
    char* ob = reinterpret_cast<char*>(p.out + grow0 * p.ldo + nt * BN);
    const int ldb = p.ldo * 2;
    tile_store<TL::THREADS, TL::BM, BN * 2 / 16, NT>(smem, rows_valid, [&](int r) { return ob + r * ldb; });
    return;
  }
#pragma unroll
  for (int i = 0; i < WMT; ++i) {
    // band row w*32 + r holds tile row w*WM + i*32 + r (wave row w's i-th 32-row block)
    if constexpr (EPI == EPI_STORE) {
      BandTile<2> t{smem, BN};
#pragma unroll
      for (int j = 0; j < WNT; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& a = acc[i][j];
          *reinterpret_cast<uint2*>(t.at(rr, wn * WN + j * 32 + acc_col(g, lane))) =
              pack4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
        }
      __syncthreads();
      for (int w = 0; w < TL::WGM; ++w) {
        const int first = w * WM + i * 32, n = min(32, rows_valid - first);
        if (n <= 0) continue;
        BandTile<2> sub{smem + w * 32 * BN * 2, BN};
        char* ob = reinterpret_cast<char*>(p.out + (grow0 + first) * p.ldo + nt * BN);
        const int ldb = p.ldo * 2;
        band_store<TL::THREADS>(sub, 32, n, tid, [&](int r) { return ob + r * ldb; });
      }
    } else if constexpr (EPI == EPI_SWIGLU) {
      const int F = p.F;
      BandTile<2> tg{smem, BN / 2}, tu{smem + RB * BN, BN / 2}, ta{smem + 2 * RB * BN, BN / 2};
#pragma unroll
      for (int j = 0; j < WNT / 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = wn * (WN / 2) + j * 32 + acc_col(g, lane);
          float gv[4], uv[4], av[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gv[q] = acc[i][j][4 * g + q];
            uv[q] = acc[i][j + WNT / 2][4 * g + q];
            av[q] = gv[q] * sigmoid(gv[q]) * uv[q];
            if constexpr (WS) av[q] *= p.wrow[i];  // 1 without routing weights
          }
          *reinterpret_cast<uint2*>(tg.at(rr, c)) = pack4(gv[0], gv[1], gv[2], gv[3]);
          *reinterpret_cast<uint2*>(tu.at(rr, c)) = pack4(uv[0], uv[1], uv[2], uv[3]);
          *reinterpret_cast<uint2*>(ta.at(rr, c)) = pack4(av[0], av[1], av[2], av[3]);
        }
      __syncthreads();
      for (int w = 0; w < TL::WGM; ++w) {
        const int first = w * WM + i * 32, n = min(32, rows_valid - first);
        if (n <= 0) continue;
        const int off = w * 32 * BN;  // bytes of 32 rows of BN/2 bf16
        const int f0 = nt * (BN / 2);
        if (p.out != nullptr) {  // H (not kept under activation recompute)
          // streaming stores: only the backward reads H, and A (read by W2 next) then keeps
          // more of the caches (30B W1+SwiGLU 0.950 -> 0.934 ms, W2 -1%; 235B equal)
          char* hb = reinterpret_cast<char*>(p.out + (grow0 + first) * 2 * F + f0);
          band_store<TL::THREADS, 2, false, true>(BandTile<2>{smem + off, BN / 2}, 32, n, tid,
                                                  [&](int r) { return hb + r * (4 * F); });
          band_store<TL::THREADS, 2, false, true>(BandTile<2>{smem + RB * BN + off, BN / 2}, 32,
                                                  n, tid,
                                                  [&](int r) { return hb + r * (4 * F) + 2 * F; });
        }
        if (p.out2 != nullptr) {  // A (not needed when H is recomputed in the backward)
          if constexpr (COH2) {
            char* ab = reinterpret_cast<char*>(p.out2 + (grow0 + first) * F + f0);
            band_store<TL::THREADS, 2, true>(BandTile<2>{smem + 2 * RB * BN + off, BN / 2}, 32, n,
                                             tid, [&](int r) { return ab + r * (2 * F); });
          }
          else
            slice_store<TL::THREADS, BN / 16>(BandTile<2>{smem + 2 * RB * BN + off, BN / 2}, n,
                                              grow0 + first, f0, p.out2, F, tid);
        }
      }
    }
    __syncthreads();  // the band buffers are reused by the next band
  }
}

// Epilogue of a per-expert weight-gradient GEMM: dW[e] tile (mt, nt) of [M, N],
// one band at a time (the whole-tile staging of the token-grouped store made
// these GEMMs slower: 30B blockwise FP8 wgrads +20%, MXFP8 W1 wgrad +2%).
template <class TL, bool OUT_F32>
__device__ __forceinline__ void wgrad_epilogue(void* C, int M, int N, int e, int mt, int nt,
                                               f32x16 (&acc)[TL::WMT][TL::WNT], int wm, int wn,
                                               int lane, char* smem, int tid) {
  constexpr int BN = TL::BN, WM = TL::WM, WN = TL::WN, ES = OUT_F32 ? 4 : 2;
  const int rr = wm * 32 + (lane & 31);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TL::WMT; ++i) {
    BandTile<ES> t{smem, BN};
#pragma unroll
    for (int j = 0; j < TL::WNT; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& a = acc[i][j];
        char* dst = t.at(rr, wn * WN + j * 32 + acc_col(g, lane));
        if constexpr (OUT_F32)
          *reinterpret_cast<float4*>(dst) = make_float4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
        else
          *reinterpret_cast<uint2*>(dst) = pack4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
      }
    __syncthreads();
    for (int w = 0; w < TL::WGM; ++w) {
      const int first = mt * TL::BM + w * WM + i * 32;
      band_store<TL::THREADS>(BandTile<ES>{smem + w * 32 * BN * ES, BN}, 32, 32, tid, [&](int r) {
        return reinterpret_cast<char*>(C) + ((size_t(e) * M + first + r) * N + nt * BN) * ES;
      });
    }
    __syncthreads();
  }
}

}  // namespace gemm
}  // namespace moe
