// Grouped expert GEMMs of the MoE layer on CDNA4 matrix cores (bf16 in, fp32 accumulate).
//
// The pages fuse "the 2 expert linear layers" and SwiGLU into one kernel and add
// the backward pass (Prime Mega MoE news item, "How does the fused kernel
// work?").  On one GPU this file provides the six expert GEMMs of a training
// step, with the element-wise work fused into their epilogues:
//
//   fwd  W1 + SwiGLU  H = x_perm W1[e]^T, A = silu(H_gate) * H_up      (token-grouped, NT)
//   fwd  W2           O = A W2[e]^T                                    (token-grouped, NT)
//   bwd  W2 dgrad     dA = dYw_perm W2[e]; dH = SwiGLU'(H) applied to dA  (token-grouped, NN)
//   bwd  W1 dgrad     dX_perm = dH W1[e]                               (token-grouped, NN)
//   bwd  W2 wgrad     dW2[e] = sum_r dYw_perm[r] A[r]^T                 (per-expert, TN)
//   bwd  W1 wgrad     dW1[e] = sum_r dH[r] x_perm[r]^T                  (per-expert, TN)
// (dYw_perm holds the dispatched upstream gradient already multiplied by the
// pair's routing weight; in bf16 at the shapes whose W1 GEMM gathers x's rows,
// A holds w * A instead, dYw_perm holds dy itself, and the W2 dgrad's epilogue
// applies w, so the same products carry the weights.)
//
// Work decomposition: a workgroup of WGM x WGN wave64s owns one BM x BN output
// tile (256 x 256 with a 2 x 4 grid of waves on the large shapes, smaller
// fallbacks for dimensions that are not multiples of 256); each wave
// accumulates (BM/WGM) x (BN/WGN) with v_mfma_f32_32x32x16_bf16.  The
// contraction advances 32 at a time through a ring of STAGES LDS buffers
// (4 or 5: up to the whole 160 KB) filled by direct-to-LDS buffer loads
// (buffer_load_dwordx4 ... lds): the loads for k-step kt+STAGES-1 are issued,
// spread between the MFMAs, while k-step kt is computed, so STAGES-1 k-steps
// of global latency are in flight without holding any of the data in
// registers.  One barrier per k-step publishes the next buffer; the first
// fragments of k-step kt+1 are read across it while the last MFMAs of k-step
// kt run.  Loads past the end of an expert's rows (or of its tokens, in the
// wgrads) fall outside the buffer resource and land as zeros.
//
// LDS layouts.  An operand whose global rows run along the contraction index
// ("k-contiguous": activations, and the weights in the forward) is staged as
// R rows x 32 k, 64 bytes per row; an MFMA fragment (8 consecutive k of one
// row) is one ds_read_b128.  An operand whose global rows run along the output
// index ("k-outer": the weights in the dgrads and both operands of the wgrads)
// is staged as 32 k-rows x R, exactly as it lies in memory, and its fragments
// are read with ds_read_b64_tr_b16: a 16-lane group pointing at a 4 (k) x 16
// (m) block gets one column of 4 consecutive k per lane, two reads give the 8
// consecutive k of an MFMA fragment.  In both layouts the 16-byte chunks of a
// row are XOR-swizzled so that each read instruction touches every LDS bank
// once; the swizzle is applied on the load side by choosing which global chunk
// each lane of the (contiguous) LDS write fetches.
//
// Epilogues stage the output tile through the (then idle) LDS ring and write
// whole rows with 16-byte stores; the SwiGLU backward reads its saved H tile
// the same way.
//
// Token-grouped GEMMs walk a flat list of (expert, m-tile, n-tile) built from
// the routing step's per-expert m-tile prefix sums; workgroups past the end
// return at once.  Per-expert GEMMs walk (expert, m-tile, n-tile) over the
// weight shape, with the contraction running over that expert's tokens (zero
// tokens -> zero gradient, no atomics).  Workgroup ids are remapped so that
// consecutive tiles of one expert land on the same XCD (hardware dispatch is
// round-robin over the 8 XCDs) and share its L2.
#include "moe_grouped.h"
#include "moe_pair.h"

namespace moe {
namespace {

using namespace gemm;


// Token-grouped GEMM over the flat (m-tile, n-tile) list, from a grid of
// resident workgroups that take the tiles in rounds of gridDim.x: in each
// round an XCD takes a contiguous run of the list, so the tiles that share an
// A or B slice start together and meet in that XCD's L2 (one workgroup per
// tile, dispatched as CUs free up, lets them drift apart by several k-steps
// and misses there about twice as often).
template <class TL, bool B_T, int EPI>
__global__ void __launch_bounds__(TL::THREADS, 1) grouped_gemm_kernel(GroupedArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[TL::LDS];
  const int total = p.tile_start[p.E] * p.ntn;
  const int G = gridDim.x, w = xcd_remap(blockIdx.x, G);
  for (int l = w; l < total; l += G) {
    grouped_tile<TL, B_T, EPI>(p, decode_tile<TL::BM>(p, l), smem);
    __syncthreads();  // the next tile's loads overwrite the epilogue's staging
  }
}

struct WgradArgs {
  const int32_t* offsets;  // [E+1]
  const int32_t* eorder;   // [E+1] experts longest first, then the skew flag
  int E, M, N, tm, tn;
  const uint16_t* A;       // [rows, M]: element (m, k) of expert e at A[(off_e + k)*M + m]
  const uint16_t* B;       // [rows, N]: element (n, k) at B[(off_e + k)*N + n]
  void* C;                 // [E, M, N] bf16 or fp32
};

template <class TL, bool OUT_F32>
__device__ __forceinline__ void wgrad_tile(const WgradArgs& p, int l, char* smem) {
  constexpr int BM = TL::BM, BN = TL::BN, WM = TL::WM, WN = TL::WN;
  constexpr int WMT = TL::WMT, WNT = TL::WNT, WAVES = TL::WAVES;

  const ExpertTile et = expert_tile(p.eorder, l, p.tm * p.tn);
  const int e = et.e;
  int mt, nt;
  wgrad_mn(et.rem, p.tm, p.tn, mt, nt);
  const int off = p.offsets[e];
  const int ne = p.offsets[e + 1] - off;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;

  f32x16 acc[WMT][WNT];
  zero(acc);
  const int ktiles = (ne + kBK - 1) / kBK;
  if (ktiles > 0) {
    TStager<BM, WAVES> sa;
    TStager<BN, WAVES> sb;
    // tokens past the expert's last row fall outside the resources and read as zeros
    sa.init(make_rsrc(p.A + size_t(off) * p.M + mt * BM, uint32_t(ne) * p.M * 2 - mt * BM * 2),
            p.M * 2, wave, lane);
    sb.init(make_rsrc(p.B + size_t(off) * p.N + nt * BN, uint32_t(ne) * p.N * 2 - nt * BN * 2),
            p.N * 2, wave, lane);
    mainloop<BM, BN, TL::WGM, TL::WGN, TL::STAGES, true, true, TL::WMT>(smem, sa, sb, ktiles, acc,
                                                                         wave, lane);
  }

  static_assert(TL::LDS >= wgrad_epi_lds<TL, OUT_F32>(), "epilogue staging exceeds LDS");
  wgrad_epilogue<TL, OUT_F32>(p.C, p.M, p.N, e, mt, nt, acc, wm, wn, lane, smem, threadIdx.x);
}

// Per-expert weight-gradient tiles (experts longest first), one workgroup per
// tile: their lengths follow the experts' token counts, and the hardware's
// dispatch of the next tile to whichever CU frees up balances them (resident
// workgroups in fixed rounds, as the grouped GEMM uses, lose 20-30% here under
// skewed routing and gain nothing under uniform routing).
template <class TL, bool OUT_F32>
__global__ void __launch_bounds__(TL::THREADS, 1) wgrad_gemm_kernel(WgradArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[TL::LDS];
  wgrad_tile<TL, OUT_F32>(p, expert_tile_start(p.eorder, p.E), smem);
}

// A token-grouped GEMM (TLA, B_T, EPI) and a weight gradient (TLB) in one
// launch over the paired schedule of moe_pair.h: a grid of resident
// workgroups takes items until every queue is exhausted.
template <class TLA, bool B_T, int EPI, class TLB, bool OUT_F32>
__global__ void __launch_bounds__(TLA::THREADS, 1) pair_kernel(GroupedArgs a, WgradArgs b,
                                                               PairSched ps) {
  static_assert(TLA::THREADS == TLB::THREADS, "one workgroup shape for both GEMMs");
  constexpr int PIPE = TLA::LDS > TLB::LDS ? TLA::LDS : TLB::LDS;
  __shared__ __attribute__((aligned(1024))) char smem[PIPE + sizeof(PairLds)];
  PairLds& L = *reinterpret_cast<PairLds*>(smem + PIPE);
  pair_setup<TLA::THREADS>(ps, L);
  int q = blockIdx.x % kPairQueues;
  for (;;) {
    const int g = pair_next(ps, L, &q);
    if (g < 0) break;
    const PairItem it = pair_decode(ps, L, g);
    if (it.is_a) grouped_tile<TLA, B_T, EPI>(a, decode_tile<TLA::BM>(a, it.l), smem);
    else wgrad_tile<TLB, OUT_F32>(b, it.l, smem);
    __syncthreads();  // the next item's loads overwrite this one's epilogue staging
  }
}

// ---------------------------------------------------------------------------
// Host-side launch helpers.

inline int max_mtiles(const moe_desc& d, int bm) {
  const long long N = (long long)d.T * d.K;
  return int((N + (long long)d.E * (bm - 1)) / bm);
}

inline int tile_index(int bm) { return bm == 64 ? 0 : (bm == 128 ? 1 : 2); }

template <class TL, bool B_T, int EPI>
int run_grouped(const moe_desc& d, const Layout& L, GroupedArgs a, int N, const char* name,
                char* scratch, hipStream_t s) {
  a.offsets = reinterpret_cast<const int32_t*>(scratch + L.offsets);
  a.tile_start = reinterpret_cast<const int32_t*>(scratch + L.tiles[tile_index(TL::BM)]);
  a.E = d.E;
  a.ntn = N / TL::BN;
  // n-tiles outer within an expert for the plain stores and W1 + SwiGLU (W2, W1
  // dgrad: a round's tiles then span all of an expert's m-tiles and fewer
  // n-tiles, 3-6% faster; W1 + SwiGLU: 1% at the 235B shape since its loads go
  // out in two sub-steps, equal at 30B); m-tiles outer for the SwiGLU backward
  // (n-tiles outer measured -1.6% at 30B and +1.6% at 235B there)
  a.nmajor = EPI == EPI_STORE || EPI == EPI_SWIGLU;
  const long long grid = (long long)max_mtiles(d, TL::BM) * a.ntn;
  if (grid <= 0) return MOE_OK;
  int resident;
  if (int rc = resident_grid<grouped_gemm_kernel<TL, B_T, EPI>>(TL::THREADS, &resident)) return rc;
  prof_begin(name, s);
  grouped_gemm_kernel<TL, B_T, EPI><<<unsigned(grid < resident ? grid : resident), TL::THREADS, 0, s>>>(a);
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

template <class TL, bool OUT_F32>
int run_wgrad(const moe_desc& d, const Layout& L, WgradArgs a, const char* name, char* scratch,
              hipStream_t s) {
  a.offsets = reinterpret_cast<const int32_t*>(scratch + L.offsets);
  a.eorder = reinterpret_cast<const int32_t*>(scratch + L.eorder);
  a.E = d.E;
  a.tm = a.M / TL::BM;
  a.tn = a.N / TL::BN;
  const long long grid = (long long)d.E * a.tm * a.tn;
  prof_begin(name, s);
  wgrad_gemm_kernel<TL, OUT_F32><<<unsigned(grid), TL::THREADS, 0, s>>>(a);
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// Tile choices (measured on the 30B shape: the 5-deep ring helps the W1 +
// SwiGLU GEMM by about 10% and none of the others); narrower fallbacks keep
// small shapes (D or F not a multiple of 256) working.
using TileBig = Tile<256, 256, 2, 4, 4>;
using TileBig5 = Tile<256, 256, 2, 4, 5>;  // whole 160 KB LDS: deeper ring for W1 + SwiGLU
using TileWide = Tile<256, 256, 2, 4, 2, true>;
using TileMid = Tile<128, 128, 2, 2, 4>;
using TileNarrow = Tile<128, 64, 2, 2, 4>;
using TileWg128x64 = Tile<128, 64, 2, 2, 4>;
using TileWg64x128 = Tile<64, 128, 2, 2, 4>;
using TileWg64x64 = Tile<64, 64, 2, 2, 4>;

template <bool B_T, int EPI>
int run_grouped_any(const moe_desc& d, const Layout& L, GroupedArgs a, int N, const char* name,
                    char* scratch, hipStream_t s) {
  if constexpr (!B_T)
    if (N % 256 == 0 && a.K % 64 == 0) return run_grouped<TileWide, B_T, EPI>(d, L, a, N, name, scratch, s);
  if constexpr (EPI == EPI_SWIGLU)
    if (N % 256 == 0) return run_grouped<TileBig5, B_T, EPI>(d, L, a, N, name, scratch, s);
  if (N % 256 == 0) return run_grouped<TileBig, B_T, EPI>(d, L, a, N, name, scratch, s);
  if (N % 128 == 0) return run_grouped<TileMid, B_T, EPI>(d, L, a, N, name, scratch, s);
  if constexpr (EPI != EPI_SWIGLU) return run_grouped<TileNarrow, B_T, EPI>(d, L, a, N, name, scratch, s);
  return MOE_EUNSUPPORTED;
}

template <bool OUT_F32>
int run_wgrad_any(const moe_desc& d, const Layout& L, WgradArgs a, const char* name,
                  char* scratch, hipStream_t s) {
  if (a.M % 256 == 0 && a.N % 256 == 0) return run_wgrad<TileBig, OUT_F32>(d, L, a, name, scratch, s);
  if (a.M % 128 == 0 && a.N % 128 == 0) return run_wgrad<TileMid, OUT_F32>(d, L, a, name, scratch, s);
  if (a.M % 128 == 0) return run_wgrad<TileWg128x64, OUT_F32>(d, L, a, name, scratch, s);
  if (a.N % 128 == 0) return run_wgrad<TileWg64x128, OUT_F32>(d, L, a, name, scratch, s);
  return run_wgrad<TileWg64x64, OUT_F32>(d, L, a, name, scratch, s);
}

// The token-grouped GEMM a (fully set up except for the routing pointers) and
// the weight gradient b in one paired launch; both on 256 x 256 tiles.
template <bool B_T, int EPI, bool OUT_F32>
int run_pair(const moe_desc& d, const Layout& L, GroupedArgs a, int N, WgradArgs b, int* ctr,
             const char* name, char* scratch, hipStream_t s) {
  using TA = TileBig;
  using TB = TileBig;
  a.offsets = reinterpret_cast<const int32_t*>(scratch + L.offsets);
  a.tile_start = reinterpret_cast<const int32_t*>(scratch + L.tiles[tile_index(TA::BM)]);
  a.E = d.E;
  a.ntn = N / TA::BN;
  a.nmajor = EPI == EPI_STORE;  // as the grouped GEMM launched alone
  b.offsets = a.offsets;
  b.eorder = reinterpret_cast<const int32_t*>(scratch + L.eorder);
  b.E = d.E;
  b.tm = b.M / TB::BM;
  b.tn = b.N / TB::BN;
  PairSched ps{};
  ps.offsets = a.offsets;
  ps.tstart = a.tile_start;
  ps.eorder = b.eorder;
  ps.E = d.E;
  ps.ntn = a.ntn;
  ps.per_b = b.tm * b.tn;
  ps.cost_a = a.K;
  ps.ctr = ctr;
  int resident;
  if (int rc = resident_grid<pair_kernel<TA, B_T, EPI, TB, OUT_F32>>(TA::THREADS, &resident)) return rc;
  prof_begin(name, s);
  pair_kernel<TA, B_T, EPI, TB, OUT_F32><<<unsigned(resident), TA::THREADS, 0, s>>>(a, b, ps);
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// Expert linear 1 with the SwiGLU epilogue; W1[e] is [2F, D].  Stores H into
// `h` and A into `act` (either may be null: the recompute forward skips H, the
// backward's recompute skips A).
int run_w1_swiglu(const moe_desc& d, const Layout& L, const uint16_t* w1, uint16_t* h,
                  uint16_t* act, const char* name, char* scratch, hipStream_t s,
                  const uint16_t* x = nullptr) {
  GroupedArgs a{};
  a.K = d.D;
  a.F = d.F;
  a.A = reinterpret_cast<const uint16_t*>(scratch + L.xperm);
  if (x != nullptr) {
    if (!w1_gathers(d)) return MOE_EINVAL;
    a.A = x;
    a.gather = reinterpret_cast<const int32_t*>(scratch + L.src);
    a.gK = d.K;
    a.gT = d.T;
    a.xcopy = reinterpret_cast<uint16_t*>(scratch + L.xperm);
    if (bf16_wide(d))  // A_w = w A (the routing wrote w_perm)
      a.rw = reinterpret_cast<const float*>(scratch + L.wperm);
  }
  a.lda = d.D;
  a.B = w1;
  a.bstride = int64_t(2) * d.F * d.D;
  a.ldb = d.D;
  a.brows = 2 * d.F;
  a.out = h;
  a.out2 = act;
  return run_grouped_any<false, EPI_SWIGLU>(d, L, a, 2 * d.F, name, scratch, s);
}

}  // namespace

int launch_recompute_h(const moe_desc& d, const Layout& L, const uint16_t* w1, char* scratch,
                       hipStream_t s) {
  return run_w1_swiglu(d, L, w1, reinterpret_cast<uint16_t*>(scratch + L.h), nullptr,
                       "gemm_w1_recompute", scratch, s);
}

int launch_fwd_gemms(const moe_desc& d, const Layout& L, const uint16_t* w1, const uint16_t* w2,
                     char* scratch, hipStream_t s, const uint16_t* x) {
  const int D = d.D, F = d.F;
  int rc = run_w1_swiglu(d, L, w1, L.recompute ? nullptr : reinterpret_cast<uint16_t*>(scratch + L.h),
                         reinterpret_cast<uint16_t*>(scratch + L.a), "gemm_w1_swiglu", scratch, s, x);
  if (rc) return rc;
  {  // expert linear 2: O.  W2[e] is [D, F].
    GroupedArgs a{};
    a.K = F;
    a.F = F;
    a.A = reinterpret_cast<const uint16_t*>(scratch + L.a);
    a.lda = F;
    a.B = w2;
    a.bstride = int64_t(D) * F;
    a.ldb = F;
    a.brows = D;
    a.out = reinterpret_cast<uint16_t*>(scratch + L.o);
    a.ldo = D;
    rc = run_grouped_any<false, EPI_STORE>(d, L, a, D, "gemm_w2", scratch, s);
    if (rc) return rc;
  }
  return MOE_OK;
}

// Paired by default in bf16 (measured 0.7-0.9% faster at the 30B and 235B
// shapes), on request in the FP8 modes (measured 2-3% slower there: their
// quantisers already sit between the GEMMs, and the paired launch needs the
// larger of the two tiles' LDS).
// The paired backward is the bf16 default only where experts are small on
// average (at most kPairDefaultTokens routed pairs each): at the Qwen3 shapes
// (1024 per expert) it gained 0.7-0.9%, but with 8192 per expert (the 16-expert
// EP-share workloads) it lost 8% at D = 4096 (an expert's dgrad and weight-
// gradient operands, tens of MB each, then thrash one XCD's L2 together) and
// 0.2% at D = 2048.
constexpr long long kPairDefaultTokens = 4096;

bool pair_capable(const moe_desc& d) {
  if (d.flags & MOE_FLAG_SERIAL_BWD) return false;
  const bool small_experts = (long long)d.T * d.K <= kPairDefaultTokens * d.E;
  const bool want = (d.flags & MOE_FLAG_OVERLAP_BWD) || (d.mode == MOE_BF16 && small_experts);
  return want && (d.mode == MOE_BF16 || fp8_mode(d.mode)) && d.D % 256 == 0 &&
         d.F % 256 == 0 && d.E <= kPairMaxE;
}

int launch_bwd_gemms(const moe_desc& d, const Layout& L, const uint16_t* w1, const uint16_t* w2,
                     void* dw1, void* dw2, bool dw_f32, char* scratch, hipStream_t s) {
  // bf16_wide: dYw_perm holds dy unscaled, A holds A_w = w A; the W2 dgrad applies w
  // (from w_perm) and writes the dProb partials
  const int D = d.D, F = d.F;
  int rc;
  // W2 wgrad: dW2[e] = sum_r dYw_perm[r] A[r]^T
  WgradArgs w2g{};
  w2g.M = D;
  w2g.N = F;
  w2g.A = reinterpret_cast<const uint16_t*>(scratch + L.dyperm);
  w2g.B = reinterpret_cast<const uint16_t*>(scratch + L.a);
  w2g.C = dw2;
  // W2 dgrad (dA = dYw W2[e], W2[e] is [D, F] = [K, N]) with SwiGLU-backward epilogue
  GroupedArgs w2d{};
  w2d.K = D;
  w2d.F = F;
  w2d.A = reinterpret_cast<const uint16_t*>(scratch + L.dyperm);
  w2d.lda = D;
  w2d.B = w2;
  w2d.bstride = int64_t(D) * F;
  w2d.ldb = F;
  w2d.brows = D;
  w2d.out = reinterpret_cast<uint16_t*>(scratch + L.dh);
  w2d.hsave = reinterpret_cast<const uint16_t*>(scratch + L.h);
  if (bf16_wide(d)) {
    w2d.rw = reinterpret_cast<const float*>(scratch + L.wperm);
    w2d.dpart = reinterpret_cast<float*>(scratch + L.dpart);
  }
  // W1 wgrad: dW1[e] = sum_r dH[r] x_perm[r]^T
  WgradArgs w1g{};
  w1g.M = 2 * F;
  w1g.N = D;
  w1g.A = reinterpret_cast<const uint16_t*>(scratch + L.dh);
  w1g.B = reinterpret_cast<const uint16_t*>(scratch + L.xperm);
  w1g.C = dw1;
  // W1 dgrad: dX_perm = dH W1[e], W1[e] is [2F, D] = [K, N]
  GroupedArgs w1d{};
  w1d.K = 2 * F;
  w1d.F = F;
  w1d.A = reinterpret_cast<const uint16_t*>(scratch + L.dh);
  w1d.lda = 2 * F;
  w1d.B = w1;
  w1d.bstride = int64_t(2) * F * D;
  w1d.ldb = D;
  w1d.brows = 2 * F;
  w1d.out = reinterpret_cast<uint16_t*>(scratch + L.dxperm);
  w1d.ldo = D;

  if (pair_capable(d) && !dw_f32) {
    // each dgrad beside its weight gradient, one launch per pair
    int* ctr = reinterpret_cast<int*>(scratch + L.pair);
    if ((rc = launch_zero(ctr, 2 * kPairQueues * sizeof(int), s))) return rc;
    if ((rc = run_pair<true, EPI_DSWIGLU, false>(d, L, w2d, F, w2g, ctr, "pair_w2", scratch, s)))
      return rc;
    return run_pair<true, EPI_STORE, false>(d, L, w1d, D, w1g, ctr + kPairQueues, "pair_w1",
                                            scratch, s);
  }
  // one kernel per GEMM.  The W2 weight gradient runs first (the W2 dgrad after
  // it then finds dYw in the caches, 5% faster at the 30B shape), and the W1
  // weight gradient before the W1 dgrad (so that the un-permute reads dX_perm
  // right after it is written)
  rc = dw_f32 ? run_wgrad_any<true>(d, L, w2g, "gemm_w2_wgrad", scratch, s)
              : run_wgrad_any<false>(d, L, w2g, "gemm_w2_wgrad", scratch, s);
  if (rc) return rc;
  if ((rc = run_grouped_any<true, EPI_DSWIGLU>(d, L, w2d, F, "gemm_w2_dgrad_dswiglu", scratch, s)))
    return rc;
  rc = dw_f32 ? run_wgrad_any<true>(d, L, w1g, "gemm_w1_wgrad", scratch, s)
              : run_wgrad_any<false>(d, L, w1g, "gemm_w1_wgrad", scratch, s);
  if (rc) return rc;
  return run_grouped_any<true, EPI_STORE>(d, L, w1d, D, "gemm_w1_dgrad", scratch, s);
}

}  // namespace moe
