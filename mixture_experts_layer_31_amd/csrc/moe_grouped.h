// Token-grouped GEMM tile: arguments, tile coordinates and the tile body,
// shared by the one-launch-per-GEMM kernels and the persistent forward.
#pragma once

#include "moe_gemm_common.h"

namespace moe {
namespace gemm {

struct GroupedArgs {
  const int32_t* offsets;     // [E+1] first permuted row of each expert
  const int32_t* tile_start;  // [E+1] prefix sum of ceil(count/BM)
  int E, K, ntn, F;
  const uint16_t* A;          // [rows, K] permuted activations (k-contiguous)
  int lda;
  const uint16_t* B;          // weights of expert 0; expert e at B + e*bstride
  int64_t bstride;
  int ldb;                    // row length of a weight matrix (elements)
  int brows;                  // rows of a weight matrix
  uint16_t* out;              // STORE: [rows, ldo]; SWIGLU: H [rows, 2F] or null; DSWIGLU: dH [rows, 2F]
  int ldo;
  uint16_t* out2;             // SWIGLU: A [rows, F] or null
  const uint16_t* hsave;      // DSWIGLU: H [rows, 2F] (may equal out: read before written, per tile)
  int nmajor;                 // tile order within an expert: n-tiles outer (1) or m-tiles outer (0)
  const int32_t* gather;      // null: A holds the permuted rows; else A is [T, lda] token rows and
  int gK;                     //   permuted row q reads token row gather[q] / gK (wide-row loop only)
  int gT;                     //   token rows in A
  const float* rw;            // routing weights carried by the epilogue (SWIGLU: A_w = w A,
  const int32_t* rsrc;        //   row r's weight rw[rsrc[r]], or rw[r] if rsrc is null;
                              //   DSWIGLU: dA = w G with row r's weight rw[r]); null: none
  float* dpart;               // DSWIGLU with rw: dProb partials [rows, F / 64]
  uint16_t* xcopy;            // gather (SwiGLU epilogue only): the permuted rows [N, lda], k-step
                              //   kt of an m-tile written by its n-tile kt % ntn
};

// Where flat tile l sits: experts in order, and within an expert either
// m-tile * ntn + n-tile (nmajor 0) or n-tile * (its m-tiles) + m-tile (nmajor 1).
struct TileCoord {
  int e, e0, ne;     // expert, its first permuted row, its row count
  int mt_g, nt;      // global m-tile index, n-tile index
  int m0;            // first row of the tile within the expert
  int rows_valid;    // rows of the tile that exist (1..BM)
};

template <int BM>
__device__ __forceinline__ TileCoord decode_tile(const GroupedArgs& p, int l) {
  TileCoord c;
  int lo;
  if (p.nmajor) {  // expert e owns flat tiles [tile_start[e] * ntn, tile_start[e + 1] * ntn)
    lo = tile_expert(p.tile_start, p.E, p.ntn, l);
    const int t0 = p.tile_start[lo], mte = p.tile_start[lo + 1] - t0;
    const int local = l - t0 * p.ntn;
    c.nt = local / mte;
    c.mt_g = t0 + (local - c.nt * mte);
  } else {
    c.mt_g = l / p.ntn;
    c.nt = l - c.mt_g * p.ntn;
    lo = tile_expert(p.tile_start, p.E, 1, c.mt_g);
  }
  c.e = lo;
  c.e0 = p.offsets[c.e];
  c.ne = p.offsets[c.e + 1] - c.e0;
  c.m0 = (c.mt_g - p.tile_start[c.e]) * BM;
  c.rows_valid = min(BM, c.ne - c.m0);
  return c;
}

// One BM x BN output tile.  B_T = false: B[e] is [N, K] (row n holds the
// k-run); true: B[e] is [K, N].  COH2: the SwiGLU activation output is written
// with device-coherent stores (read by other workgroups in the same launch).
template <class TL, bool B_T, int EPI, bool COH2 = false>
__device__ __forceinline__ void grouped_tile(const GroupedArgs& p, const TileCoord& c, char* smem) {
  constexpr int BM = TL::BM, BN = TL::BN, WN = TL::WN;
  constexpr int WMT = TL::WMT, WNT = TL::WNT, WAVES = TL::WAVES;
  static_assert(EPI != EPI_SWIGLU || (WNT % 2 == 0 && !B_T), "SwiGLU pairs gate/up sub-tiles");
  static_assert(TL::LDS >= grouped_epi_lds<TL, EPI>(), "epilogue staging exceeds LDS");
  const int e = c.e, e0 = c.e0, ne = c.ne, m0 = c.m0, nt = c.nt, rows_valid = c.rows_valid;

  const int tid = opaque_tid();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;

  constexpr int ROWB = TL::WIDE ? 128 : kBK * 2;  // bytes of a k-step's row
  static_assert(!TL::WIDE || !B_T, "the wide-row loop takes k-contiguous operands");
  KStager<BM, WAVES, ROWB> sa;
  constexpr bool CAN_GATHER = TL::WIDE && EPI == EPI_SWIGLU;
  const bool gathered = CAN_GATHER && p.gather != nullptr;
  if (gathered) {
    const int32_t* g = p.gather + e0 + m0;
    sa.init(make_rsrc(p.A, uint32_t(p.gT) * p.lda * 2),
            [&](int r) { return r < rows_valid ? (g[r] / p.gK) * p.lda * 2 : -1; }, wave, lane);
  } else {
    sa.init(make_rsrc(p.A + size_t(e0) * p.lda, uint32_t(ne) * p.lda * 2),
            [&](int r) { return r < rows_valid ? (m0 + r) * p.lda * 2 : -1; }, wave, lane);
  }
  const uint16_t* Be = p.B + size_t(e) * p.bstride;
  const uint32_t bbytes = uint32_t(p.brows) * p.ldb * 2;
  EpiArgs ea{p.out, p.ldo, p.out2, p.hsave, p.F};
  if constexpr (EPI == EPI_SWIGLU) {  // the routing weights of the lane's rows, ahead of the main loop
    static_assert(WMT <= 4, "one routing weight per 32-row block");
#pragma unroll
    for (int i = 0; i < WMT; ++i) {
      const int trow = wm * TL::WM + i * 32 + (lane & 31);
      const int r = e0 + m0 + trow;
      ea.wrow[i] = p.rw == nullptr ? 1.f  // no routing weights: A itself
                   : trow < rows_valid ? p.rw[p.rsrc != nullptr ? p.rsrc[r] : r] : 0.f;
    }
  } else if constexpr (EPI == EPI_DSWIGLU) {  // loaded by the epilogue (rsrc unused)
    ea.wp = p.rw;
    ea.dpart = p.dpart;
  }
  f32x16 acc[WMT][WNT];
  zero(acc);
  const int ktiles = p.K / (ROWB / 2);
  // 32-row blocks of this wave's share of the tile that hold rows
  const int act = min(WMT, max(0, (rows_valid - wm * TL::WM + 31) / 32));
  if constexpr (B_T) {
    TStager<BN, WAVES> sb;
    sb.init(make_rsrc(Be + nt * BN, bbytes - nt * BN * 2), p.ldb * 2, wave, lane);
    with_active<WMT>(act, [&](auto a) {
      mainloop<BM, BN, TL::WGM, TL::WGN, TL::STAGES, false, true, decltype(a)::value>(
          smem, sa, sb, ktiles, acc, wave, lane);
    });
  } else {
    KStager<BN, WAVES, ROWB> sb;
    sb.init(make_rsrc(Be, bbytes),
            [&](int n) {
              int row;
              if constexpr (EPI == EPI_SWIGLU) {
                const int w = n / WN, rem = n % WN;
                const int half = rem / (WN / 2), cc = rem % (WN / 2);
                row = half * p.F + nt * (BN / 2) + w * (WN / 2) + cc;
              } else {
                row = nt * BN + n;
              }
              return row * p.ldb * 2;
            },
            wave, lane);
    with_active<WMT>(act, [&](auto a) {
      if constexpr (TL::WIDE) {
        bool copy = false;
        if constexpr (CAN_GATHER) copy = gathered && p.xcopy != nullptr;
        if (copy) {
          if constexpr (CAN_GATHER) {
            // k-step kt's 128-byte row segments of A, from LDS to the permuted rows, by the
            // n-tile kt % ntn (the m-tile's n-tiles share the copy evenly), with streaming
            // stores (read only by the backward: W1 0.993 -> 0.977 ms at 30B against plain)
            uint16_t* xc = p.xcopy + (size_t(e0) + m0) * p.lda;
            const int lda = p.lda, ntn = p.ntn;
            mainloop_w<BM, BN, TL::WGM, TL::WGN, decltype(a)::value>(
                smem, sa, sb, ktiles, acc, wave, lane, [&](int kt, const char* ta) {
                  if (kt % ntn != nt) return;
                  const int tid = wave * 64 + lane;
#pragma unroll
                  for (int i = 0; i < BM * 8 / TL::THREADS; ++i) {
                    const int c = tid + i * TL::THREADS, r = c >> 3, ch = c & 7;
                    if (r < rows_valid)
                      store16_nt(xc + size_t(r) * lda + kt * 64 + ch * 8,
                                 *reinterpret_cast<const uint4*>(ta + r * 128 + ((ch ^ swz_row<128>(r)) << 4)));
                  }
                });
          }
        } else {
          mainloop_w<BM, BN, TL::WGM, TL::WGN, decltype(a)::value>(smem, sa, sb, ktiles, acc,
                                                                   wave, lane);
        }
      }
      else
        mainloop<BM, BN, TL::WGM, TL::WGN, TL::STAGES, false, false, decltype(a)::value>(
            smem, sa, sb, ktiles, acc, wave, lane);
    });
  }

  // the dgrads' plain stores (dX_perm, read once by the un-permute after the launch) stream
  // past the caches, which keep the operands of the tiles still running
  grouped_epilogue<TL, EPI, COH2, TL::LDS, true, B_T>(ea, acc, size_t(e0) + m0, rows_valid, nt, wm,
                                                     wn, lane, smem, tid);
}

}  // namespace gemm
}  // namespace moe
