// Grouped expert GEMMs of the MoE layer on CDNA4 matrix cores (bf16 in, fp32 accumulate).
//
// The pages fuse "the 2 expert linear layers" and SwiGLU into one kernel and add
// the backward pass (Prime Mega MoE news item, "How does the fused kernel
// work?").  On one GPU this file provides the six expert GEMMs of a training
// step, with the element-wise work fused into their epilogues:
//
//   fwd  W1 + SwiGLU  H = x_perm W1[e]^T, A = silu(H_gate) * H_up   (token-grouped, NT)
//   fwd  W2           O = A W2[e]^T                                 (token-grouped, NT)
//   bwd  W2 dgrad     G = dY_perm W2[e]; dH = SwiGLU'(H, w G); partial <G, A>  (NN)
//   bwd  W1 dgrad     dX_perm = dH W1[e]                            (token-grouped, NN)
//   bwd  W2 wgrad     dW2[e] = sum_r (w_r dY_perm[r]) A[r]^T         (per-expert, TN)
//   bwd  W1 wgrad     dW1[e] = sum_r dH[r] x_perm[r]^T               (per-expert, TN)
//
// Work decomposition: a 256-thread workgroup (four wave64s in a 2x2 grid) owns
// one BM x BN output tile; each wave accumulates (BM/2) x (BN/2) with
// v_mfma_f32_32x32x16_bf16.  K advances in steps of 64 through a double-buffered
// LDS stage: the next step's global loads are issued into registers before the
// current step's MFMAs and written to the other LDS buffer after them.
//
// LDS tiles hold R rows x 64 bf16 with the contraction index contiguous, so
// every MFMA operand fragment (8 consecutive k of one row) is one 16-byte
// ds_read.  The eight 16-byte chunks of a row are XOR-swizzled with (row & 7) so
// those reads and the staging writes spread over all banks.  Operands whose
// global layout has the contraction index outermost (weights in the dgrads,
// both operands of the wgrads) are transposed in registers while staging: each
// thread loads KB rows of 8 consecutive elements and writes 8 LDS rows of KB
// elements.
//
// Token-grouped GEMMs walk a flat list of (expert, m-tile, n-tile) built from
// the routing step's per-expert m-tile prefix sums; workgroups past the end
// return at once.  Per-expert GEMMs walk (expert, m-tile, n-tile) over the
// weight shape, with the contraction running over that expert's tokens (zero
// tokens -> zero gradient, no atomics).  Workgroup ids are remapped so that
// consecutive tiles of one expert land on the same XCD (hardware dispatch is
// round-robin over the 8 XCDs) and share its L2.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;

__device__ __forceinline__ int lds_idx(int row, int chunk) {
  return row * kBK + ((chunk ^ (row & 7)) << 3);
}

__device__ __forceinline__ int xcd_remap(int b, int G) {
  const int xcd = b & 7, local = b >> 3;
  const int q = G >> 3, r = G & 7;
  return xcd * q + (xcd < r ? xcd : r) + local;
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// ---------------------------------------------------------------------------
// Staging of an operand whose rows are contiguous along k (R rows x 64 k).
template <int R>
struct KRows {
  static constexpr int CPT = R / 32;  // 16-byte chunks per thread
  const uint16_t* rp[CPT];
  uint4 v[CPT];

  template <class RowPtr>
  __device__ __forceinline__ void init(RowPtr rowptr) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) rp[j] = rowptr((threadIdx.x + j * kThreads) >> 3);
  }
  __device__ __forceinline__ void load(int k0) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int ch = (threadIdx.x + j * kThreads) & 7;
      v[j] = rp[j] ? *reinterpret_cast<const uint4*>(rp[j] + k0 + ch * 8) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = threadIdx.x + j * kThreads;
      *reinterpret_cast<uint4*>(lds + lds_idx(c >> 3, c & 7)) = v[j];
    }
  }
};

// Staging of an operand stored with k outermost: element (row, k) at
// kptr(k)[row].  Each thread loads KB consecutive k of 8 consecutive rows and
// transposes them in registers.  With SCALED, k-row k is multiplied by kscale(k)
// (fp32) before rounding back to bf16.
template <int R, bool SCALED>
struct MNRows {
  static constexpr int KB = R / 32;      // k per thread: 8, 4 or 2
  static constexpr int KG = kBK / KB;    // threads along k
  uint4 v[KB];
  float sc[KB];
  int kb, mg;

  __device__ __forceinline__ void init() {
    kb = threadIdx.x % KG;
    mg = threadIdx.x / KG;
  }
  template <class KPtr, class KScale>
  __device__ __forceinline__ void load(KPtr kptr, KScale kscale, int k0) {
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int k = k0 + kb * KB + i;
      const uint16_t* p = kptr(k);
      v[i] = p ? *reinterpret_cast<const uint4*>(p + mg * 8) : make_uint4(0, 0, 0, 0);
      if constexpr (SCALED) sc[i] = p ? kscale(k) : 0.f;
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
    uint32_t w[KB][4];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const uint32_t in[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (SCALED) {
          const float lo = __uint_as_float(in[q] << 16) * sc[i];
          const float hi = __uint_as_float(in[q] & 0xffff0000u) * sc[i];
          w[i][q] = uint32_t(f2bf(lo)) | (uint32_t(f2bf(hi)) << 16);
        } else {
          w[i][q] = in[q];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = mg * 8 + j;
      uint32_t o[KB / 2];
#pragma unroll
      for (int q = 0; q < KB / 2; ++q) {
        const uint32_t a = w[2 * q][j >> 1], b = w[2 * q + 1][j >> 1];
        o[q] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      const int k = kb * KB;
      uint16_t* dst = lds + row * kBK + (((k >> 3) ^ (row & 7)) << 3) + (k & 7);
      if constexpr (KB == 8)
        *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
      else if constexpr (KB == 4)
        *reinterpret_cast<uint2*>(dst) = make_uint2(o[0], o[1]);
      else
        *reinterpret_cast<uint32_t*>(dst) = o[0];
    }
  }
};

// One 64-deep step of MFMAs for a wave's (WMT*32) x (WNT*32) sub-tile.
template <int WMT, int WNT>
__device__ __forceinline__ void mma_step(const uint16_t* la, const uint16_t* lb, int arow0,
                                         int brow0, int lane, f32x16 (&acc)[WMT][WNT]) {
  const int r = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < kBK / 16; ++kk) {
    const int ch = kk * 2 + hi;
    bf16x8 af[WMT], bfr[WNT];
#pragma unroll
    for (int i = 0; i < WMT; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(la + lds_idx(arow0 + i * 32 + r, ch));
#pragma unroll
    for (int j = 0; j < WNT; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8*>(lb + lds_idx(brow0 + j * 32 + r, ch));
#pragma unroll
    for (int i = 0; i < WMT; ++i)
#pragma unroll
      for (int j = 0; j < WNT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  }
}

// Row (within the wave's sub-tile) of accumulator element r of a 32x32 block.
__device__ __forceinline__ int acc_row(int r, int lane) {
  return (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
}

enum Epi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2 };

struct GroupedArgs {
  const int32_t* offsets;     // [E+1] first permuted row of each expert
  const int32_t* tile_start;  // [E+1] prefix sum of ceil(count/BM)
  int E, K, ntn, F;
  const uint16_t* A;          // [rows, K] permuted activations
  int lda;
  const uint16_t* B;          // weights of expert 0; expert e at B + e*bstride
  int64_t ldb, bstride;
  uint16_t* out;              // STORE: [rows, ldo]; SWIGLU: H [rows, 2F]; DSWIGLU: dH [rows, 2F]
  int ldo;
  uint16_t* out2;             // SWIGLU: A [rows, F]
  const uint16_t* hsave;      // DSWIGLU: H [rows, 2F]
  const uint16_t* asave;      // DSWIGLU: A [rows, F]
  const float* wperm;         // DSWIGLU: routing weight per permuted row
  float* part;                // DSWIGLU: [rows, pstride] partial <G, A> per n-tile half
  int pstride;
};

template <int BM, int BN, bool B_MN, int EPI>
__global__ void __launch_bounds__(kThreads, 1) grouped_gemm_kernel(GroupedArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2, WMT = WM / 32, WNT = WN / 32;
  static_assert(EPI != EPI_SWIGLU || WNT % 2 == 0, "SwiGLU pairs gate and up sub-tiles");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * kBK];

  const int l = xcd_remap(blockIdx.x, gridDim.x);
  const int mt_g = l / p.ntn, nt = l - mt_g * p.ntn;
  if (mt_g >= p.tile_start[p.E]) return;
  int lo = 0, hi = p.E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.tile_start[mid] <= mt_g) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int row0 = p.offsets[e] + (mt_g - p.tile_start[e]) * BM;
  const int rows_valid = min(BM, p.offsets[e + 1] - row0);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const uint16_t* Be = p.B + size_t(e) * p.bstride;

  KRows<BM> ga;
  ga.init([&](int r) -> const uint16_t* {
    return r < rows_valid ? p.A + size_t(row0 + r) * p.lda : nullptr;
  });
  KRows<BN> gbk;
  MNRows<BN, false> gbm;
  auto bk_ptr = [&](int k) -> const uint16_t* { return Be + size_t(k) * p.ldb + nt * BN; };
  auto no_scale = [](int) { return 1.f; };
  if constexpr (B_MN) {
    gbm.init();
  } else {
    gbk.init([&](int n) -> const uint16_t* {
      int row;
      if constexpr (EPI == EPI_SWIGLU) {
        const int w = n / WN, rem = n % WN;
        const int half = rem / (WN / 2), c = rem % (WN / 2);
        row = half * p.F + nt * (BN / 2) + w * (WN / 2) + c;
      } else {
        row = nt * BN + n;
      }
      return Be + size_t(row) * p.ldb;
    });
  }

  f32x16 acc[WMT][WNT];
#pragma unroll
  for (int i = 0; i < WMT; ++i)
#pragma unroll
    for (int j = 0; j < WNT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int ktiles = p.K / kBK;
  constexpr int kStage = (BM + BN) * kBK;
  ga.load(0);
  if constexpr (B_MN) gbm.load(bk_ptr, no_scale, 0); else gbk.load(0);
  ga.store(smem);
  if constexpr (B_MN) gbm.store(smem + BM * kBK); else gbk.store(smem + BM * kBK);
  __syncthreads();
  for (int kt = 0; kt < ktiles; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < ktiles;
    if (more) {
      ga.load((kt + 1) * kBK);
      if constexpr (B_MN) gbm.load(bk_ptr, no_scale, (kt + 1) * kBK); else gbk.load((kt + 1) * kBK);
    }
    uint16_t* sc = smem + cur * kStage;
    uint16_t* sn = smem + (cur ^ 1) * kStage;
    mma_step<WMT, WNT>(sc, sc + BM * kBK, wm * WM, wn * WN, lane, acc);
    if (more) {
      ga.store(sn);
      if constexpr (B_MN) gbm.store(sn + BM * kBK); else gbk.store(sn + BM * kBK);
    }
    __syncthreads();
  }

  const int col = lane & 31;
  if constexpr (EPI == EPI_STORE) {
#pragma unroll
    for (int i = 0; i < WMT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * WM + i * 32 + acc_row(r, lane);
        if (m < rows_valid) {
          uint16_t* o = p.out + size_t(row0 + m) * p.ldo + nt * BN + wn * WN + col;
#pragma unroll
          for (int j = 0; j < WNT; ++j) o[j * 32] = f2bf(acc[i][j][r]);
        }
      }
  } else if constexpr (EPI == EPI_SWIGLU) {
    const int F = p.F;
#pragma unroll
    for (int i = 0; i < WMT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * WM + i * 32 + acc_row(r, lane);
        if (m < rows_valid) {
          const size_t row = size_t(row0 + m);
#pragma unroll
          for (int j = 0; j < WNT / 2; ++j) {
            const int f = nt * (BN / 2) + wn * (WN / 2) + j * 32 + col;
            const float g = acc[i][j][r], u = acc[i][j + WNT / 2][r];
            const float a = g / (1.f + __expf(-g)) * u;
            p.out[row * 2 * F + f] = f2bf(g);
            p.out[row * 2 * F + F + f] = f2bf(u);
            p.out2[row * F + f] = f2bf(a);
          }
        }
      }
  } else {  // EPI_DSWIGLU
    const int F = p.F;
#pragma unroll
    for (int i = 0; i < WMT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * WM + i * 32 + acc_row(r, lane);
        float psum = 0.f;
        if (m < rows_valid) {
          const size_t row = size_t(row0 + m);
          const float w = p.wperm[row];
#pragma unroll
          for (int j = 0; j < WNT; ++j) {
            const int f = nt * BN + wn * WN + j * 32 + col;
            const float G = acc[i][j][r];
            psum += G * bf2f(p.asave[row * F + f]);
            const float g = bf2f(p.hsave[row * 2 * F + f]);
            const float u = bf2f(p.hsave[row * 2 * F + F + f]);
            const float s = 1.f / (1.f + __expf(-g));
            const float dA = w * G;
            p.out[row * 2 * F + f] = f2bf(dA * u * s * (1.f + g * (1.f - s)));
            p.out[row * 2 * F + F + f] = f2bf(dA * g * s);
          }
        }
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) psum += __shfl_xor(psum, off, 64);
        if (col == 0 && m < rows_valid)
          p.part[size_t(row0 + m) * p.pstride + nt * 2 + wn] = psum;
      }
  }
}

struct WgradArgs {
  const int32_t* offsets;  // [E+1]
  int E, M, N, tm, tn;
  const uint16_t* A;       // [rows, lda]: element (m, k) of expert e at A[(off_e + k)*lda + m]
  int lda;
  const uint16_t* B;       // [rows, ldb]: element (n, k) at B[(off_e + k)*ldb + n]
  int ldb;
  const float* kscale;     // per permuted row, multiplies A (SCALED only)
  void* C;                 // [E, M, N] bf16 or fp32
};

template <int BM, int BN, bool SCALED, bool OUT_F32>
__global__ void __launch_bounds__(kThreads, 1) wgrad_gemm_kernel(WgradArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2, WMT = WM / 32, WNT = WN / 32;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * kBK];

  const int l = xcd_remap(blockIdx.x, gridDim.x);
  const int per = p.tm * p.tn;
  const int e = l / per, rem = l - e * per;
  const int mt = rem / p.tn, nt = rem - mt * p.tn;
  const int off = p.offsets[e];
  const int ne = p.offsets[e + 1] - off;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  MNRows<BM, SCALED> ga;
  MNRows<BN, false> gb;
  ga.init();
  gb.init();
  auto a_ptr = [&](int k) -> const uint16_t* {
    return k < ne ? p.A + size_t(off + k) * p.lda + mt * BM : nullptr;
  };
  auto a_scale = [&](int k) -> float { return p.kscale[off + k]; };
  auto b_ptr = [&](int k) -> const uint16_t* {
    return k < ne ? p.B + size_t(off + k) * p.ldb + nt * BN : nullptr;
  };
  auto no_scale = [](int) { return 1.f; };

  f32x16 acc[WMT][WNT];
#pragma unroll
  for (int i = 0; i < WMT; ++i)
#pragma unroll
    for (int j = 0; j < WNT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int ktiles = (ne + kBK - 1) / kBK;
  if (ktiles > 0) {
    constexpr int kStage = (BM + BN) * kBK;
    ga.load(a_ptr, a_scale, 0);
    gb.load(b_ptr, no_scale, 0);
    ga.store(smem);
    gb.store(smem + BM * kBK);
    __syncthreads();
    for (int kt = 0; kt < ktiles; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < ktiles;
      if (more) {
        ga.load(a_ptr, a_scale, (kt + 1) * kBK);
        gb.load(b_ptr, no_scale, (kt + 1) * kBK);
      }
      uint16_t* sc = smem + cur * kStage;
      uint16_t* sn = smem + (cur ^ 1) * kStage;
      mma_step<WMT, WNT>(sc, sc + BM * kBK, wm * WM, wn * WN, lane, acc);
      if (more) {
        ga.store(sn);
        gb.store(sn + BM * kBK);
      }
      __syncthreads();
    }
  }

  const int col = lane & 31;
#pragma unroll
  for (int i = 0; i < WMT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = mt * BM + wm * WM + i * 32 + acc_row(r, lane);
      const size_t o = (size_t(e) * p.M + m) * p.N + nt * BN + wn * WN + col;
#pragma unroll
      for (int j = 0; j < WNT; ++j) {
        if constexpr (OUT_F32)
          reinterpret_cast<float*>(p.C)[o + j * 32] = acc[i][j][r];
        else
          reinterpret_cast<uint16_t*>(p.C)[o + j * 32] = f2bf(acc[i][j][r]);
      }
    }
}

// ---------------------------------------------------------------------------
// Host-side launch helpers.

inline int max_mtiles(const moe_desc& d, int bm) {
  const long long N = (long long)d.T * d.K;
  return int((N + (long long)d.E * (bm - 1)) / bm);
}

inline int tile_index(int bm) { return bm == 64 ? 0 : (bm == 128 ? 1 : 2); }

template <int BM, int BN, bool B_MN, int EPI>
int run_grouped(const moe_desc& d, const Layout& L, GroupedArgs a, const char* name,
                char* scratch, hipStream_t s) {
  a.offsets = reinterpret_cast<const int32_t*>(scratch + L.offsets);
  a.tile_start = reinterpret_cast<const int32_t*>(scratch + L.tiles[tile_index(BM)]);
  a.E = d.E;
  const long long grid = (long long)max_mtiles(d, BM) * a.ntn;
  if (grid <= 0) return MOE_OK;
  prof_begin(name, s);
  grouped_gemm_kernel<BM, BN, B_MN, EPI><<<unsigned(grid), kThreads, 0, s>>>(a);
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

template <int BM, int BN, bool SCALED, bool OUT_F32>
int run_wgrad(const moe_desc& d, const Layout& L, WgradArgs a, const char* name, char* scratch,
              hipStream_t s) {
  a.offsets = reinterpret_cast<const int32_t*>(scratch + L.offsets);
  a.E = d.E;
  a.tm = a.M / BM;
  a.tn = a.N / BN;
  const long long grid = (long long)d.E * a.tm * a.tn;
  prof_begin(name, s);
  wgrad_gemm_kernel<BM, BN, SCALED, OUT_F32><<<unsigned(grid), kThreads, 0, s>>>(a);
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

template <bool SCALED, bool OUT_F32>
int run_wgrad_any(const moe_desc& d, const Layout& L, WgradArgs a, const char* name,
                  char* scratch, hipStream_t s) {
  const bool m128 = a.M % 128 == 0, n128 = a.N % 128 == 0;
  if (m128 && n128) return run_wgrad<128, 128, SCALED, OUT_F32>(d, L, a, name, scratch, s);
  if (m128) return run_wgrad<128, 64, SCALED, OUT_F32>(d, L, a, name, scratch, s);
  if (n128) return run_wgrad<64, 128, SCALED, OUT_F32>(d, L, a, name, scratch, s);
  return run_wgrad<64, 64, SCALED, OUT_F32>(d, L, a, name, scratch, s);
}

}  // namespace

int launch_fwd_gemms(const moe_desc& d, const Layout& L, const uint16_t* w1, const uint16_t* w2,
                     char* scratch, hipStream_t s) {
  const int D = d.D, F = d.F;
  int rc;
  {  // expert linear 1 with SwiGLU epilogue: H, A
    GroupedArgs a{};
    a.K = D;
    a.F = F;
    a.A = reinterpret_cast<const uint16_t*>(scratch + L.xperm);
    a.lda = D;
    a.B = w1;
    a.ldb = D;
    a.bstride = int64_t(2) * F * D;
    a.out = reinterpret_cast<uint16_t*>(scratch + L.h);
    a.out2 = reinterpret_cast<uint16_t*>(scratch + L.a);
    if (F % 128 == 0) {
      a.ntn = 2 * F / 256;
      rc = run_grouped<128, 256, false, EPI_SWIGLU>(d, L, a, "gemm_w1_swiglu", scratch, s);
    } else {
      a.ntn = 2 * F / 128;
      rc = run_grouped<128, 128, false, EPI_SWIGLU>(d, L, a, "gemm_w1_swiglu", scratch, s);
    }
    if (rc) return rc;
  }
  {  // expert linear 2: O
    GroupedArgs a{};
    a.K = F;
    a.F = F;
    a.A = reinterpret_cast<const uint16_t*>(scratch + L.a);
    a.lda = F;
    a.B = w2;
    a.ldb = F;
    a.bstride = int64_t(D) * F;
    a.out = reinterpret_cast<uint16_t*>(scratch + L.o);
    a.ldo = D;
    if (D % 256 == 0) {
      a.ntn = D / 256;
      rc = run_grouped<128, 256, false, EPI_STORE>(d, L, a, "gemm_w2", scratch, s);
    } else if (D % 128 == 0) {
      a.ntn = D / 128;
      rc = run_grouped<128, 128, false, EPI_STORE>(d, L, a, "gemm_w2", scratch, s);
    } else {
      a.ntn = D / 64;
      rc = run_grouped<128, 64, false, EPI_STORE>(d, L, a, "gemm_w2", scratch, s);
    }
    if (rc) return rc;
  }
  return MOE_OK;
}

int launch_bwd_gemms(const moe_desc& d, const Layout& L, const uint16_t* w1, const uint16_t* w2,
                     void* dw1, void* dw2, bool dw_f32, int* nparts, char* scratch,
                     hipStream_t s) {
  const int D = d.D, F = d.F;
  int rc;
  {  // W2 dgrad with SwiGLU-backward, routing weight and partial <dy, o> in the epilogue
    GroupedArgs a{};
    a.K = D;
    a.F = F;
    a.A = reinterpret_cast<const uint16_t*>(scratch + L.dyperm);
    a.lda = D;
    a.B = w2;
    a.ldb = F;
    a.bstride = int64_t(D) * F;
    a.out = reinterpret_cast<uint16_t*>(scratch + L.dh);
    a.hsave = reinterpret_cast<const uint16_t*>(scratch + L.h);
    a.asave = reinterpret_cast<const uint16_t*>(scratch + L.a);
    a.wperm = reinterpret_cast<const float*>(scratch + L.wperm);
    a.part = reinterpret_cast<float*>(scratch + L.dprob_part);
    a.pstride = L.nparts_max;
    if (F % 128 == 0) {
      a.ntn = F / 128;
      rc = run_grouped<128, 128, true, EPI_DSWIGLU>(d, L, a, "gemm_w2_dgrad_dswiglu", scratch, s);
    } else {
      a.ntn = F / 64;
      rc = run_grouped<128, 64, true, EPI_DSWIGLU>(d, L, a, "gemm_w2_dgrad_dswiglu", scratch, s);
    }
    *nparts = 2 * a.ntn;
    if (rc) return rc;
  }
  {  // W2 wgrad: dW2[e] = sum_r (w_r dY_perm[r]) A[r]^T
    WgradArgs a{};
    a.M = D;
    a.N = F;
    a.A = reinterpret_cast<const uint16_t*>(scratch + L.dyperm);
    a.lda = D;
    a.kscale = reinterpret_cast<const float*>(scratch + L.wperm);
    a.B = reinterpret_cast<const uint16_t*>(scratch + L.a);
    a.ldb = F;
    a.C = dw2;
    rc = dw_f32 ? run_wgrad_any<true, true>(d, L, a, "gemm_w2_wgrad", scratch, s)
                : run_wgrad_any<true, false>(d, L, a, "gemm_w2_wgrad", scratch, s);
    if (rc) return rc;
  }
  {  // W1 dgrad: dX_perm = dH W1[e]
    GroupedArgs a{};
    a.K = 2 * F;
    a.F = F;
    a.A = reinterpret_cast<const uint16_t*>(scratch + L.dh);
    a.lda = 2 * F;
    a.B = w1;
    a.ldb = D;
    a.bstride = int64_t(2) * F * D;
    a.out = reinterpret_cast<uint16_t*>(scratch + L.dxperm);
    a.ldo = D;
    if (D % 256 == 0) {
      a.ntn = D / 256;
      rc = run_grouped<128, 256, true, EPI_STORE>(d, L, a, "gemm_w1_dgrad", scratch, s);
    } else if (D % 128 == 0) {
      a.ntn = D / 128;
      rc = run_grouped<128, 128, true, EPI_STORE>(d, L, a, "gemm_w1_dgrad", scratch, s);
    } else {
      a.ntn = D / 64;
      rc = run_grouped<128, 64, true, EPI_STORE>(d, L, a, "gemm_w1_dgrad", scratch, s);
    }
    if (rc) return rc;
  }
  {  // W1 wgrad: dW1[e] = sum_r dH[r] x_perm[r]^T
    WgradArgs a{};
    a.M = 2 * F;
    a.N = D;
    a.A = reinterpret_cast<const uint16_t*>(scratch + L.dh);
    a.lda = 2 * F;
    a.B = reinterpret_cast<const uint16_t*>(scratch + L.xperm);
    a.ldb = D;
    a.C = dw1;
    rc = dw_f32 ? run_wgrad_any<false, true>(d, L, a, "gemm_w1_wgrad", scratch, s)
                : run_wgrad_any<false, false>(d, L, a, "gemm_w1_wgrad", scratch, s);
    if (rc) return rc;
  }
  return MOE_OK;
}

}  // namespace moe
