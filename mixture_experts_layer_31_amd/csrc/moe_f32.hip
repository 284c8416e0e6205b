// fp32 expert GEMMs of the MoE layer (mode MOE_FP32: fp32 storage and fp32
// arithmetic end to end).  Same six products and fused epilogues as the bf16
// kernels (moe_gemm.hip): W1 + SwiGLU and W2 over token-grouped rows, the W2
// dgrad with the SwiGLU backward, the W1 dgrad, and the two per-expert weight
// gradients contracted over each expert's tokens.
//
// This mode exists for the fp32 workloads (the tiny parity layer); it is not a
// throughput path, so the kernels are plain LDS-tiled vector-ALU GEMMs: a
// 256-thread workgroup owns a 64 x 64 output tile, the contraction advances 16
// at a time through two LDS panels, and each thread accumulates a 4 x 4 block
// with fused multiply-adds.  Rows past an expert's end and tokens past its last
// row read as zeros.
#include "moe_common.h"

namespace moe {

namespace {

constexpr int kT = 64;    // tile rows and columns
constexpr int kKs = 16;   // contraction step
constexpr int kThr = 256;
enum { F32_STORE = 0, F32_SWIGLU = 1, F32_DSWIGLU = 2 };

struct F32Grouped {
  const int32_t* offsets;     // [E+1]
  const int32_t* tile_start;  // [E+1] prefix sum of ceil(count / 64)
  int E, K, ntn, F;
  const float* A;             // [rows, K] permuted rows (contraction contiguous)
  int lda;
  const float* B;             // weights of expert 0; expert e at B + e * bstride
  int64_t bstride;
  int ldb;
  float* out;                 // STORE: [rows, ldo]; SWIGLU: H [rows, 2F] or null; DSWIGLU: dH [rows, 2F]
  int ldo;
  float* out2;                // SWIGLU: A [rows, F] or null
  const float* hsave;         // DSWIGLU: H [rows, 2F] (may equal out: each thread reads its
                              // g and u before it stores their gradients)
};

__device__ __forceinline__ float sigmoidf(float z) { return 1.f / (1.f + expf(-z)); }

// Tile column handled by thread column tx, slot j.  SwiGLU tiles hold 32 gate
// and the matching 32 up columns; each thread takes two of each so that the
// epilogue has gate and up of the same feature in registers.
template <int EPI>
__device__ __forceinline__ int tile_col(int tx, int j) {
  if constexpr (EPI == F32_SWIGLU) return j < 2 ? 2 * tx + j : 32 + 2 * tx + (j - 2);
  else return 4 * tx + j;
}

// B_T = false: B[e] is [N, K] (row n holds the k-run); true: B[e] is [K, N].
template <bool B_T, int EPI>
__global__ void __launch_bounds__(kThr) f32_grouped_kernel(F32Grouped p) {
  const int l = blockIdx.x;
  const int mt = l / p.ntn, nt = l - mt * p.ntn;
  if (mt >= p.tile_start[p.E]) return;
  int lo = 0, hi = p.E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.tile_start[mid] <= mt) lo = mid; else hi = mid;
  }
  const int e = lo, e0 = p.offsets[e], ne = p.offsets[e + 1] - e0;
  const int m0 = (mt - p.tile_start[e]) * kT;
  const int rows = min(kT, ne - m0);
  const float* Be = p.B + size_t(e) * p.bstride;

  __shared__ float As[kKs][kT + 4], Bs[kKs][kT + 4];
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += kKs) {
#pragma unroll
    for (int j = 0; j < kT * kKs / kThr; ++j) {
      const int idx = tid + j * kThr;
      const int r = idx / kKs, kk = idx % kKs;
      As[kk][r] = r < rows ? p.A[size_t(e0 + m0 + r) * p.lda + k0 + kk] : 0.f;
      if constexpr (B_T) {
        const int kb = idx / kT, n = idx % kT;
        Bs[kb][n] = Be[size_t(k0 + kb) * p.ldb + nt * kT + n];
      } else {
        int brow;
        if constexpr (EPI == F32_SWIGLU) brow = r < 32 ? nt * 32 + r : p.F + nt * 32 + (r - 32);
        else brow = nt * kT + r;
        Bs[kk][r] = Be[size_t(brow) * p.ldb + k0 + kk];
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kKs; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tile_col<EPI>(tx, j)];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    if (r >= rows) continue;
    const size_t row = size_t(e0 + m0 + r);
    if constexpr (EPI == F32_STORE) {
#pragma unroll
      for (int j = 0; j < 4; ++j) p.out[row * p.ldo + nt * kT + 4 * tx + j] = acc[i][j];
    } else if constexpr (EPI == F32_SWIGLU) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int f = nt * 32 + 2 * tx + j;
        const float g = acc[i][j], u = acc[i][2 + j];
        if (p.out != nullptr) {
          p.out[row * 2 * p.F + f] = g;
          p.out[row * 2 * p.F + p.F + f] = u;
        }
        if (p.out2 != nullptr) p.out2[row * p.F + f] = g * sigmoidf(g) * u;
      }
    } else {  // DSWIGLU: acc is dA for features nt*64 + 4tx + j
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int f = nt * kT + 4 * tx + j;
        const float g = p.hsave[row * 2 * p.F + f], u = p.hsave[row * 2 * p.F + p.F + f];
        const float sg = sigmoidf(g), dA = acc[i][j];
        p.out[row * 2 * p.F + f] = dA * u * sg * (1.f + g * (1.f - sg));
        p.out[row * 2 * p.F + p.F + f] = dA * g * sg;
      }
    }
  }
}

struct F32Wgrad {
  const int32_t* offsets;  // [E+1]
  int E, M, N, tm, tn;
  const float* A;          // [rows, M]: element (m, k) of expert e at A[(off_e + k) * M + m]
  const float* B;          // [rows, N]: element (n, k) at B[(off_e + k) * N + n]
  float* C;                // [E, M, N]
};

__global__ void __launch_bounds__(kThr) f32_wgrad_kernel(F32Wgrad p) {
  const int l = blockIdx.x, per = p.tm * p.tn;
  const int e = l / per, rem = l - e * per, mt = rem / p.tn, nt = rem - mt * p.tn;
  const int off = p.offsets[e], ne = p.offsets[e + 1] - off;
  __shared__ float As[kKs][kT + 4], Bs[kKs][kT + 4];
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < ne; k0 += kKs) {
#pragma unroll
    for (int j = 0; j < kT * kKs / kThr; ++j) {
      const int idx = tid + j * kThr;
      const int kk = idx / kT, c = idx % kT;
      const bool ok = k0 + kk < ne;
      As[kk][c] = ok ? p.A[size_t(off + k0 + kk) * p.M + mt * kT + c] : 0.f;
      Bs[kk][c] = ok ? p.B[size_t(off + k0 + kk) * p.N + nt * kT + c] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kKs; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][4 * tx + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      p.C[(size_t(e) * p.M + mt * kT + ty * 4 + i) * p.N + nt * kT + 4 * tx + j] = acc[i][j];
}

inline int max_mtiles64(const moe_desc& d) {
  const long long N = (long long)d.T * d.K;
  return int((N + (long long)d.E * (kT - 1)) / kT);
}

template <bool B_T, int EPI>
int run_f32(const moe_desc& d, const Layout& L, F32Grouped a, int ntn, const char* name,
            char* scratch, hipStream_t s) {
  a.offsets = reinterpret_cast<const int32_t*>(scratch + L.offsets);
  a.tile_start = reinterpret_cast<const int32_t*>(scratch + L.tiles[0]);
  a.E = d.E;
  a.ntn = ntn;
  const long long grid = (long long)max_mtiles64(d) * ntn;
  if (grid <= 0) return MOE_OK;
  prof_begin(name, s);
  f32_grouped_kernel<B_T, EPI><<<unsigned(grid), kThr, 0, s>>>(a);
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int run_f32_wgrad(const moe_desc& d, const Layout& L, F32Wgrad a, const char* name, char* scratch,
                  hipStream_t s) {
  a.offsets = reinterpret_cast<const int32_t*>(scratch + L.offsets);
  a.E = d.E;
  a.tm = a.M / kT;
  a.tn = a.N / kT;
  prof_begin(name, s);
  f32_wgrad_kernel<<<unsigned(d.E * a.tm * a.tn), kThr, 0, s>>>(a);
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace

int launch_fwd_gemms_f32(const moe_desc& d, const Layout& L, const float* w1, const float* w2,
                         char* scratch, hipStream_t s) {
  const int D = d.D, F = d.F;
  int rc;
  {  // H = x_perm W1[e]^T with A = silu(gate) * up; W1[e] is [2F, D]
    F32Grouped a{};
    a.K = D;
    a.F = F;
    a.A = reinterpret_cast<const float*>(scratch + L.xperm);
    a.lda = D;
    a.B = w1;
    a.bstride = int64_t(2) * F * D;
    a.ldb = D;
    a.out = L.recompute ? nullptr : reinterpret_cast<float*>(scratch + L.h);
    a.out2 = reinterpret_cast<float*>(scratch + L.a);
    if ((rc = run_f32<false, F32_SWIGLU>(d, L, a, F / 32, "gemm_w1_swiglu", scratch, s))) return rc;
  }
  {  // O = A W2[e]^T; W2[e] is [D, F]
    F32Grouped a{};
    a.K = F;
    a.F = F;
    a.A = reinterpret_cast<const float*>(scratch + L.a);
    a.lda = F;
    a.B = w2;
    a.bstride = int64_t(D) * F;
    a.ldb = F;
    a.out = reinterpret_cast<float*>(scratch + L.o);
    a.ldo = D;
    if ((rc = run_f32<false, F32_STORE>(d, L, a, D / kT, "gemm_w2", scratch, s))) return rc;
  }
  return MOE_OK;
}

int launch_recompute_h_f32(const moe_desc& d, const Layout& L, const float* w1, char* scratch,
                           hipStream_t s) {
  F32Grouped a{};
  a.K = d.D;
  a.F = d.F;
  a.A = reinterpret_cast<const float*>(scratch + L.xperm);
  a.lda = d.D;
  a.B = w1;
  a.bstride = int64_t(2) * d.F * d.D;
  a.ldb = d.D;
  a.out = reinterpret_cast<float*>(scratch + L.h);
  a.out2 = nullptr;
  return run_f32<false, F32_SWIGLU>(d, L, a, d.F / 32, "gemm_w1_recompute", scratch, s);
}

int launch_bwd_gemms_f32(const moe_desc& d, const Layout& L, const float* w1, const float* w2,
                         float* dw1, float* dw2, char* scratch, hipStream_t s) {
  const int D = d.D, F = d.F;
  int rc;
  {  // dA = dYw_perm W2[e] ([rows, D] x [D, F]) with the SwiGLU backward -> dH
    F32Grouped a{};
    a.K = D;
    a.F = F;
    a.A = reinterpret_cast<const float*>(scratch + L.dyperm);
    a.lda = D;
    a.B = w2;
    a.bstride = int64_t(D) * F;
    a.ldb = F;
    a.out = reinterpret_cast<float*>(scratch + L.dh);
    a.hsave = reinterpret_cast<const float*>(scratch + L.h);
    if ((rc = run_f32<true, F32_DSWIGLU>(d, L, a, F / kT, "gemm_w2_dgrad_dswiglu", scratch, s)))
      return rc;
  }
  {  // dW2[e] = sum_r dYw_perm[r] A[r]^T  ([D, F])
    F32Wgrad a{};
    a.M = D;
    a.N = F;
    a.A = reinterpret_cast<const float*>(scratch + L.dyperm);
    a.B = reinterpret_cast<const float*>(scratch + L.a);
    a.C = dw2;
    if ((rc = run_f32_wgrad(d, L, a, "gemm_w2_wgrad", scratch, s))) return rc;
  }
  {  // dX_perm = dH W1[e]  ([rows, 2F] x [2F, D])
    F32Grouped a{};
    a.K = 2 * F;
    a.F = F;
    a.A = reinterpret_cast<const float*>(scratch + L.dh);
    a.lda = 2 * F;
    a.B = w1;
    a.bstride = int64_t(2) * F * D;
    a.ldb = D;
    a.out = reinterpret_cast<float*>(scratch + L.dxperm);
    a.ldo = D;
    if ((rc = run_f32<true, F32_STORE>(d, L, a, D / kT, "gemm_w1_dgrad", scratch, s))) return rc;
  }
  {  // dW1[e] = sum_r dH[r] x_perm[r]^T  ([2F, D])
    F32Wgrad a{};
    a.M = 2 * F;
    a.N = D;
    a.A = reinterpret_cast<const float*>(scratch + L.dh);
    a.B = reinterpret_cast<const float*>(scratch + L.xperm);
    a.C = dw1;
    if ((rc = run_f32_wgrad(d, L, a, "gemm_w1_wgrad", scratch, s))) return rc;
  }
  return MOE_OK;
}

}  // namespace moe
