// HBM-bound row movers of the MoE layer: dispatch, combine, combine-backward, un-permute.
//
// Dispatch copies every token row to the expert-contiguous row of each of its
// routed pairs (the single-GPU form of the pages' expert-parallel dispatch,
// Prime Mega MoE news item, "How does the fused kernel work?").  Combine is the
// weighted gather-reduce y_t = sum_k w[t,k] o_{t,k}; the un-permute reduction
// is the same gather-reduce of the dx rows without weights.  Gathering per
// token (instead of scattering per pair with atomics) makes both deterministic:
// every output element is one fp32 sum over k in ascending order, rounded once.
//
// Each token row is read once and written K times (dispatch), or read K times
// and written once (combine): T*D*b + T*K*D*b bytes plus the index traffic.
// A group of TPR = min(256, D/8) threads owns one token row; a thread moves
// 16 bytes (8 bf16) per access, so a wavefront touches whole 128-byte lines.
#include <type_traits>

#include "moe_common.h"
#include "moe_fp8_codec.h"

namespace moe {

namespace {

constexpr int kRowThreads = 256;

__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
}

// Eight consecutive elements of a row, as fp32, for either storage type
// (bf16 bit patterns in uint16_t, or fp32); index i8 counts groups of eight.
__device__ __forceinline__ void load8(const uint16_t* p, size_t i8, float (&f)[8]) {
  unpack8(reinterpret_cast<const uint4*>(p)[i8], f);
}
__device__ __forceinline__ void load8(const float* p, size_t i8, float (&f)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[2 * i8];
  const float4 b = reinterpret_cast<const float4*>(p)[2 * i8 + 1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
// Streaming forms (load16_nt, store16_nt in moe_common.h) for rows touched
// exactly once per pass.  Measured on gfx950 at the 30B shape: streaming loads
// take the top-8 gather-reduce from 5.0 to 6.2 TB/s; the dispatch keeps plain
// stores (streaming ones measured slower there: 5.6 -> 5.2 TB/s, the next
// kernel reading the rows back).
__device__ __forceinline__ void load8_nt(const uint16_t* p, size_t i8, float (&f)[8]) {
  unpack8(load16_nt(reinterpret_cast<const uint4*>(p) + i8), f);
}
__device__ __forceinline__ void load8_nt(const float* p, size_t i8, float (&f)[8]) {
  const uint4 a = load16_nt(reinterpret_cast<const float4*>(p) + 2 * i8);
  const uint4 b = load16_nt(reinterpret_cast<const float4*>(p) + 2 * i8 + 1);
  f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y);
  f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
  f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y);
  f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
}
__device__ __forceinline__ void store8_nt(uint16_t* p, size_t i8, const float (&f)[8]) {
  store16_nt(reinterpret_cast<uint4*>(p) + i8, pack8(f));
}
__device__ __forceinline__ void store8_nt(float* p, size_t i8, const float (&f)[8]) {
  store16_nt(reinterpret_cast<float4*>(p) + 2 * i8,
             make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                        __float_as_uint(f[3])));
  store16_nt(reinterpret_cast<float4*>(p) + 2 * i8 + 1,
             make_uint4(__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]),
                        __float_as_uint(f[7])));
}
__device__ __forceinline__ void store8(uint16_t* p, size_t i8, const float (&f)[8]) {
  reinterpret_cast<uint4*>(p)[i8] = pack8(f);
}
__device__ __forceinline__ void store8(float* p, size_t i8, const float (&f)[8]) {
  reinterpret_cast<float4*>(p)[2 * i8] = make_float4(f[0], f[1], f[2], f[3]);
  reinterpret_cast<float4*>(p)[2 * i8 + 1] = make_float4(f[4], f[5], f[6], f[7]);
}

// IO: element type of the layer's inputs/outputs; ACT: of the permuted rows in
// scratch (uint16_t = bf16, or float).  A bf16 -> bf16 or fp32 -> fp32 move is
// a bitwise copy; fp32 -> bf16 rounds once (RNE).  With QM (FP8 forward modes,
// bf16 rows) the token's row is also quantised along D once and its codes
// written with every copy: codes [N, D], scale entries [D/128][N], as the
// standalone row quantiser writes them (a token's chunks sit on consecutive
// threads, so the groups are aligned lanes when D / 8 is a multiple of 16);
// with dst null only the codes are written.
template <typename IO, typename ACT, int QM>
__global__ void __launch_bounds__(kRowThreads) dispatch_kernel(
    const IO* __restrict__ rows, int T, int K, int D, const int32_t* __restrict__ pos,
    ACT* __restrict__ dst,
    uint8_t* __restrict__ qcodes, uint32_t* __restrict__ qsc, int N) {
  const int chunks = D / 8;
  const int tpr = chunks < kRowThreads ? chunks : kRowThreads;
  const int rpb = kRowThreads / tpr;
  const int t = blockIdx.x * rpb + threadIdx.x / tpr;
  const int c0 = threadIdx.x % tpr;
  if (t >= T || threadIdx.x >= rpb * tpr) return;
  const int32_t* prow = pos + size_t(t) * K;
  for (int c = c0; c < chunks; c += tpr) {
    const size_t src = (size_t(t) * D) / 8 + c;
    if constexpr (std::is_same<IO, uint16_t>::value && std::is_same<ACT, uint16_t>::value) {
      const uint4 v = reinterpret_cast<const uint4*>(rows)[src];
      if constexpr (QM != QM_NONE) {
        float f[8];
        unpack8(v, f);
        uint32_t entry;
        const uint2 codes = quantise8<QM>(f, threadIdx.x & 63, entry);
        for (int k = 0; k < K; ++k) {
          const int q = prow[k];
          if (q >= 0) {
            if (dst != nullptr) reinterpret_cast<uint4*>(dst)[(size_t(q) * D) / 8 + c] = v;
            *reinterpret_cast<uint2*>(qcodes + size_t(q) * D + 8 * c) = codes;
            if ((c & 15) == 0) qsc[size_t(c >> 4) * N + q] = entry;
          }
        }
      } else {
        for (int k = 0; k < K; ++k) {
          const int q = prow[k];
          if (q >= 0) reinterpret_cast<uint4*>(dst)[(size_t(q) * D) / 8 + c] = v;
        }
      }
    } else {
      float f[8];
      load8(rows, src, f);
      for (int k = 0; k < K; ++k) {
        const int q = prow[k];
        if (q >= 0) store8(dst, (size_t(q) * D) / 8 + c, f);
      }
    }
  }
}

// Gather-reduce of bf16 rows of more than 256 16-byte chunks (D = 4096 or
// 8192): a thread owns CPT chunks of the token's row, tpr = D / 8 / CPT apart,
// and per batch of KB pairs issues all CPT * KB loads before it adds any (same
// sums in the same order as gather_reduce_kernel; looping over the chunks
// instead measured 5% slower in the 235B-shaped combine).  The same form of
// the dispatch measured slower than its chunk loop, which it keeps.
template <typename OUT, bool WEIGHTED, int CPT, int KB>
__global__ void __launch_bounds__(kRowThreads) gather_reduce_wide_kernel(
    const uint16_t* __restrict__ rows, const int32_t* __restrict__ pos,
    const float* __restrict__ topk_w, int T, int K, int D, OUT* __restrict__ out) {
  const int tpr = D / 8 / CPT;
  const int rpb = kRowThreads / tpr;
  const int t = blockIdx.x * rpb + threadIdx.x / tpr;
  const int c0 = threadIdx.x % tpr;
  if (t >= T || threadIdx.x >= rpb * tpr) return;
  const int32_t* prow = pos + size_t(t) * K;
  const float* wrow = WEIGHTED ? topk_w + size_t(t) * K : nullptr;
  float acc[CPT][8];
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = 0.f;
  auto add = [&](float (&a)[8], bool live, float w, const uint4& raw) {
    float f[8];
    unpack8(raw, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float s = WEIGHTED ? __builtin_fmaf(w, f[i], a[i]) : a[i] + f[i];
      a[i] = live ? s : a[i];
    }
  };
  const int kfull = K - K % KB;
  for (int k0 = 0; k0 < kfull; k0 += KB) {
    int q[KB];
    float w[KB];
    uint4 v[KB][CPT];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      q[b] = prow[k0 + b];
      w[b] = WEIGHTED ? wrow[k0 + b] : 1.f;
    }
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      const uint4* r = reinterpret_cast<const uint4*>(rows) + (size_t(q[b] < 0 ? 0 : q[b]) * D) / 8 + c0;
#pragma unroll
      for (int j = 0; j < CPT; ++j) v[b][j] = load16_nt(r + j * tpr);
    }
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int j = 0; j < CPT; ++j) add(acc[j], q[b] >= 0, w[b], v[b][j]);
  }
  for (int k = kfull; k < K; ++k) {
    const int qk = prow[k];
    const uint4* r = reinterpret_cast<const uint4*>(rows) + (size_t(qk < 0 ? 0 : qk) * D) / 8 + c0;
#pragma unroll
    for (int j = 0; j < CPT; ++j) add(acc[j], qk >= 0, WEIGHTED ? wrow[k] : 1.f, load16_nt(r + j * tpr));
  }
#pragma unroll
  for (int j = 0; j < CPT; ++j) store8_nt(out, (size_t(t) * D) / 8 + c0 + j * tpr, acc[j]);
}

// Dispatch of bf16 rows of 64 * CPL chunks (D = 512 * CPL): one token per
// block; each wave holds the whole row in registers (its re-reads of the row
// come from the cache) and writes whole destination rows, copies k = wave,
// wave + 4, ..., so each copy is written contiguously by one wave (235B
// shape: 227 -> 218 us against every thread writing its chunk of every copy;
// the 30B shape is unchanged).  Used when every wave has a copy (K >= 4): with
// one pair per token three waves of four would idle.
// With QM (FP8 forward modes) every wave also quantises the row along D (a
// 128-column group is 16 consecutive lanes' chunks) and writes the codes and
// scale entries of its copies, as dispatch_kernel does; with dst null it
// writes only those.
template <int CPL, int QM>
__global__ void __launch_bounds__(kRowThreads) dispatch_rows_kernel(
    const uint16_t* __restrict__ rows, int T, int K, int D, const int32_t* __restrict__ pos,
    uint16_t* __restrict__ dst,
    uint8_t* __restrict__ qcodes, uint32_t* __restrict__ qsc, int N) {
  constexpr int WAVES = kRowThreads / 64;
  const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (t >= T) return;
  const int32_t* prow = pos + size_t(t) * K;
  const uint4* src = reinterpret_cast<const uint4*>(rows) + (size_t(t) * D) / 8 + lane;
  uint4 v[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) v[j] = src[64 * j];
  uint2 codes[QM != QM_NONE ? CPL : 1];
  uint32_t entry[QM != QM_NONE ? CPL : 1];
  if constexpr (QM != QM_NONE) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      float f[8];
      unpack8(v[j], f);
      codes[j] = quantise8<QM>(f, lane, entry[j]);
    }
  }
  for (int k = wave; k < K; k += WAVES) {
    const int q = prow[k];
    if (q < 0) continue;
    if (QM == QM_NONE || dst != nullptr) {  // FP8 modes may keep only the codes
      uint4* d = reinterpret_cast<uint4*>(dst) + (size_t(q) * D) / 8 + lane;
#pragma unroll
      for (int j = 0; j < CPL; ++j) d[64 * j] = v[j];
    }
    if constexpr (QM != QM_NONE) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        *reinterpret_cast<uint2*>(qcodes + size_t(q) * D + 8 * c) = codes[j];
        if ((c & 15) == 0) qsc[size_t(c >> 4) * N + q] = entry[j];
      }
    }
  }
}

// Per-token gather-reduce over the K pair rows: combine (WEIGHTED: y_t =
// sum_k w_tk * O[pos]) and the un-permute of dx (plain sum), fp32, k ascending.
// Pairs are taken KB at a time with no branch between the loads, so each
// thread keeps KB 16-byte loads in flight: a pair with no row (pos < 0) loads
// row 0 and its sum is dropped by a select (the accumulator is left exactly as
// it was).  The last K % KB pairs go one at a time.
template <typename ACT, typename OUT, bool WEIGHTED, int KB>
__global__ void __launch_bounds__(kRowThreads) gather_reduce_kernel(
    const ACT* __restrict__ rows, const int32_t* __restrict__ pos,
    const float* __restrict__ topk_w, int T, int K, int D, OUT* __restrict__ out) {
  const int chunks = D / 8;
  const int tpr = chunks < kRowThreads ? chunks : kRowThreads;
  const int rpb = kRowThreads / tpr;
  const int t = blockIdx.x * rpb + threadIdx.x / tpr;
  const int c0 = threadIdx.x % tpr;
  if (t >= T || threadIdx.x >= rpb * tpr) return;
  const int32_t* prow = pos + size_t(t) * K;
  const float* wrow = WEIGHTED ? topk_w + size_t(t) * K : nullptr;
  const int kfull = K - K % KB;
  for (int c = c0; c < chunks; c += tpr) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto add = [&](bool live, float w, const float (&f)[8]) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float s = WEIGHTED ? __builtin_fmaf(w, f[i], acc[i]) : acc[i] + f[i];
        acc[i] = live ? s : acc[i];
      }
    };
    for (int k0 = 0; k0 < kfull; k0 += KB) {
      int q[KB];
      float w[KB], f[KB][8];
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        q[j] = prow[k0 + j];
        w[j] = WEIGHTED ? wrow[k0 + j] : 1.f;
      }
#pragma unroll
      for (int j = 0; j < KB; ++j) load8_nt(rows, (size_t(q[j] < 0 ? 0 : q[j]) * D) / 8 + c, f[j]);
#pragma unroll
      for (int j = 0; j < KB; ++j) add(q[j] >= 0, w[j], f[j]);
    }
    for (int k = kfull; k < K; ++k) {
      const int q = prow[k];
      float f[8];
      load8_nt(rows, (size_t(q < 0 ? 0 : q) * D) / 8 + c, f);
      add(q >= 0, WEIGHTED ? wrow[k] : 1.f, f);
    }
    store8_nt(out, (size_t(t) * D) / 8 + c, acc);
  }
}

// Combine-backward: for each routed pair p of token t (row q = pos[p]),
//   dYw_perm[q] = w_p * dy_t          (fp32 product, stored as ACT)
//   dtopk_w[p]  = <dy_t, O[q]>         (fp32, the routing-weight gradient)
// WPT wavefronts own one token, each a contiguous quarter, half or all of the
// row (64 * CPL chunks of 16 bytes: CPL per lane); their dy slices stay in
// registers while the K expert-output rows are streamed and dotted against
// them.  With WPT > 1 the waves' partial dot products meet in LDS and are
// added in wave order (fixed, so the result is the same on every run); rows of
// 512 or 1024 chunks (D = 4096 or 8192) take two or four waves, which halves
// or quarters each wave's registers and puts more rows in flight.
// QM (FP8 backward modes, bf16 rows): the kernel also writes the e4m3 row
// quantisation of each dYw row along D (the W2 dgrad's A operand), from the
// same bf16-rounded values it stores: QM_BLOCK, an fp32 scale per 128 columns
// (a group is 16 consecutive lanes' chunks); QM_MX, an e8m0 scale per 32 (4
// lanes).  Codes are [N, D] bytes, scale entries [D/128][N], as the standalone
// row quantiser writes them.  With dst null the bf16 rows are not stored (the
// FP8 backward's token quantiser gathers w * dy itself; in MXFP8 it also writes
// the row codes, and this kernel computes only dtopk_w).  D / 8 must be a multiple of 16 so a group never
// straddles active and idle lanes.
constexpr int kSplitMaxK = 64;  // K up to this many slots may split a row over waves

template <typename IO, typename ACT, int CPL, int QM, int WPT>
__global__ void __launch_bounds__(kRowThreads) dispatch_dy_kernel(
    const IO* __restrict__ dy, int T, int K, int D, const int32_t* __restrict__ pos,
    const float* __restrict__ topk_w, const ACT* __restrict__ O, ACT* __restrict__ dst,
    float* __restrict__ dprob, uint8_t* __restrict__ qcodes, uint32_t* __restrict__ qsc, int N) {
  constexpr int WAVES = kRowThreads / 64;
  __shared__ float sdot[WPT > 1 ? WAVES : 1][WPT > 1 ? kSplitMaxK : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * (WAVES / WPT) + wave / WPT;
  const int c0 = (wave % WPT) * 64 * CPL + lane;  // this lane's first chunk of the row
  const bool live = t < T;
  if (WPT == 1 && !live) return;
  const int chunks = D / 8;
  if (live) {
    float v[CPL][8];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = c0 + 64 * j;
      if (c < chunks) load8(dy, (size_t(t) * D) / 8 + c, v[j]);
    }
    for (int k = 0; k < K; ++k) {
      const int p = t * K + k;
      const int q = pos[p];
      if (q < 0) {
        if (lane == 0) {
          if constexpr (WPT > 1) sdot[wave][k] = 0.f;
          else dprob[p] = 0.f;
        }
        continue;
      }
      const float w = topk_w[p];
      float dot = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = c0 + 64 * j;
        float sc[8];
        if (c < chunks) {
          float o[8];
          load8_nt(O, (size_t(q) * D) / 8 + c, o);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            dot = __builtin_fmaf(v[j][i], o[i], dot);
            sc[i] = w * v[j][i];
          }
          if (dst != nullptr) store8(dst, (size_t(q) * D) / 8 + c, sc);
        }
        if constexpr (QM != QM_NONE) {
          // quantise the stored (bf16-rounded) values; idle lanes join the reductions with 0
#pragma unroll
          for (int i = 0; i < 8; ++i) sc[i] = c < chunks ? float((__bf16)sc[i]) : 0.f;
          uint32_t entry;
          const uint2 codes = quantise8<QM>(sc, lane, entry);
          if (c < chunks) {
            *reinterpret_cast<uint2*>(qcodes + size_t(q) * D + 8 * c) = codes;
            if ((lane & 15) == 0) qsc[size_t(c >> 4) * N + q] = entry;
          }
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
      if (lane == 0) {
        if constexpr (WPT > 1) sdot[wave][k] = dot;
        else dprob[p] = dot;
      }
    }
  }
  if constexpr (WPT > 1) {
    __syncthreads();
    if (live && wave % WPT == 0) {
      for (int k = lane; k < K; k += 64) {
        float sum = sdot[wave][k];
#pragma unroll
        for (int i = 1; i < WPT; ++i) sum += sdot[wave + i][k];
        dprob[size_t(t) * K + k] = sum;
      }
    }
  }
}

__global__ void convert_bf16_kernel(const float* __restrict__ in, uint16_t* __restrict__ out,
                                    size_t n8) {
  for (size_t i = blockIdx.x * size_t(blockDim.x) + threadIdx.x; i < n8;
       i += size_t(gridDim.x) * blockDim.x) {
    const float4 a = reinterpret_cast<const float4*>(in)[2 * i];
    const float4 b = reinterpret_cast<const float4*>(in)[2 * i + 1];
    const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    reinterpret_cast<uint4*>(out)[i] = pack8(f);
  }
}

inline int row_blocks(const moe_desc& d) {
  const int chunks = d.D / 8;
  const int tpr = chunks < kRowThreads ? chunks : kRowThreads;
  const int rpb = kRowThreads / tpr;
  return (d.T + rpb - 1) / rpb;
}

// Pairs per batch for a top-K: at most 8, and no more than K.
// Chunks per thread of the wide gather-reduce for bf16 rows of D elements: 2 or
// 4 when D is 4096 or 8192, else 0 (the one-chunk-at-a-time kernel).
inline int wide_cpt(int D) { return D == 4096 ? 2 : D == 8192 ? 4 : 0; }

template <typename ACT, typename OUT, bool WEIGHTED>
static void launch_gather_reduce(const moe_desc& d, const ACT* rows, const int32_t* pos,
                                 const float* topk_w, OUT* out, hipStream_t s) {
  if constexpr (std::is_same<ACT, uint16_t>::value) {
    const int cpt = wide_cpt(d.D);
    if (cpt != 0 && d.K >= 8) {  // one token per block: tpr = 256
      if (cpt == 2)
        gather_reduce_wide_kernel<OUT, WEIGHTED, 2, 8><<<d.T, kRowThreads, 0, s>>>(rows, pos, topk_w, d.T, d.K, d.D, out);
      else
        gather_reduce_wide_kernel<OUT, WEIGHTED, 4, 8><<<d.T, kRowThreads, 0, s>>>(rows, pos, topk_w, d.T, d.K, d.D, out);
      return;
    }
  }
#define MOE_GR(KB) gather_reduce_kernel<ACT, OUT, WEIGHTED, KB><<<row_blocks(d), kRowThreads, 0, s>>>(rows, pos, topk_w, d.T, d.K, d.D, out)
  if (d.K >= 8) MOE_GR(8);
  else if (d.K >= 4) MOE_GR(4);
  else if (d.K >= 2) MOE_GR(2);
  else MOE_GR(1);
#undef MOE_GR
}

}  // namespace

// Element types of a mode: I/O fp32 in the fp32-storage modes, intermediates
// fp32 only in MOE_FP32.
template <class F>
static int with_types(const moe_desc& d, bool io_f32, F f) {
  if (d.mode == MOE_FP32) return f(float{}, float{});
  if (io_f32) return f(float{}, uint16_t{});
  return f(uint16_t{}, uint16_t{});
}

int launch_dispatch(const moe_desc& d, const Layout& L, const void* rows, bool in_f32,
                    char* scratch, size_t dst_off, hipStream_t s, int qmode, uint8_t* qcodes,
                    uint32_t* qsc, bool store_rows, const char* name) {
  if (!store_rows && qmode == 0) return MOE_EINVAL;
  const auto* pos = reinterpret_cast<const int32_t*>(scratch + L.pos);
  prof_begin(name, s);
  const int rc = with_types(d, in_f32, [&](auto io, auto act) {
    using IO = decltype(io);
    using ACT = decltype(act);
    const IO* src = static_cast<const IO*>(rows);
    ACT* dst = store_rows ? reinterpret_cast<ACT*>(scratch + dst_off) : nullptr;
    const int N = d.T * d.K;
    if constexpr (std::is_same<IO, uint16_t>::value && std::is_same<ACT, uint16_t>::value) {
      if (qmode != 0 && d.D == 2048 && d.K >= kRowThreads / 64) {  // FP8 forward, 30B shape
        if (qmode == 1)
          dispatch_rows_kernel<4, QM_MX><<<d.T, kRowThreads, 0, s>>>(src, d.T, d.K, d.D, pos, dst, qcodes, qsc, N);
        else
          dispatch_rows_kernel<4, QM_BLOCK><<<d.T, kRowThreads, 0, s>>>(src, d.T, d.K, d.D, pos, dst, qcodes, qsc, N);
        return 0;
      }
      if (qmode == 1) {
        dispatch_kernel<IO, ACT, QM_MX><<<row_blocks(d), kRowThreads, 0, s>>>(
            src, d.T, d.K, d.D, pos, dst, qcodes, qsc, N);
        return 0;
      }
      if (qmode == 2) {
        dispatch_kernel<IO, ACT, QM_BLOCK><<<row_blocks(d), kRowThreads, 0, s>>>(
            src, d.T, d.K, d.D, pos, dst, qcodes, qsc, N);
        return 0;
      }
    }
    if (qmode != 0) return int(MOE_EUNSUPPORTED);
    if constexpr (std::is_same<IO, uint16_t>::value && std::is_same<ACT, uint16_t>::value) {
      if ((d.D == 2048 || d.D == 4096) && d.K >= kRowThreads / 64) {
        if (d.D == 2048)
          dispatch_rows_kernel<4, QM_NONE><<<d.T, kRowThreads, 0, s>>>(src, d.T, d.K, d.D, pos, dst, nullptr, nullptr, N);
        else
          dispatch_rows_kernel<8, QM_NONE><<<d.T, kRowThreads, 0, s>>>(src, d.T, d.K, d.D, pos, dst, nullptr, nullptr, N);
        return 0;
      }
    }
    dispatch_kernel<IO, ACT, QM_NONE><<<row_blocks(d), kRowThreads, 0, s>>>(
        src, d.T, d.K, d.D, pos, dst, nullptr, nullptr, N);
    return 0;
  });
  prof_end(s);
  if (rc) return rc;
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int launch_combine(const moe_desc& d, const Layout& L, const float* topk_w, void* y,
                   bool out_f32, const char* scratch, hipStream_t s, bool weighted) {
  const auto* pos = reinterpret_cast<const int32_t*>(scratch + L.pos);
  prof_begin("combine", s);
  with_types(d, out_f32, [&](auto io, auto act) {
    using IO = decltype(io);
    using ACT = decltype(act);
    if (weighted)
      launch_gather_reduce<ACT, IO, true>(d, reinterpret_cast<const ACT*>(scratch + L.o), pos,
                                          topk_w, static_cast<IO*>(y), s);
    else
      launch_gather_reduce<ACT, IO, false>(d, reinterpret_cast<const ACT*>(scratch + L.o), pos,
                                           nullptr, static_cast<IO*>(y), s);
    return 0;
  });
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int launch_unpermute(const moe_desc& d, const Layout& L, void* dx, bool out_f32,
                     const char* scratch, hipStream_t s) {
  const auto* pos = reinterpret_cast<const int32_t*>(scratch + L.pos);
  prof_begin("unpermute", s);
  with_types(d, out_f32, [&](auto io, auto act) {
    using IO = decltype(io);
    using ACT = decltype(act);
    launch_gather_reduce<ACT, IO, false>(d, reinterpret_cast<const ACT*>(scratch + L.dxperm),
                                         pos, nullptr, static_cast<IO*>(dx), s);
    return 0;
  });
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// dtopk_w[src[q]] = sum over j of part[q * J + j], j ascending, for every
// permuted row q (thread q: a wave reads 64 consecutive rows of partials), and
// dtopk_w[p] = 0 for the pairs without a row (thread p).
__global__ void __launch_bounds__(256) dprob_reduce_kernel(const int32_t* __restrict__ pos,
                                                           const int32_t* __restrict__ src,
                                                           const int32_t* __restrict__ nrows,
                                                           const float* __restrict__ part, int J,
                                                           float* __restrict__ dtopk_w, int N) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  if (i < *nrows) {  // J is even (F % 128 == 0): the row's pairs of partials, loads first
    const float2* r = reinterpret_cast<const float2*>(part + size_t(i) * J);
    float s = 0.f;
#pragma unroll 6
    for (int j = 0; j < J / 2; ++j) {
      const float2 v = r[j];
      s += v.x;
      s += v.y;
    }
    dtopk_w[src[i]] = s;
  }
  if (pos[i] < 0) dtopk_w[i] = 0.f;
}

int launch_dprob_reduce(const moe_desc& d, const Layout& L, float* dtopk_w, const char* scratch,
                        hipStream_t s) {
  const int N = d.T * d.K;
  if (N == 0) return MOE_OK;
  prof_begin("dprob_reduce", s);
  dprob_reduce_kernel<<<unsigned((N + 255) / 256), 256, 0, s>>>(
      reinterpret_cast<const int32_t*>(scratch + L.pos),
      reinterpret_cast<const int32_t*>(scratch + L.src),
      reinterpret_cast<const int32_t*>(scratch + L.offsets) + d.E,
      reinterpret_cast<const float*>(scratch + L.dpart), dprob_parts(d), dtopk_w, N);
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

template <typename IO, typename ACT, int QM>
static int dispatch_dy_cpl(const moe_desc& d, const IO* dy, const int32_t* pos,
                           const float* topk_w, const ACT* o, ACT* dst, float* dprob,
                           uint8_t* qcodes, uint32_t* qsc, hipStream_t s) {
  const int cpl = (d.D / 8 + 63) / 64;  // 16-byte chunks per lane with one wave per token
  const int waves = kRowThreads / 64;
  auto blocks = [&](int wpt) { return unsigned((d.T + waves / wpt - 1) / (waves / wpt)); };
#define MOE_DY(C, W) dispatch_dy_kernel<IO, ACT, C, QM, W><<<blocks(W), kRowThreads, 0, s>>>(dy, d.T, d.K, d.D, pos, topk_w, o, dst, dprob, qcodes, qsc, d.T * d.K)
  if (cpl <= 1) MOE_DY(1, 1);
  else if (cpl <= 2) MOE_DY(2, 1);
  else if (cpl <= 4) MOE_DY(4, 1);
  else if (cpl <= 8) { if (d.K <= kSplitMaxK) MOE_DY(4, 2); else MOE_DY(8, 1); }
  else if (cpl <= 16) { if (d.K <= kSplitMaxK) MOE_DY(4, 4); else MOE_DY(16, 1); }
  else return MOE_EUNSUPPORTED;
#undef MOE_DY
  return MOE_OK;
}

int launch_dispatch_dy(const moe_desc& d, const Layout& L, const void* dy, bool in_f32,
                       const float* topk_w, float* dtopk_w, char* scratch, hipStream_t s,
                       int qmode, uint8_t* qcodes, uint32_t* qsc, bool store_rows) {
  const auto* pos = reinterpret_cast<const int32_t*>(scratch + L.pos);
  prof_begin("dispatch_dy", s);
  const int rc = with_types(d, in_f32, [&](auto io, auto act) {
    using IO = decltype(io);
    using ACT = decltype(act);
    const IO* src = static_cast<const IO*>(dy);
    const ACT* o = reinterpret_cast<const ACT*>(scratch + L.o);
    ACT* dst = store_rows ? reinterpret_cast<ACT*>(scratch + L.dyperm) : nullptr;
    if constexpr (std::is_same<ACT, uint16_t>::value) {
      if (qmode == 1)
        return dispatch_dy_cpl<IO, ACT, QM_MX>(d, src, pos, topk_w, o, dst, dtopk_w, qcodes, qsc, s);
      if (qmode == 2)
        return dispatch_dy_cpl<IO, ACT, QM_BLOCK>(d, src, pos, topk_w, o, dst, dtopk_w, qcodes, qsc, s);
    }
    if (qmode != 0) return int(MOE_EUNSUPPORTED);
    return dispatch_dy_cpl<IO, ACT, QM_NONE>(d, src, pos, topk_w, o, dst, dtopk_w, nullptr, nullptr, s);
  });
  prof_end(s);
  if (rc) return rc;
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

__global__ void zero16_kernel(uint4* __restrict__ out, size_t n16) {
  for (size_t i = blockIdx.x * size_t(blockDim.x) + threadIdx.x; i < n16;
       i += size_t(gridDim.x) * blockDim.x)
    out[i] = make_uint4(0, 0, 0, 0);
}

int launch_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes % 16 != 0) return MOE_EINVAL;
  const size_t n16 = bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) return MOE_OK;
  prof_begin("zero", s);
  zero16_kernel<<<unsigned(blocks), 256, 0, s>>>(static_cast<uint4*>(p), n16);
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int launch_convert_bf16(const float* in, uint16_t* out, size_t n, hipStream_t s) {
  const size_t n8 = n / 8;
  size_t blocks = (n8 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) return MOE_OK;
  prof_begin("convert_bf16", s);
  convert_bf16_kernel<<<unsigned(blocks), 256, 0, s>>>(in, out, n8);
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
