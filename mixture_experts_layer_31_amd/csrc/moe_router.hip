// Top-k router ahead of the layer: softmax over a token's E expert logits, the
// K most probable experts, their probabilities renormalised to sum to 1; and
// its backward from the routing-weight gradient to the logits.
//
// The pages' layer takes a top-8-of-128 routing decision as its input (Prime
// Mega MoE news item, "TL;DR" and "Why is MoE training communication-bound?":
// each token goes to a small subset of experts).  This file computes that
// decision from the logits and returns the gradient the layer's dtopk_w
// induces on them.
//
// One wave64 per token, logits held in registers (E/64 per lane, E <= 512):
//   * Selection is exact and needs no softmax: exp is increasing, so the K
//     largest probabilities are the K largest logits.  Each logit's bits are
//     mapped to an unsigned key of the same order (sign set -> all bits
//     flipped, else the sign bit set).  A 32-step radix select finds the K-th
//     largest key tau bit by bit, counting keys >= a candidate with one ballot
//     and popcount per register (scalar work, no lane-to-lane data movement).
//     The selection is every key > tau plus the lowest-index keys == tau (rank
//     among equals from mbcnt over the ballot, index order = register order,
//     then lane order).  The K winners are compacted into LDS in index order;
//     each of lanes 0..K-1 takes one and counts the winners ahead of it (larger
//     key, or equal key and lower index) to find its output slot, so the slots
//     come out in descending order, ties to the lower index.
//   * Weights: renormalising the top-K softmax probabilities cancels the full
//     softmax denominator, so w_k = exp(z_k - z_max) / sum_k' exp(z_k' - z_max)
//     over the selected logits only.  Every lane sums the K exponentials in the
//     same (index) order, so all lanes hold the same total.
//   * Backward: through the renormalisation and the softmax the gradient
//     collapses to dz_j = w_j (dw_j - sum_k w_k dw_k) for a selected expert j
//     and 0 for the others (the softmax's own correction term is
//     sum_j p_j dp_j = 0 here); the sum and the K (id, value) pairs are read
//     with readlane in slot order, and each lane writes its E/64 entries.
#include <type_traits>

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kRouterThreads = 256;  // four tokens per workgroup

// Float bits -> unsigned key with the same order (for non-NaN values).
__device__ __forceinline__ uint32_t order_key(float z) {
  const uint32_t u = __float_as_uint(z);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Set bits of a wave mask below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
}

template <int VPL>
__global__ void __launch_bounds__(kRouterThreads) router_fwd_kernel(
    const float* __restrict__ logits, int T, int E, int K, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
  __shared__ uint32_t s_key[kRouterThreads / 64][64];
  __shared__ int32_t s_idx[kRouterThreads / 64][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * (kRouterThreads / 64) + wv;
  if (t >= T) return;  // whole wave
  const float* row = logits + size_t(t) * E;
  // padding (index >= E) gets key 0: it can tie only with a real key of 0 and
  // then loses on index, and K <= E real keys always exist
  uint32_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int j = lane + 64 * i;
    key[i] = j < E ? order_key(row[j]) : 0u;
  }
  // tau = the largest value with #{keys >= tau} >= K, i.e. the K-th largest key
  uint32_t tau = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = tau | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) cnt += __popcll(__ballot(key[i] >= cand));
    if (cnt >= K) tau = cand;
  }
  int ngt = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) ngt += __popcll(__ballot(key[i] > tau));
  const int need = K - ngt;  // >= 1 keys equal to tau, lowest indices first
  int eq_before = 0, sel_before = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const uint64_t eq = __ballot(key[i] == tau);
    const bool sel = key[i] > tau || (key[i] == tau && eq_before + lanes_below(eq) < need);
    const uint64_t sm = __ballot(sel);
    if (sel) {
      const int p = sel_before + lanes_below(sm);
      s_key[wv][p] = key[i];
      s_idx[wv][p] = lane + 64 * i;
    }
    eq_before += __popcll(eq);
    sel_before += __popcll(sm);
  }
  // the compaction above is this wave's own LDS traffic: order it before the reads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < K) {
    const uint32_t mk = s_key[wv][lane];
    const int mj = s_idx[wv][lane];
    uint32_t kmax = 0;
    int slot = 0;
    for (int q = 0; q < K; ++q) {
      const uint32_t kq = s_key[wv][q];
      kmax = kq > kmax ? kq : kmax;
      slot += (kq > mk || (kq == mk && s_idx[wv][q] < mj)) ? 1 : 0;
    }
    const float zmax = order_value(kmax);
    float sum = 0.f;
    for (int q = 0; q < K; ++q) sum += expf(order_value(s_key[wv][q]) - zmax);
    topk_idx[size_t(t) * K + slot] = mj;
    topk_w[size_t(t) * K + slot] = expf(order_value(mk) - zmax) / sum;
  }
}

template <int VPL>
__global__ void __launch_bounds__(kRouterThreads) router_bwd_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
    const float* __restrict__ dtopk_w, int T, int E, int K, float* __restrict__ dlogits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kRouterThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave
  int j = -1;
  float w = 0.f, dw = 0.f;
  if (lane < K) {
    j = topk_idx[size_t(t) * K + lane];
    w = topk_w[size_t(t) * K + lane];
    dw = dtopk_w[size_t(t) * K + lane];
  }
  const float wdw = w * dw;
  float c = 0.f;
  for (int k = 0; k < K; ++k) c += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wdw), k));
  const float g = w * (dw - c);
  float val[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) val[i] = 0.f;
  for (int k = 0; k < K; ++k) {
    const int jk = __builtin_amdgcn_readlane(j, k);
    const float gk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), k));
    if (jk >= 0 && jk < E && (jk & 63) == lane) {
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (i == (jk >> 6)) val[i] += gk;
    }
  }
  float* out = dlogits + size_t(t) * E;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int jj = lane + 64 * i;
    if (jj < E) out[jj] = val[i];
  }
}

template <class F>
int with_vpl(int E, F&& f) {
  if (E <= 64) return f(std::integral_constant<int, 1>{});
  if (E <= 128) return f(std::integral_constant<int, 2>{});
  if (E <= 256) return f(std::integral_constant<int, 4>{});
  return f(std::integral_constant<int, 8>{});
}

}  // namespace

int launch_router_fwd(int T, int E, int K, const float* logits, int32_t* topk_idx, float* topk_w,
                      hipStream_t s) {
  const unsigned grid = unsigned((T + kRouterThreads / 64 - 1) / (kRouterThreads / 64));
  return with_vpl(E, [&](auto v) {
    prof_begin("router_fwd", s);
    router_fwd_kernel<decltype(v)::value><<<grid, kRouterThreads, 0, s>>>(logits, T, E, K, topk_idx,
                                                                           topk_w);
    prof_end(s);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
  });
}

int launch_router_bwd(int T, int E, int K, const int32_t* topk_idx, const float* topk_w,
                      const float* dtopk_w, float* dlogits, hipStream_t s) {
  const unsigned grid = unsigned((T + kRouterThreads / 64 - 1) / (kRouterThreads / 64));
  return with_vpl(E, [&](auto v) {
    prof_begin("router_bwd", s);
    router_bwd_kernel<decltype(v)::value><<<grid, kRouterThreads, 0, s>>>(topk_idx, topk_w, dtopk_w,
                                                                           T, E, K, dlogits);
    prof_end(s);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
  });
}

}  // namespace moe
