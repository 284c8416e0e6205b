// HBM-bound row movers of the MoE layer: dispatch, combine, un-permute.
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
#include "moe_common.h"

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

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const uint32_t a = __builtin_bit_cast(uint16_t, (__bf16)lo);
  const uint32_t b = __builtin_bit_cast(uint16_t, (__bf16)hi);
  return a | (b << 16);
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
}

template <bool IN_F32>
__global__ void __launch_bounds__(kRowThreads) dispatch_kernel(
    const void* __restrict__ rows, int T, int K, int D, const int32_t* __restrict__ pos,
    const float* __restrict__ topk_w, float* __restrict__ wperm, uint16_t* __restrict__ dst) {
  const int chunks = D / 8;
  const int tpr = chunks < kRowThreads ? chunks : kRowThreads;
  const int rpb = kRowThreads / tpr;
  const int t = blockIdx.x * rpb + threadIdx.x / tpr;
  const int c0 = threadIdx.x % tpr;
  if (t >= T || threadIdx.x >= rpb * tpr) return;
  const int32_t* prow = pos + size_t(t) * K;
  for (int c = c0; c < chunks; c += tpr) {
    uint4 v;
    if constexpr (IN_F32) {
      const float4* src = reinterpret_cast<const float4*>(rows) + (size_t(t) * D + c * 8) / 4;
      const float4 a = src[0], b = src[1];
      const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      v = pack8(f);
    } else {
      v = reinterpret_cast<const uint4*>(rows)[(size_t(t) * D) / 8 + c];
    }
    for (int k = 0; k < K; ++k) {
      const int q = prow[k];
      if (q >= 0) reinterpret_cast<uint4*>(dst)[(size_t(q) * D) / 8 + c] = v;
    }
  }
  if (wperm != nullptr) {
    for (int k = c0; k < K; k += tpr) {
      const int q = prow[k];
      if (q >= 0) wperm[q] = topk_w[size_t(t) * K + k];
    }
  }
}

template <bool OUT_F32, bool WEIGHTED>
__global__ void __launch_bounds__(kRowThreads) gather_reduce_kernel(
    const uint16_t* __restrict__ rows, const int32_t* __restrict__ pos,
    const float* __restrict__ topk_w, int T, int K, int D, void* __restrict__ out) {
  const int chunks = D / 8;
  const int tpr = chunks < kRowThreads ? chunks : kRowThreads;
  const int rpb = kRowThreads / tpr;
  const int t = blockIdx.x * rpb + threadIdx.x / tpr;
  const int c0 = threadIdx.x % tpr;
  if (t >= T || threadIdx.x >= rpb * tpr) return;
  const int32_t* prow = pos + size_t(t) * K;
  for (int c = c0; c < chunks; c += tpr) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; ++k) {
      const int q = prow[k];
      if (q < 0) continue;
      float f[8];
      unpack8(reinterpret_cast<const uint4*>(rows)[(size_t(q) * D) / 8 + c], f);
      if constexpr (WEIGHTED) {
        const float w = topk_w[size_t(t) * K + k];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(w, f[i], acc[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += f[i];
      }
    }
    if constexpr (OUT_F32) {
      float4* o = reinterpret_cast<float4*>(out) + (size_t(t) * D + c * 8) / 4;
      o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
      reinterpret_cast<uint4*>(out)[(size_t(t) * D) / 8 + c] = pack8(acc);
    }
  }
}

// dtopk_w[p] = sum of the per-tile partial <dy, o> sums of pair p, in tile order.
__global__ void dprob_reduce_kernel(const int32_t* __restrict__ pos,
                                    const float* __restrict__ part, int nparts, int stride,
                                    int N, float* __restrict__ dprob) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= N) return;
  const int q = pos[p];
  float s = 0.f;
  if (q >= 0) {
    const float* r = part + size_t(q) * stride;
    for (int j = 0; j < nparts; ++j) s += r[j];
  }
  dprob[p] = s;
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

}  // namespace

int launch_dispatch(const moe_desc& d, const Layout& L, const void* rows, bool in_f32,
                    const float* topk_w, char* scratch, size_t dst_off, hipStream_t s) {
  const auto* pos = reinterpret_cast<const int32_t*>(scratch + L.pos);
  auto* wperm = topk_w ? reinterpret_cast<float*>(scratch + L.wperm) : nullptr;
  auto* dst = reinterpret_cast<uint16_t*>(scratch + dst_off);
  prof_begin("dispatch", s);
  if (in_f32)
    dispatch_kernel<true><<<row_blocks(d), kRowThreads, 0, s>>>(rows, d.T, d.K, d.D, pos,
                                                                  topk_w, wperm, dst);
  else
    dispatch_kernel<false><<<row_blocks(d), kRowThreads, 0, s>>>(rows, d.T, d.K, d.D, pos,
                                                                   topk_w, wperm, dst);
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int launch_combine(const moe_desc& d, const Layout& L, const float* topk_w, void* y,
                   bool out_f32, const char* scratch, hipStream_t s) {
  const auto* pos = reinterpret_cast<const int32_t*>(scratch + L.pos);
  const auto* o = reinterpret_cast<const uint16_t*>(scratch + L.o);
  prof_begin("combine", s);
  if (out_f32)
    gather_reduce_kernel<true, true><<<row_blocks(d), kRowThreads, 0, s>>>(o, pos, topk_w, d.T,
                                                                            d.K, d.D, y);
  else
    gather_reduce_kernel<false, true><<<row_blocks(d), kRowThreads, 0, s>>>(o, pos, topk_w, d.T,
                                                                             d.K, d.D, y);
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int launch_unpermute(const moe_desc& d, const Layout& L, void* dx, bool out_f32, float* dtopk_w,
                     int nparts, const char* scratch, hipStream_t s) {
  const auto* pos = reinterpret_cast<const int32_t*>(scratch + L.pos);
  const auto* rows = reinterpret_cast<const uint16_t*>(scratch + L.dxperm);
  prof_begin("unpermute", s);
  if (out_f32)
    gather_reduce_kernel<true, false><<<row_blocks(d), kRowThreads, 0, s>>>(rows, pos, nullptr,
                                                                             d.T, d.K, d.D, dx);
  else
    gather_reduce_kernel<false, false><<<row_blocks(d), kRowThreads, 0, s>>>(rows, pos, nullptr,
                                                                              d.T, d.K, d.D, dx);
  prof_end(s);
  const int N = d.T * d.K;
  prof_begin("dprob_reduce", s);
  dprob_reduce_kernel<<<(N + 255) / 256, 256, 0, s>>>(
      pos, reinterpret_cast<const float*>(scratch + L.dprob_part), nparts, L.nparts_max, N,
      dtopk_w);
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
