// OCP e4m3 encodings shared by the FP8 quantisers (moe_fp8.hip) and the row
// movers that quantise while they copy (moe_rows.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Smallest X in [-127, 127] with amax <= 448 * 2^X (0 for amax == 0).
__device__ __forceinline__ int e8m0_exponent(float amax) {
  if (amax == 0.f) return 0;
  int e;
  const float m = frexpf(amax, &e);  // amax = m * 2^e, m in [0.5, 1); 448 = 0.875 * 2^9
  int X = (m <= 0.875f) ? e - 9 : e - 8;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

// Four OCP e4m3 codes (byte k = code of value k) by the hardware conversion:
// nearest value, ties to even mantissa, magnitudes >= 448 saturate to 448
// (checked against a software encoder of that rule with an in-bounds probe
// over every code, every rounding midpoint and its neighbours, and 4e5 random
// values).
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return uint32_t(w);
}

// The quotients x[i] / sc rounded to fp32 (IEEE division): the values whose
// e4m3 codes a blockwise tile stores.  The product x * rc (rc = 1/sc) lies
// within about 1.5 fp32 ulps of the quotient, so both have the same e4m3 code
// unless an e4m3 rounding midpoint lies within a few ulps of the product (its
// low 20 mantissa bits near 0x80000 in the normal e4m3 range) or the product
// is in the subnormal e4m3 range (below 2^-6).  Only then is the division
// done, behind a wave-uniform branch that is skipped unless some lane needs
// it (a per-element select would make every element pay for the division).
__device__ __forceinline__ bool near_e4m3_midpoint(float y) {
  const float a = fabsf(y);
  const int d = int(__float_as_uint(a) & 0xFFFFFu) - 0x80000;
  return (a < 0.015625f && a != 0.f) || (d >= -4 && d <= 4);
}

template <int N>
__device__ __forceinline__ void block_quotients(const float* x, float sc, float rc, float (&y)[N]) {
  bool any = false;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    y[i] = x[i] * rc;
    any |= near_e4m3_midpoint(y[i]);
  }
  if (__ballot(any) != 0) {
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (near_e4m3_midpoint(y[i])) y[i] = x[i] / sc;
  }
}

// Reductions over aligned groups of 4 or 16 lanes with DPP lane moves (VALU
// operations, no LDS crossbar): swaps within pairs and quads (quad_perm), then
// the mirror within each 8 lanes (which pairs quad 0 with quad 1 once each
// quad is uniform) and within each 16 (which pairs the two halves).  Every
// lane of a group ends with the group's result.
__device__ __forceinline__ int dpp_swap1(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ int dpp_swap2(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
}
__device__ __forceinline__ int dpp_mirror8(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
}
__device__ __forceinline__ int dpp_mirror16(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
}
__device__ __forceinline__ float max4(float v) {
  v = fmaxf(v, __int_as_float(dpp_swap1(__float_as_int(v))));
  return fmaxf(v, __int_as_float(dpp_swap2(__float_as_int(v))));
}
__device__ __forceinline__ float max16(float v) {
  v = max4(v);
  v = fmaxf(v, __int_as_float(dpp_mirror8(__float_as_int(v))));
  return fmaxf(v, __int_as_float(dpp_mirror16(__float_as_int(v))));
}
// OR over 16 lanes of values that are uniform within each group of 4
__device__ __forceinline__ uint32_t or16_of_quads(uint32_t v) {
  v |= uint32_t(dpp_mirror8(int(v)));
  return v | uint32_t(dpp_mirror16(int(v)));
}

// Row quantisation fused into a kernel that writes the rows (FP8 modes, bf16
// rows): none, MXFP8 (e8m0 scale per 32 columns) or blockwise (fp32 scale per
// 128 columns).
enum { QM_NONE = 0, QM_MX = 1, QM_BLOCK = 2 };

// e4m3 codes (and the group's scale entry, valid in every lane) of eight
// consecutive values whose 32-column (MX: 4 lanes) or 128-column (blockwise:
// 16 lanes) group is held by aligned consecutive lanes, all of which call this.
template <int QM>
__device__ __forceinline__ uint2 quantise8(const float (&v)[8], int lane, uint32_t& entry) {
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
  uint2 codes;
  if constexpr (QM == QM_MX) {
    am = max4(am);
    const int X = e8m0_exponent(am);
    const float m = ldexpf(1.f, -X);
    codes.x = pack_e4m3x4(v[0] * m, v[1] * m, v[2] * m, v[3] * m);
    codes.y = pack_e4m3x4(v[4] * m, v[5] * m, v[6] * m, v[7] * m);
    entry = or16_of_quads(uint32_t(X + 127) << (8 * ((lane & 15) >> 2)));
  } else {
    am = max16(am);
    const float s = am == 0.f ? 1.f : am / 448.f;
    float y[8];
    block_quotients(v, s, 1.f / s, y);
    codes.x = pack_e4m3x4(y[0], y[1], y[2], y[3]);
    codes.y = pack_e4m3x4(y[4], y[5], y[6], y[7]);
    entry = __float_as_uint(s);
  }
  return codes;
}

}  // namespace moe
