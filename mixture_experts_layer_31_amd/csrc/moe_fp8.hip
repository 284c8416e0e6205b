// FP8 paths of the MoE layer: blockwise FP8 (fp32 scale per 1x128 activation
// tile and per 128x128 weight block) and MXFP8 (e8m0 scale per 32 contiguous
// contraction elements), both on OCP e4m3 elements.  The pages list BF16, MXFP8
// and blockwise FP8, plus an fp8_bwd mode with a BF16 forward and an FP8
// backward (Prime Mega MoE news item, "How does the fused kernel work?" and
// "How do developers use it?").
//
// Every FP8 GEMM here is "NT": both operands are stored with the contraction
// index contiguous, so both are staged with the same direct-to-LDS loads and
// 128-byte swizzled rows as the bf16 kernels (a 128-element fp8 k-step is 128
// bytes, like a 64-element bf16 step).  The quantisers produce operands in that
// orientation: activations whose contraction runs along the row are quantised
// in place; operands contracted over tokens (the weight-gradient GEMMs) and
// weights contracted over their first dimension are transposed while being
// quantised (the quantiser stages a 128 x 128 tile in LDS anyway).
//
// Scales are stored as 4-byte entries in [k-step][row] order: an fp32 block
// scale, or the four e8m0 bytes of the step's four 32-element groups.  For one
// k-step the entries of a tile's rows are contiguous, so they travel to LDS in
// the same pipeline as the data (one 1 KB direct-to-LDS load per operand).
//
// MXFP8 uses v_mfma_scale_f32_32x32x64_f8f6f4 with the scales applied by the
// matrix core.  Its operand layout (established with an in-bounds probe): lane
// l holds row (l & 31); bytes 0-15 are k = 16*(l>>5) + 0..15 and bytes 16-31 are
// k = 32 + 16*(l>>5) + 0..15 of the 64-wide step; the scale register of lane l
// covers row (l & 31), k-group (l >> 5), and op_sel picks its byte.
// Blockwise FP8 runs the same instruction with unit scales over each 128-wide
// k-step and promotes the partial sum in fp32: acc += partial * s_a * s_b.
#include <type_traits>

#include "moe_fp8_codec.h"
#include "moe_gemm_common.h"
#include "moe_pair.h"

namespace moe {
namespace {

using namespace gemm;

typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Encodings.

enum QMode { Q_MX = 1, Q_BLOCK_TILE = 2 };  // weight quantiser modes

// ---------------------------------------------------------------------------
// Weight quantiser (moe_prepare_weights): one workgroup quantises a 128 (r) x
// 128 (c) tile of one expert's bf16 weight matrix [R, C].
//   TRANS = false: the contraction runs along c; codes out[r][c], scale entry
//                  [c-step][r].
//   TRANS = true:  the contraction runs along r; codes out[c][r], scale entry
//                  [r-step][c].
// Blockwise tiles share one fp32 scale (the 128 x 128 block's amax / 448);
// MXFP8 groups are 32 consecutive contraction elements.  Activations have
// their own kernels below (quant_rows_kernel, quant_tokens_kernel).
struct QArgs {
  const uint16_t* in;   // bf16 rows of length cols
  int64_t in_bstride;   // elements between batches (weights: between experts)
  int cols;             // input row length (multiple of 128)
  int rows;             // weights: rows per expert (multiple of 128)
  uint8_t* out;
  int64_t out_ld, out_bstride;
  uint32_t* sc;
  int64_t sc_ld, sc_bstride;
  const int32_t* offsets;  // token quantiser: [E+1] expert row offsets
  const int32_t* tstart;   // token quantiser: [E+1] prefix of ceil(count / 128)
  const int32_t* src;      // gathering token quantiser: [N] pair of each permuted row
  const float* topk_w;     // TOK_GATHER_W: [T*K] routing weight of each pair
  int K;                   // gathering token quantiser: pairs per token
  uint8_t* rcodes;         // token quantiser with ROWQ: the rows' own codes [N, cols]
  uint32_t* rsc;           //   and their scale entries [cols / 128][rsc_ld]
  int64_t rsc_ld;
  int E;
  int ntr;                 // weights: r-steps per expert
  int total_rows;          // row quantiser: rows of the input
};

template <bool TRANS, int MODE>
__global__ void __launch_bounds__(256) quant_tile_kernel(QArgs p) {
  static_assert(MODE == Q_MX || MODE == Q_BLOCK_TILE, "weights: MXFP8 groups or 128x128 blocks");
  __shared__ __attribute__((aligned(16))) uint16_t tile[128 * 128];
  __shared__ float red[4];
  const int ctiles = p.cols / 128;
  const int rt = blockIdx.x / ctiles, ct = blockIdx.x % ctiles;
  const int b = rt / p.ntr;  // expert
  const int r0 = (rt % p.ntr) * 128, valid = min(128, p.total_rows - r0), slot0 = r0;
  const int c0 = ct * 128;
  const uint16_t* in = p.in + b * p.in_bstride;
  const int t = threadIdx.x, lane = t & 63;

  // Each thread owns 64 consecutive values along the contraction axis:
  // index q (row for !TRANS, column for TRANS) = t / 2, half h = t & 1.
  const int q = t >> 1, h = t & 1;
  float v[64];
  if constexpr (TRANS) {
    for (int i = t; i < 128 * 16; i += 256) {  // 16 chunks of 8 per row
      const int r = i >> 4, ch = i & 15;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (r < valid) val = *reinterpret_cast<const uint4*>(in + size_t(r0 + r) * p.cols + c0 + ch * 8);
      *reinterpret_cast<uint4*>(&tile[r * 128 + ch * 8]) = val;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 64; ++i) v[i] = bf2f(tile[(h * 64 + i) * 128 + q]);
  } else {
    const bool ok = q < valid;
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
      uint4 val = make_uint4(0, 0, 0, 0);
      if (ok) val = *reinterpret_cast<const uint4*>(in + size_t(r0 + q) * p.cols + c0 + h * 64 + ch * 8);
      const uint32_t w[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[ch * 8 + 2 * k] = __uint_as_float(w[k] << 16);
        v[ch * 8 + 2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    }
  }

  float am[2] = {0.f, 0.f};  // amax of the two 32-groups
#pragma unroll
  for (int i = 0; i < 64; ++i) am[i >> 5] = fmaxf(am[i >> 5], fabsf(v[i]));

  uint32_t entry = 0;  // scale entry written by h == 0
  uint32_t packed[16];
  if constexpr (MODE == Q_MX) {
    // x * 2^-X is exact, so the hardware conversion sees the exact quotient
    const int X0 = e8m0_exponent(am[0]), X1 = e8m0_exponent(am[1]);
    const float mul[2] = {ldexpf(1.f, -X0), ldexpf(1.f, -X1)};
    const uint32_t mine = uint32_t(X0 + 127) | (uint32_t(X1 + 127) << 8);
    const uint32_t other = __shfl_xor(mine, 1, 64);
    entry = h == 0 ? (mine | (other << 16)) : 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float m = mul[i >> 3];
      packed[i] = pack_e4m3x4(v[4 * i] * m, v[4 * i + 1] * m, v[4 * i + 2] * m, v[4 * i + 3] * m);
    }
  } else {
    // the whole 128 x 128 block's amax
    float amax = fmaxf(am[0], am[1]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if (lane == 0) red[t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float sc = amax == 0.f ? 1.f : amax / 448.f;
    entry = __float_as_uint(sc);
    const float rc = 1.f / sc;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float y[8];
      block_quotients(v + 8 * i, sc, rc, y);
      packed[2 * i] = pack_e4m3x4(y[0], y[1], y[2], y[3]);
      packed[2 * i + 1] = pack_e4m3x4(y[4], y[5], y[6], y[7]);
    }
  }
  uint8_t* out = p.out + b * p.out_bstride;
  uint32_t* sc = p.sc + b * p.sc_bstride;
  if constexpr (TRANS) {
    uint4* dst = reinterpret_cast<uint4*>(out + size_t(c0 + q) * p.out_ld + slot0 + h * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dst[i] = make_uint4(packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]);
    if (h == 0) sc[size_t(slot0 / 128) * p.sc_ld + c0 + q] = entry;
  } else {
    if (q < valid) {
      uint4* dst = reinterpret_cast<uint4*>(out + size_t(r0 + q) * p.out_ld + c0 + h * 64);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dst[i] = make_uint4(packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]);
      if (h == 0) sc[size_t(ct) * p.sc_ld + r0 + q] = entry;
    }
  }
}

// Row quantiser for activations whose contraction runs along the row: one
// workgroup per 128 (rows) x 128 (columns) tile; sixteen lanes share a row
// (eight consecutive values each), so every load and store instruction covers
// four whole 256-byte (in) / 128-byte (out) row segments, and the group amax is
// a reduction over 4 (MX, 32 columns) or 16 (blockwise, 128 columns) lanes.
template <bool MX>
__global__ void __launch_bounds__(256) quant_rows_kernel(QArgs p) {
  const int ctiles = p.cols / 128;
  const int rt = blockIdx.x / ctiles, ct = blockIdx.x % ctiles;
  const int r0 = rt * 128, valid = min(128, p.total_rows - r0);
  const int c0 = ct * 128;
  const int lane = threadIdx.x & 63, l16 = lane & 15;
  const int rw = (threadIdx.x >> 6) * 4 + (lane >> 4);  // row within a 16-row slab
  uint4 raw[8];
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int r = it * 16 + rw;
    raw[it] = r < valid ? *reinterpret_cast<const uint4*>(p.in + size_t(r0 + r) * p.cols + c0 + 8 * l16)
                        : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int r = it * 16 + rw;
    float v[8];
    const uint32_t w[4] = {raw[it].x, raw[it].y, raw[it].z, raw[it].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
    float am = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) am = fmaxf(am, fabsf(v[k]));
    uint32_t entry;
    uint2 codes;
    if constexpr (MX) {
      am = max4(am);
      const int X = e8m0_exponent(am);
      const float m = ldexpf(1.f, -X);
      codes.x = pack_e4m3x4(v[0] * m, v[1] * m, v[2] * m, v[3] * m);
      codes.y = pack_e4m3x4(v[4] * m, v[5] * m, v[6] * m, v[7] * m);
      // byte g of the entry: group g's exponent
      entry = or16_of_quads(uint32_t(X + 127) << (8 * (l16 >> 2)));
    } else {
      am = max16(am);
      const float sc = am == 0.f ? 1.f : am / 448.f;
      const float rc = 1.f / sc;
      float y[8];
      block_quotients(v, sc, rc, y);
      codes.x = pack_e4m3x4(y[0], y[1], y[2], y[3]);
      codes.y = pack_e4m3x4(y[4], y[5], y[6], y[7]);
      entry = __float_as_uint(sc);
    }
    if (r < valid) {
      *reinterpret_cast<uint2*>(p.out + size_t(r0 + r) * p.out_ld + c0 + 8 * l16) = codes;
      if (l16 == 0) p.sc[size_t(ct) * p.sc_ld + r0 + r] = entry;
    }
  }
}

// Where the token quantiser's rows come from:
//   TOK_PERM      row q of the permuted activations `in` [N, C] (read once:
//                 streaming loads);
//   TOK_GATHER    the dispatched token itself, row src[q] / K of `in` [T, C]
//                 (x: the dispatched rows need not be stored at all);
//   TOK_GATHER_W  the combine-backward's row w * dy: row src[q] / K of `in`
//                 (dy) times the pair's routing weight, the fp32 product
//                 rounded to bf16 as the combine-backward rounds it.
// A token's row is gathered once per routed pair (K times), mostly from the
// caches: plain loads.
enum TokSrc { TOK_PERM = 0, TOK_GATHER = 1, TOK_GATHER_W = 2 };

// Eight bf16 values times w, each fp32 product rounded to bf16 (RNE).
__device__ __forceinline__ uint4 scale_bf16x8(const uint4& v, float w) {
  const uint32_t in[4] = {v.x, v.y, v.z, v.w};
  uint32_t out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float lo = w * __uint_as_float(in[k] << 16), hi = w * __uint_as_float(in[k] & 0xffff0000u);
    out[k] = pack_bf16x2(lo, hi);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// Token quantiser for activations contracted over tokens (the weight-gradient
// operands): one workgroup per 128-token step of an expert segment x NCT
// column tiles of 128.  A tile is loaded with whole 256-byte row segments per
// sixteen lanes into LDS, its 32-byte column blocks XOR-swizzled by row; then
// each thread takes one column and 64 consecutive tokens, four tokens per
// ds_read_b64_tr_b16 (a sixteen-lane group reads a 4-token x 16-column block
// and lane i receives column i).  The other 64 tokens of the column are in
// lane ^ 16, so the 128-token amax is one shuffle away.  The codes go back
// through the same LDS tile as 128 rows of 128 bytes (one per column, 16-byte
// chunks XOR-swizzled by row), so each wave's store covers eight whole
// 128-byte output rows instead of 16-byte pieces of 32 rows.  With NCT > 1 the
// next tile's rows are loaded into registers as soon as the current tile is
// in LDS, so they arrive while it is quantised and stored, and a gathered
// row's index and weight are looked up once for all NCT tiles.
template <bool MX, int SRC, int NCT, bool ROWQ = false>
__global__ void __launch_bounds__(256) quant_tokens_kernel(QArgs p) {
  __shared__ __attribute__((aligned(16))) char tile[128 * 256];
  const int groups = p.cols / (128 * NCT);
  const int rt = blockIdx.x / groups, cg = blockIdx.x % groups;
  if (rt >= p.tstart[p.E]) return;
  const int lo = tile_expert(p.tstart, p.E, 1, rt);
  const int r0 = p.offsets[lo] + (rt - p.tstart[lo]) * 128;
  const int valid = min(128, p.offsets[lo + 1] - r0);
  const int slot0 = rt * 128;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15;
  auto at = [&](int r, int cb) { return r * 256 + ((cb ^ (r & 7)) << 5); };  // 32-byte block cb of row r
  auto oat = [&](int row, int ch) { return row * 128 + ((ch ^ (row & 7)) << 4); };
  // this thread's 8 rows (16 apart): the input row each comes from (-1: past
  // the segment's end, zeros)
  const int rw = w * 4 + (lane >> 4);
  int row[8];
  float wt[SRC == TOK_GATHER_W ? 8 : 1];
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int r = it * 16 + rw;
    row[it] = -1;
    if constexpr (SRC == TOK_GATHER_W) wt[it] = 0.f;
    if (r < valid) {
      if constexpr (SRC == TOK_PERM) {
        row[it] = r0 + r;
      } else {
        const int pr = p.src[r0 + r];
        row[it] = pr / p.K;
        if constexpr (SRC == TOK_GATHER_W) wt[it] = p.topk_w[pr];
      }
    }
  }
  uint4 raw[8];
  auto load = [&](int c0) {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      raw[it] = make_uint4(0, 0, 0, 0);
      if (row[it] >= 0) {
        const uint16_t* a = p.in + size_t(row[it]) * p.cols + c0 + 8 * l16;
        if constexpr (SRC == TOK_PERM) raw[it] = load16_nt(a);
        else raw[it] = *reinterpret_cast<const uint4*>(a);
      }
    }
  };
  load(cg * NCT * 128);
  for (int k = 0; k < NCT; ++k) {
    const int c0 = (cg * NCT + k) * 128;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = it * 16 + rw;
      if constexpr (SRC == TOK_GATHER_W) raw[it] = scale_bf16x8(raw[it], wt[it]);
      *reinterpret_cast<uint4*>(tile + at(r, l16 >> 1) + (l16 & 1) * 16) = raw[it];
    }
    if constexpr (ROWQ) {
      // the same rows quantised along their columns, as quant_rows_kernel does
      // (sixteen lanes per row): one read of the input for both operands
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int r = it * 16 + rw;
        const uint32_t wd[4] = {raw[it].x, raw[it].y, raw[it].z, raw[it].w};
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = __uint_as_float(wd[e] << 16);
          f[2 * e + 1] = __uint_as_float(wd[e] & 0xffff0000u);
        }
        uint32_t ent;
        const uint2 codes = quantise8<MX ? QM_MX : QM_BLOCK>(f, lane, ent);
        if (r < valid) {
          *reinterpret_cast<uint2*>(p.rcodes + size_t(r0 + r) * p.cols + c0 + 8 * l16) = codes;
          if (l16 == 0) p.rsc[size_t(c0 / 128) * p.rsc_ld + r0 + r] = ent;
        }
      }
    }
    if (k + 1 < NCT) load(c0 + 128);  // in flight while this tile is quantised and stored
    __syncthreads();
    const int g = lane >> 4, h = g & 1, cb = 2 * w + (g >> 1);
    const int q = 16 * cb + l16;  // this thread's column; tokens 64h .. 64h + 63
    float v[64];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 64 * h + 4 * j + (l16 >> 2);
      const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)AS3(tile + at(r, cb) + (l16 & 3) * 8));
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * j + e] = __uint_as_float(uint32_t(uint16_t(x[e])) << 16);
    }
    float am[2] = {0.f, 0.f};  // amax of the two 32-token groups
#pragma unroll
    for (int i = 0; i < 64; ++i) am[i >> 5] = fmaxf(am[i >> 5], fabsf(v[i]));
    uint32_t packed[16], entry;
    if constexpr (MX) {
      const int X0 = e8m0_exponent(am[0]), X1 = e8m0_exponent(am[1]);
      const float mul[2] = {ldexpf(1.f, -X0), ldexpf(1.f, -X1)};
      const uint32_t mine = uint32_t(X0 + 127) | (uint32_t(X1 + 127) << 8);
      entry = mine | (__shfl_xor(mine, 16, 64) << 16);  // meaningful in the h == 0 lane
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float m = mul[i >> 3];
        packed[i] = pack_e4m3x4(v[4 * i] * m, v[4 * i + 1] * m, v[4 * i + 2] * m, v[4 * i + 3] * m);
      }
    } else {
      float amax = fmaxf(am[0], am[1]);
      amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
      const float sc = amax == 0.f ? 1.f : amax / 448.f;
      const float rc = 1.f / sc;
      entry = __float_as_uint(sc);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float y[8];
        block_quotients(v + 8 * i, sc, rc, y);
        packed[2 * i] = pack_e4m3x4(y[0], y[1], y[2], y[3]);
        packed[2 * i + 1] = pack_e4m3x4(y[4], y[5], y[6], y[7]);
      }
    }
    if (h == 0) p.sc[size_t(slot0 / 128) * p.sc_ld + c0 + q] = entry;
    // codes of column q, tokens 64h .. 64h + 63: chunks 4h .. 4h + 3 of LDS row q
    __syncthreads();  // every wave is done reading the input tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(tile + oat(q, 4 * h + i)) =
          make_uint4(packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]);
    __syncthreads();
    // 128 rows of 128 bytes, eight lanes per row.  The gathering forms store
    // with streaming stores, which keep the re-read token rows in the caches
    // (235B dYw 0.44 -> 0.43 ms); the permuted form keeps plain stores (the
    // 30B MXFP8 dH pass measured 0.107 ms with them, 0.125 streaming)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int id = threadIdx.x + 256 * u, row = id >> 3, ch = id & 7;
      uint8_t* dst = p.out + size_t(c0 + row) * p.out_ld + slot0 + 16 * ch;
      const uint4 val = *reinterpret_cast<const uint4*>(tile + oat(row, ch));
      if constexpr (SRC == TOK_PERM) *reinterpret_cast<uint4*>(dst) = val;
      else store16_nt(dst, val);
    }
    __syncthreads();  // the next tile's rows overwrite the staged codes
  }
}

// ---------------------------------------------------------------------------
// FP8 GEMM.

// Scale stager: one 1 KB direct-to-LDS load per k-step (256 four-byte entries
// of consecutive rows; lane l fetches rows 4l..4l+3).
struct ScaleStager {
  i32x4 rsrc;
  int vb, step;
  bool active;
  __device__ __forceinline__ void issue(uint32_t lds, int kt) const {
    if (active) dma16(rsrc, lds, vb + kt * step);
  }
};

// fp8 fragment (32 bytes: two 16-byte chunks of a 128-byte row) for sub-step kk.
__device__ __forceinline__ i32x8 frag8(const char* tile, int row, int kk, int lane) {
  const int h = lane >> 5;
  const int c0 = 4 * kk + h, c1 = 4 * kk + 2 + h;
  const i32x4 a = *reinterpret_cast<const i32x4*>(tile + row * 128 + ((c0 ^ swz_k(row)) << 4));
  const i32x4 b = *reinterpret_cast<const i32x4*>(tile + row * 128 + ((c1 ^ swz_k(row)) << 4));
  const i32x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return r;
}

template <int SEL>
__device__ __forceinline__ f32x16 mfma8(i32x8 b, i32x8 a, f32x16 c, int sb, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 0, 0, SEL, sb, SEL, sa);
}

// The MXFP8 loop: 128-element k-steps in two LDS stages of 128-byte rows; the
// matrix core applies the e8m0 scales (the lane's row and column entries,
// shifted so that op_sel 0 and 2 pick the lane's 32-group of each 64-deep
// half).  Each step waits for its stage, meets every wave at the barrier and
// issues the next step's loads into the other stage; then a half-step's two B
// fragments stay in registers while its A fragments stream one 32-row block
// ahead of the MFMAs that use them (the second half's B fragments are read
// beside the first half's last blocks), so only the step's first three
// fragments are read in front of the matrix core.  All branches stay at the
// top of the step, before the MFMAs.
template <class TL, class SA, class SB>
__device__ __forceinline__ void mainloop8(char* smem, const SA& sa, const SB& sb,
                                          const ScaleStager& ssa, const ScaleStager& ssb,
                                          int ktiles, f32x16 (&acc)[TL::WMT][TL::WNT], int wave,
                                          int lane) {
  constexpr int BM = TL::BM, BN = TL::BN, WM = TL::WM, WN = TL::WN;
  constexpr int WMT = TL::WMT, WNT = TL::WNT;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, STAGE = A_BYTES + B_BYTES + 2048;
  static_assert(TL::STAGES == 2, "two stages");
  static_assert(WMT >= 2 && WNT == 2, "the second half's B fragments go beside the last two A blocks");
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;
  const uint32_t base = lds_addr(smem);
  auto issue = [&](int s, int kt) {
    const uint32_t st = base + s * STAGE;
    sa.issue(st, wave, kt);
    sb.issue(st + A_BYTES, wave, kt);
    ssa.issue(st + A_BYTES + B_BYTES, kt);
    ssb.issue(st + A_BYTES + B_BYTES + 1024, kt);
  };
  const int sh = 8 * (lane >> 5);
  if (ktiles > 0) issue(0, 0);
  for (int kt = 0; kt < ktiles; ++kt) {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (kt + 1 < ktiles) issue((kt + 1) & 1, kt + 1);
    const char* ta = smem + (kt & 1) * STAGE;
    const char* tb = ta + A_BYTES;
    auto fa = [&](int h, int i) { return frag8(ta, wm * WM + i * 32 + (lane & 31), h, lane); };
    auto fb = [&](int h, int j) { return frag8(tb, wn * WN + j * 32 + (lane & 31), h, lane); };
    const uint32_t* sca = reinterpret_cast<const uint32_t*>(tb + B_BYTES);
    const uint32_t* scb = sca + 256;
    int sa_w[WMT], sb_w[WNT];
#pragma unroll
    for (int i = 0; i < WMT; ++i) sa_w[i] = int(sca[wm * WM + i * 32 + (lane & 31)] >> sh);
#pragma unroll
    for (int j = 0; j < WNT; ++j) sb_w[j] = int(scb[wn * WN + j * 32 + (lane & 31)] >> sh);
    i32x8 bc[WNT], bn[WNT], ac, an;
#pragma unroll
    for (int j = 0; j < WNT; ++j) bc[j] = fb(0, j);
    ac = fa(0, 0);
    auto half = [&](auto H) {
      constexpr int h = decltype(H)::value;
#pragma unroll
      for (int i = 0; i < WMT; ++i) {
        if (i + 1 < WMT) an = fa(h, i + 1);
        if constexpr (h == 0) {
          if (i == WMT - 2) bn[0] = fb(1, 0);
          if (i == WMT - 1) {
            bn[1] = fb(1, 1);
            an = fa(1, 0);
          }
        }
#pragma unroll
        for (int j = 0; j < WNT; ++j)
          acc[i][j] = mfma8<2 * h>(bc[j], ac, acc[i][j], sb_w[j], sa_w[i]);
        // the reads first, so they have both MFMAs (and the other wave's) to return
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, WNT, 0);
        __builtin_amdgcn_sched_barrier(0);
        ac = an;
      }
      if constexpr (h == 0) {
#pragma unroll
        for (int j = 0; j < WNT; ++j) bc[j] = bn[j];
      }
    };
    half(std::integral_constant<int, 0>{});
    half(std::integral_constant<int, 1>{});
  }
}

// The blockwise loop on 128-element k-steps (one scale block per step) in two
// LDS stages of 128-byte rows, as the MX loop: a 32x32 block's two 64-deep
// MFMAs accumulate into a partial that is promoted once per step,
// acc += part * s_a[row] * s_b[col].  Token-grouped GEMMs (SB_COL false): s_b
// is uniform over a 32-column block (weights in 128 x 128 blocks), one scale
// product and 16 FMAs per block and step.  Weight gradients (SB_COL true):
// both operands are scaled per 128-token block along an output axis, so each
// of the lane's 16 columns has its own s_b, read from LDS right before the
// promotion (16 products and 16 FMAs).  The step's B fragments stay in
// registers while the A fragments stream one 32-row block at a time, which
// keeps the loop inside 256 registers.
template <class TL, bool SB_COL, class SA, class SB>
__device__ __forceinline__ void block8(char* smem, const SA& sa, const SB& sb,
                                       const ScaleStager& ssa, const ScaleStager& ssb, int ktiles,
                                       f32x16 (&acc)[TL::WMT][TL::WNT], int wave, int lane) {
  constexpr int BM = TL::BM, BN = TL::BN, WM = TL::WM, WN = TL::WN;
  constexpr int WMT = TL::WMT, WNT = TL::WNT;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, STAGE = A_BYTES + B_BYTES + 2048;
  static_assert(TL::STAGES == 2, "two stages");
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;
  const uint32_t base = lds_addr(smem);
  auto issue = [&](int s, int kt) {
    const uint32_t st = base + s * STAGE;
    sa.issue(st, wave, kt);
    sb.issue(st + A_BYTES, wave, kt);
    ssa.issue(st + A_BYTES + B_BYTES, kt);
    ssb.issue(st + A_BYTES + B_BYTES + 1024, kt);
  };
  if (ktiles > 0) issue(0, 0);
  for (int kt = 0; kt < ktiles; ++kt) {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (kt + 1 < ktiles) issue((kt + 1) & 1, kt + 1);
    const char* ta = smem + (kt & 1) * STAGE;
    const char* tb = ta + A_BYTES;
    const uint32_t* sca = reinterpret_cast<const uint32_t*>(tb + B_BYTES);
    const uint32_t* scb = sca + 256;
    i32x8 b0[WNT], b1[WNT];
    float sbv[WNT];
#pragma unroll
    for (int j = 0; j < WNT; ++j) {
      const int n = wn * WN + j * 32;
      b0[j] = frag8(tb, n + (lane & 31), 0, lane);
      b1[j] = frag8(tb, n + (lane & 31), 1, lane);
      sbv[j] = __uint_as_float(scb[n]);
    }
    const int r0 = wm * WM + (lane & 31);
    i32x8 a0 = frag8(ta, r0, 0, lane), a1 = frag8(ta, r0, 1, lane);
    float sav = __uint_as_float(sca[r0]);
    {
      // Software-pipelined over the wave's 32x32 blocks u = 2i + j: block u's two
      // MFMAs are issued before block u-1 is promoted, so that promotion's VALU
      // work can run while the matrix core works on block u.  Against promoting
      // each block behind its own MFMAs: the weight gradients 2% faster (a timing
      // probe that skipped their promotion put its cost at 0.6 ms of the 235B W1
      // wgrad's 2.8 ms), the 30B token-grouped GEMMs 2-8% (their register spills
      // gone).  At 256 registers a block's A fragments are read at its start
      // instead of one block ahead.
      static_assert(WNT == 2, "two column blocks per wave");
      f32x16 P[2];
      float savp = 0.f;
      auto promote = [&](int i, int j, const f32x16& part, float s) {
        if constexpr (SB_COL) {
          float sbc[16];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 v4 = *reinterpret_cast<const float4*>(scb + wn * WN + j * 32 + acc_col(g, lane));
            sbc[4 * g] = v4.x; sbc[4 * g + 1] = v4.y; sbc[4 * g + 2] = v4.z; sbc[4 * g + 3] = v4.w;
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(part[r], s * sbc[r], acc[i][j][r]);
        } else {
          const float sc = s * sbv[j];
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(part[r], sc, acc[i][j][r]);
        }
      };
#pragma unroll
      for (int u = 0; u < 2 * WMT; ++u) {
        const int i = u >> 1, j = u & 1;
        if (j == 0 && i > 0) {
          a0 = frag8(ta, r0 + i * 32, 0, lane);
          a1 = frag8(ta, r0 + i * 32, 1, lane);
          savp = sav;
          sav = __uint_as_float(sca[r0 + i * 32]);
        }
        P[u & 1] = mfma8<0>(b0[j], a0, f32x16{}, 127, 127);
        P[u & 1] = mfma8<0>(b1[j], a1, P[u & 1], 127, 127);
        if (u > 0) promote((u - 1) >> 1, (u - 1) & 1, P[(u - 1) & 1], j == 0 ? savp : sav);
        // the block's LDS reads, then its MFMAs with the previous block's promotion between
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      promote(WMT - 1, 1, P[1], sav);
    }
  }
}

struct F8Args {
  const int32_t* offsets;  // [E+1] expert row offsets
  const int32_t* eorder;   // [E+1] experts longest first, then the skew flag (wgrad)
  const int32_t* tstart;   // [E+1] m-tile prefix (token-grouped) or 128-token step prefix (wgrad)
  int E, K, ntn;           // K: contraction of a token-grouped GEMM
  int nmajor;              // token-grouped: n-tiles outer within an expert (1) or m-tiles (0)
  int M, N, tm, tn;        // wgrad: dW[e] is [M, N]
  const uint8_t* A;        // token-grouped: [rows, K] codes; wgrad: [M, lda] codes
  int64_t lda;
  const uint32_t* SA;      // scale entries [k-step][sa_ld]
  int64_t sa_ld;
  uint32_t sa_bytes;
  const uint8_t* B;        // token-grouped: weights [E][N][K]; wgrad: [N, ldb]
  int64_t ldb, b_bstride;
  const uint32_t* SB;
  int64_t sb_ld, sb_bstride;
  uint32_t sb_bytes;
  EpiArgs epi;
  int F;
  void* C;                 // wgrad output [E, M, N]
};

// Token-grouped FP8 GEMM: rows of expert e times B[e]^T ([N, K] codes).
template <class TL, bool MX>
constexpr int f8_grouped_lds() {
  return TL::STAGES * ((TL::BM + TL::BN) * 128 + 2048);
}
template <class TL, bool MX, int EPI>
__device__ __forceinline__ void f8_grouped_tile(const F8Args& p, int l, char* smem) {
  constexpr int BM = TL::BM, BN = TL::BN, WN = TL::WN, WAVES = TL::WAVES;
  static_assert(EPI != EPI_SWIGLU || TL::WNT % 2 == 0, "SwiGLU pairs gate/up sub-tiles");
  constexpr int ROWB = 128;  // 128-element k-steps (one MX or blockwise scale step)
  int mt_g, nt, lo;
  if (p.nmajor) {  // expert e owns flat tiles [tstart[e] * ntn, tstart[e + 1] * ntn)
    lo = tile_expert(p.tstart, p.E, p.ntn, l);
    const int t0 = p.tstart[lo], mte = p.tstart[lo + 1] - t0;
    const int local = l - t0 * p.ntn;
    nt = local / mte;
    mt_g = t0 + (local - nt * mte);
  } else {
    mt_g = l / p.ntn;
    nt = l - mt_g * p.ntn;
    lo = tile_expert(p.tstart, p.E, 1, mt_g);
  }
  const int e = lo;
  const int e0 = p.offsets[e];
  const int ne = p.offsets[e + 1] - e0;
  const int m0 = (mt_g - p.tstart[e]) * BM;
  const int rows_valid = min(BM, ne - m0);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;

  KStager<BM, WAVES, ROWB> sa;
  sa.init(make_rsrc(p.A + size_t(e0) * p.K, uint32_t(ne) * p.K),
          [&](int r) { return r < rows_valid ? (m0 + r) * p.K : -1; }, wave, lane);
  auto brow = [&](int n) {
    if constexpr (EPI == EPI_SWIGLU) {
      const int w = n / WN, rem = n % WN;
      const int half = rem / (WN / 2), c = rem % (WN / 2);
      return half * p.F + nt * (BN / 2) + w * (WN / 2) + c;
    } else {
      return nt * BN + n;
    }
  };
  KStager<BN, WAVES, ROWB> sb;
  sb.init(make_rsrc(p.B + size_t(e) * p.b_bstride, uint32_t(p.N) * p.K),
          [&](int n) { return brow(n) * p.K; }, wave, lane);
  ScaleStager ssa{make_rsrc(p.SA, p.sa_bytes), (e0 + m0 + 4 * lane) * 4, int(p.sa_ld * 4), wave == 0};
  ScaleStager ssb{make_rsrc(p.SB + size_t(e) * p.sb_bstride, p.sb_bytes),
                  brow(min(4 * lane, BN - 4)) * 4, int(p.sb_ld * 4), wave == 1};

  f32x16 acc[TL::WMT][TL::WNT];
  zero(acc);
  if constexpr (MX) mainloop8<TL>(smem, sa, sb, ssa, ssb, p.K / 128, acc, wave, lane);
  else block8<TL, false>(smem, sa, sb, ssa, ssb, p.K / 128, acc, wave, lane);
  static_assert(f8_grouped_lds<TL, MX>() >= grouped_epi_lds<TL, EPI>(), "epilogue staging exceeds LDS");
  grouped_epilogue<TL, EPI, false, f8_grouped_lds<TL, MX>()>(p.epi, acc, size_t(e0) + m0, rows_valid,
                                                               nt, wm, wn, lane, smem, threadIdx.x);
}

// The tiles from a grid of resident workgroups, in rounds of gridDim.x (an XCD
// takes a contiguous run of the list per round), as the bf16 grouped GEMM.
template <class TL, bool MX, int EPI>
__global__ void __launch_bounds__(TL::THREADS, 1) f8_grouped_kernel(F8Args p) {
  __shared__ __attribute__((aligned(1024))) char smem[f8_grouped_lds<TL, MX>()];
  const int total = p.tstart[p.E] * p.ntn;
  for (int l = xcd_remap(blockIdx.x, gridDim.x); l < total; l += gridDim.x) {
    f8_grouped_tile<TL, MX, EPI>(p, l, smem);
    __syncthreads();  // the next tile's loads overwrite the epilogue's staging
  }
}

// Per-expert FP8 weight-gradient GEMM over the expert's padded token steps.
template <class TL>
constexpr int f8_wgrad_lds() { return TL::STAGES * ((TL::BM + TL::BN) * 128 + 2048); }
template <class TL, bool MX, bool OUT_F32>
__device__ __forceinline__ void f8_wgrad_tile(const F8Args& p, int l, char* smem) {
  constexpr int BM = TL::BM, BN = TL::BN, WAVES = TL::WAVES;
  constexpr int ROWB = 128;
  const ExpertTile et = expert_tile(p.eorder, l, p.tm * p.tn);
  const int e = et.e;
  int mt, nt;
  wgrad_mn(et.rem, p.tm, p.tn, mt, nt);
  const int s0 = p.tstart[e], ksteps = p.tstart[e + 1] - s0;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;
  f32x16 acc[TL::WMT][TL::WNT];
  zero(acc);
  if (ksteps > 0) {
    const size_t kb0 = size_t(s0) * 128;  // first padded token of the expert
    KStager<BM, WAVES, ROWB> sa;
    sa.init(make_rsrc(p.A + size_t(mt) * BM * p.lda + kb0, uint32_t(BM - 1) * p.lda + ksteps * 128),
            [&](int r) { return r * int(p.lda); }, wave, lane);
    KStager<BN, WAVES, ROWB> sb;
    sb.init(make_rsrc(p.B + size_t(nt) * BN * p.ldb + kb0, uint32_t(BN - 1) * p.ldb + ksteps * 128),
            [&](int r) { return r * int(p.ldb); }, wave, lane);
    ScaleStager ssa{make_rsrc(p.SA, p.sa_bytes), int((size_t(s0) * p.sa_ld + mt * BM + 4 * lane) * 4),
                    int(p.sa_ld * 4), wave == 0};
    ScaleStager ssb{make_rsrc(p.SB, p.sb_bytes), int((size_t(s0) * p.sb_ld + nt * BN + 4 * lane) * 4),
                    int(p.sb_ld * 4), wave == 1};
    if constexpr (MX) mainloop8<TL>(smem, sa, sb, ssa, ssb, ksteps, acc, wave, lane);
    else block8<TL, true>(smem, sa, sb, ssa, ssb, ksteps, acc, wave, lane);
  }
  static_assert(f8_wgrad_lds<TL>() >= wgrad_epi_lds<TL, OUT_F32>(), "epilogue staging exceeds LDS");
  wgrad_epilogue<TL, OUT_F32>(p.C, p.M, p.N, e, mt, nt, acc, wm, wn, lane, smem, threadIdx.x);
}

// Experts longest first, one workgroup per tile, as the bf16 weight-gradient GEMM.
template <class TL, bool MX, bool OUT_F32>
__global__ void __launch_bounds__(TL::THREADS, 1) f8_wgrad_kernel(F8Args p) {
  __shared__ __attribute__((aligned(1024))) char smem[f8_wgrad_lds<TL>()];
  f8_wgrad_tile<TL, MX, OUT_F32>(p, expert_tile_start(p.eorder, p.E), smem);
}

// A token-grouped FP8 GEMM (TLA) and an FP8 weight gradient (TLB) in one
// launch over the paired schedule of moe_pair.h.
template <class TLA, bool MX, int EPI, class TLB>
__global__ void __launch_bounds__(TLA::THREADS, 1) f8_pair_kernel(F8Args a, F8Args b, PairSched ps) {
  static_assert(TLA::THREADS == TLB::THREADS, "one workgroup shape for both GEMMs");
  constexpr int LA = f8_grouped_lds<TLA, MX>(), LB = f8_wgrad_lds<TLB>();
  constexpr int PIPE = LA > LB ? LA : LB;
  __shared__ __attribute__((aligned(1024))) char smem[PIPE + sizeof(PairLds)];
  PairLds& L = *reinterpret_cast<PairLds*>(smem + PIPE);
  pair_setup<TLA::THREADS>(ps, L);
  int q = blockIdx.x % kPairQueues;
  for (;;) {
    const int g = pair_next(ps, L, &q);
    if (g < 0) break;
    const PairItem it = pair_decode(ps, L, g);
    if (it.is_a) f8_grouped_tile<TLA, MX, EPI>(a, it.l, smem);
    else f8_wgrad_tile<TLB, MX, false>(b, it.l, smem);
    __syncthreads();  // the next item's loads overwrite this one's epilogue staging
  }
}

}  // namespace
}  // namespace moe

// ---------------------------------------------------------------------------
// Host side.
namespace moe {
namespace {

using namespace gemm;

// Tiles, measured on the 235B fp8_bwd and 30B MXFP8 layers:
//  * MXFP8 (scales applied by the matrix core): 256 x 256, eight waves, the
//    two-stage 128-element loop (about 10% faster than a four-stage ring of
//    64-element steps: half the barriers, scales read once per 128 elements);
//  * blockwise token-grouped GEMMs: the same tiles and stages with the
//    promoting loop block8 (one promotion per 128-element scale block).  The
//    four-stage ring of 64-element steps it replaced promoted every 64
//    elements, twice per scale block, and spilled registers; block8 cut the
//    235B W1 dgrad from 2.42 to 1.95 ms and the W2 dgrad + SwiGLU-backward
//    from 1.93 to 1.69 ms (30B blockwise step 4.98 -> 4.69 ms);
//  * blockwise weight-gradient GEMMs, whose scales vary along both output
//    axes (a scale product per output element and 128-token block): the same
//    256 x 256 tiles with block8's per-column-scale path (each column's 16
//    scales read from LDS right before its promotion, so the streaming loop
//    still fits 256 registers).  An expert's tile covers only n_e / 128 steps
//    (8 at the Qwen3 shapes), so the halved prologue and epilogue cost per
//    flop pays: against 256 x 128 tiles of eight 64 x 64 waves in three
//    stages, 235B W1 wgrad 3.50 -> 2.92 ms, W2 wgrad 1.56 -> 1.38 ms (fp8_bwd
//    backward 10.59 -> 9.84 ms), 30B fp8 W1 wgrad 0.81 -> 0.69 ms.
using TileF8 = Tile<256, 256, 2, 4, 2>;
template <bool MX> using F8GrTile = TileF8;
template <bool MX> using F8WgTile = TileF8;

inline int max_steps128(const moe_desc& d) {
  const long long N = (long long)d.T * d.K;
  return int((N + (long long)d.E * 127) / 128);
}

int launch_quant_weights(bool trans, bool mx, const QArgs& a, int blocks, const char* name,
                         hipStream_t s) {
  if (blocks <= 0) return MOE_OK;
  prof_begin(name, s);
  if (trans) {
    if (mx) quant_tile_kernel<true, Q_MX><<<unsigned(blocks), 256, 0, s>>>(a);
    else quant_tile_kernel<true, Q_BLOCK_TILE><<<unsigned(blocks), 256, 0, s>>>(a);
  } else {
    if (mx) quant_tile_kernel<false, Q_MX><<<unsigned(blocks), 256, 0, s>>>(a);
    else quant_tile_kernel<false, Q_BLOCK_TILE><<<unsigned(blocks), 256, 0, s>>>(a);
  }
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// Quantise permuted activations [N, C] along C (rows stay in place).
int quant_rows(const moe_desc& d, const uint16_t* in, int C, bool mx, uint8_t* out, uint32_t* sc,
               const char* name, hipStream_t s) {
  const int N = d.T * d.K;
  QArgs a{};
  a.in = in;
  a.cols = C;
  a.out = out;
  a.out_ld = C;
  a.sc = sc;
  a.sc_ld = N;
  a.ntr = (N + 127) / 128;
  a.total_rows = N;
  const int blocks = a.ntr * (C / 128);
  if (blocks <= 0) return MOE_OK;
  prof_begin(name, s);
  if (mx) quant_rows_kernel<true><<<unsigned(blocks), 256, 0, s>>>(a);
  else quant_rows_kernel<false><<<unsigned(blocks), 256, 0, s>>>(a);
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// Quantise activations along tokens within expert segments, transposed to
// [C, Npad] (row stride npad) with scale entries [step][C].  `in` is the
// permuted rows [N, C] (TOK_PERM) or the per-token rows [T, C] the permuted
// rows are gathered from (TOK_GATHER, TOK_GATHER_W with the weights topk_w).
// With rcodes the same pass also writes the rows' own quantisation along C,
// as quant_rows does: codes [N, C] into rcodes, scale entries [C/128][N] into
// rsc (permuted rows, or gathered rows without weights).
int quant_tokens(const moe_desc& d, const Layout& L, const uint16_t* in, int C, bool mx,
                 uint8_t* out, uint32_t* sc, const char* name, const char* scratch, hipStream_t s,
                 int src = TOK_PERM, const float* topk_w = nullptr, uint8_t* rcodes = nullptr,
                 uint32_t* rsc = nullptr) {
  QArgs a{};
  a.in = in;
  a.cols = C;
  a.out = out;
  a.out_ld = int64_t(max_steps128(d)) * 128;
  a.sc = sc;
  a.sc_ld = C;
  a.offsets = reinterpret_cast<const int32_t*>(scratch + L.offsets);
  a.tstart = reinterpret_cast<const int32_t*>(scratch + L.tiles[1]);
  a.src = reinterpret_cast<const int32_t*>(scratch + L.src);
  a.topk_w = topk_w;
  a.K = d.K;
  a.E = d.E;
  a.rcodes = rcodes;
  a.rsc = rsc;
  a.rsc_ld = int64_t(d.T) * d.K;
  if (src == TOK_GATHER_W && topk_w == nullptr) return MOE_EINVAL;
  if (rcodes != nullptr && rsc == nullptr) return MOE_EINVAL;
  // column tiles per workgroup: the gathering forms pipeline the next tile's
  // row loads behind the current tile's quantisation (at the 30B shape x
  // 0.19 -> 0.17 ms and dYw 0.21 -> 0.19 ms, at 235B dYw 0.43 -> 0.38 ms);
  // the permuted form, whose rows stream from consecutive addresses, is
  // faster at one tile per workgroup and the occupancy that leaves
  const int nct = src == TOK_PERM ? 1 : (C / 128) % 4 == 0 ? 4 : (C / 128) % 2 == 0 ? 2 : 1;
  const int blocks = max_steps128(d) * (C / 128 / nct);
  if (blocks <= 0) return MOE_OK;
  prof_begin(name, s);
#define MOE_QT(S, W) \
  (mx ? quant_tokens_kernel<true, S, W><<<unsigned(blocks), 256, 0, s>>>(a) \
      : quant_tokens_kernel<false, S, W><<<unsigned(blocks), 256, 0, s>>>(a))
#define MOE_QTW(S) (nct == 4 ? MOE_QT(S, 4) : nct == 2 ? MOE_QT(S, 2) : MOE_QT(S, 1))
#define MOE_QTR(S, W) \
  (mx ? quant_tokens_kernel<true, S, W, true><<<unsigned(blocks), 256, 0, s>>>(a) \
      : quant_tokens_kernel<false, S, W, true><<<unsigned(blocks), 256, 0, s>>>(a))
  if (src == TOK_GATHER && rcodes != nullptr)
    (nct == 4 ? MOE_QTR(TOK_GATHER, 4) : nct == 2 ? MOE_QTR(TOK_GATHER, 2) : MOE_QTR(TOK_GATHER, 1));
  else if (src == TOK_GATHER_W && rcodes != nullptr)
    (nct == 4 ? MOE_QTR(TOK_GATHER_W, 4)
              : nct == 2 ? MOE_QTR(TOK_GATHER_W, 2) : MOE_QTR(TOK_GATHER_W, 1));
  else if (src == TOK_GATHER) MOE_QTW(TOK_GATHER);
  else if (src == TOK_GATHER_W) MOE_QTW(TOK_GATHER_W);
  else if (rcodes != nullptr)
    (mx ? quant_tokens_kernel<true, TOK_PERM, 1, true><<<unsigned(blocks), 256, 0, s>>>(a)
        : quant_tokens_kernel<false, TOK_PERM, 1, true><<<unsigned(blocks), 256, 0, s>>>(a));
  else MOE_QT(TOK_PERM, 1);
#undef MOE_QTR
#undef MOE_QTW
#undef MOE_QT
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// Quantise a batch of E weight matrices [R, C].  trans = false: contraction along
// C, codes [E][R][C], entries [E][C/128][R]; trans = true: contraction along R,
// codes [E][C][R], entries [E][R/128][C].  Blockwise mode uses 128 x 128 blocks.
int quant_weights(const moe_desc& d, const uint16_t* w, int R, int C, bool trans, bool mx,
                  uint8_t* out, uint32_t* sc, const char* name, hipStream_t s) {
  QArgs a{};
  a.in = w;
  a.in_bstride = int64_t(R) * C;
  a.cols = C;
  a.rows = R;
  a.total_rows = R;
  a.ntr = R / 128;
  a.out = out;
  a.out_bstride = int64_t(R) * C;
  if (trans) {
    a.out_ld = R;
    a.sc_ld = C;
    a.sc_bstride = int64_t(R / 128) * C;
  } else {
    a.out_ld = C;
    a.sc_ld = R;
    a.sc_bstride = int64_t(C / 128) * R;
  }
  a.sc = sc;
  return launch_quant_weights(trans, mx, a, d.E * (R / 128) * (C / 128), name, s);
}

template <bool MX, int EPI>
int run_f8_grouped(const moe_desc& d, const Layout& L, F8Args a, int N, const char* name,
                   char* scratch, hipStream_t s) {
  a.offsets = reinterpret_cast<const int32_t*>(scratch + L.offsets);
  a.tstart = reinterpret_cast<const int32_t*>(scratch + L.tiles[2]);  // 256-row m-tiles
  a.E = d.E;
  using TL = F8GrTile<MX>;
  a.ntn = N / TL::BN;
  a.N = N;
  a.nmajor = EPI == EPI_STORE;  // tile order within an expert, as the bf16 grouped GEMM
  const long long Nr = (long long)d.T * d.K;
  const long long grid = ((Nr + (long long)d.E * 255) / 256) * a.ntn;
  int resident;
  if (int rc = resident_grid<f8_grouped_kernel<TL, MX, EPI>>(TL::THREADS, &resident)) return rc;
  prof_begin(name, s);
  f8_grouped_kernel<TL, MX, EPI><<<unsigned(grid < resident ? grid : resident), TL::THREADS, 0, s>>>(a);
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

template <bool MX>
int run_f8_wgrad(const moe_desc& d, const Layout& L, F8Args a, const char* name, char* scratch,
                 hipStream_t s) {
  a.offsets = reinterpret_cast<const int32_t*>(scratch + L.offsets);
  a.tstart = reinterpret_cast<const int32_t*>(scratch + L.tiles[1]);  // 128-token steps
  a.eorder = reinterpret_cast<const int32_t*>(scratch + L.eorder);
  a.E = d.E;
  using TL = F8WgTile<MX>;
  a.tm = a.M / TL::BM;
  a.tn = a.N / TL::BN;
  const long long grid = (long long)d.E * a.tm * a.tn;
  prof_begin(name, s);
  f8_wgrad_kernel<TL, MX, false><<<unsigned(grid), TL::THREADS, 0, s>>>(a);
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// The token-grouped GEMM a (operands set) and the weight gradient b (operands
// set) in one paired launch.
template <bool MX, int EPI>
int run_f8_pair(const moe_desc& d, const Layout& L, F8Args a, int N, F8Args b, int* ctr,
                const char* name, char* scratch, hipStream_t s) {
  using TA = F8GrTile<MX>;
  using TB = F8WgTile<MX>;
  a.offsets = reinterpret_cast<const int32_t*>(scratch + L.offsets);
  a.tstart = reinterpret_cast<const int32_t*>(scratch + L.tiles[2]);  // 256-row m-tiles
  a.E = d.E;
  a.ntn = N / TA::BN;
  a.N = N;
  a.nmajor = EPI == EPI_STORE;
  b.offsets = a.offsets;
  b.tstart = reinterpret_cast<const int32_t*>(scratch + L.tiles[1]);  // 128-token steps
  b.eorder = reinterpret_cast<const int32_t*>(scratch + L.eorder);
  b.E = d.E;
  b.tm = b.M / TB::BM;
  b.tn = b.N / TB::BN;
  PairSched ps{};
  ps.offsets = a.offsets;
  ps.tstart = a.tstart;
  ps.eorder = b.eorder;
  ps.E = d.E;
  ps.ntn = a.ntn;
  ps.per_b = b.tm * b.tn;
  ps.cost_a = a.K;
  ps.ctr = ctr;
  int resident;
  if (int rc = resident_grid<f8_pair_kernel<TA, MX, EPI, TB>>(TA::THREADS, &resident)) return rc;
  prof_begin(name, s);
  f8_pair_kernel<TA, MX, EPI, TB><<<unsigned(resident), TA::THREADS, 0, s>>>(a, b, ps);
  prof_end(s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// Regions of the prepared-weight buffer.
struct WLayout {
  size_t w1f, w1f_sc, w2f, w2f_sc, w2t, w2t_sc, w1t, w1t_sc, total;
};

WLayout wlayout(const moe_desc& d) {
  WLayout W{};
  const size_t E = d.E, D = d.D, F = d.F;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
  const bool fwd = d.mode == MOE_MXFP8 || d.mode == MOE_FP8;
  if (fwd) {
    W.w1f = take(E * 2 * F * D);
    W.w1f_sc = take(E * (D / 128) * 2 * F * 4);
    W.w2f = take(E * D * F);
    W.w2f_sc = take(E * (F / 128) * D * 4);
  }
  W.w2t = take(E * F * D);
  W.w2t_sc = take(E * (D / 128) * F * 4);
  W.w1t = take(E * D * 2 * F);
  W.w1t_sc = take(E * (2 * F / 128) * D * 4);
  W.total = o;
  return W;
}

inline bool fp8_fwd(int mode) { return mode == MOE_MXFP8 || mode == MOE_FP8; }

}  // namespace

bool fp8_mode(int mode) { return mode == MOE_FP8_BWD || mode == MOE_MXFP8 || mode == MOE_FP8; }

size_t fp8_wprep_bytes(const moe_desc& d) { return fp8_mode(d.mode) ? wlayout(d).total : 0; }

// Regions of the FP8 operands in scratch (after the bf16 layout), as offsets
// from its FP8 region: the row codes of one activation, and three (paired
// backward: four) buffers of token codes:
//   qt1  A's row codes in the forward (from the pass over A), then
//        dYw's row codes, dYw's token codes (one-GEMM-per-launch backward),
//        dH's token codes;
//   qt2  x's token codes: written by the forward in MXFP8 and FP8 (gathered
//        from x), by the backward in fp8_bwd (from the dispatched rows);
//   qta  A's token codes (written by the forward in MXFP8 and FP8, beside A's
//        row codes, else by the backward): their own buffer when the forward
//        fills qt2 (F columns), else qt2 itself, which the W2 weight gradient
//        has read before x's token codes replace them;
//   qt3  dYw's token codes when the W2 dgrad still reads dYw's row codes in
//        qt1: in the paired backward (same launch), and in MXFP8, where one
//        pass writes both before the W2 dgrad.
struct F8Offsets {
  size_t qrow, qrow_sc, qt1, qt1_sc, qt2, qt2_sc, qta, qta_sc, qt3, qt3_sc, total;
  size_t qrow_sc_bytes, qt_sc_bytes, qta_sc_bytes;
  bool own_qta, has_qt3;
};

static F8Offsets f8offsets(const moe_desc& d) {
  F8Offsets f{};
  const size_t N = size_t(d.T) * d.K, C = d.D > 2 * d.F ? d.D : 2 * d.F;
  const size_t npad = size_t(max_steps128(d)) * 128;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
  f.qrow_sc_bytes = (C / 128) * N * 4;
  f.qt_sc_bytes = (npad / 128) * C * 4;
  f.qrow = take(N * C);
  f.qrow_sc = take(f.qrow_sc_bytes);
  f.qt1 = take(C * npad);
  f.qt1_sc = take(f.qt_sc_bytes);
  f.qt2 = take(C * npad);
  f.qt2_sc = take(f.qt_sc_bytes);
  f.own_qta = fp8_fwd(d.mode);
  if (f.own_qta) {
    f.qta_sc_bytes = (npad / 128) * size_t(d.F) * 4;
    f.qta = take(size_t(d.F) * npad);
    f.qta_sc = take(f.qta_sc_bytes);
  } else {
    f.qta_sc_bytes = f.qt_sc_bytes;
    f.qta = f.qt2;
    f.qta_sc = f.qt2_sc;
  }
  f.has_qt3 = pair_capable(d) || d.mode == MOE_MXFP8;
  if (f.has_qt3) {
    f.qt3 = take(C * npad);
    f.qt3_sc = take(f.qt_sc_bytes);
  }
  f.total = o;
  return f;
}

size_t fp8_scratch_bytes(const moe_desc& d) {
  if (!fp8_mode(d.mode)) return 0;
  return f8offsets(d).total;
}

int fp8_prepare_weights(const moe_desc& d, const uint16_t* w1, const uint16_t* w2, char* wprep,
                        hipStream_t s) {
  const WLayout W = wlayout(d);
  const bool mx = d.mode == MOE_MXFP8;
  const int D = d.D, F = d.F;
  int rc;
  if (fp8_fwd(d.mode)) {
    if ((rc = quant_weights(d, w1, 2 * F, D, false, mx, reinterpret_cast<uint8_t*>(wprep + W.w1f),
                            reinterpret_cast<uint32_t*>(wprep + W.w1f_sc), "quant_w1", s)))
      return rc;
    if ((rc = quant_weights(d, w2, D, F, false, mx, reinterpret_cast<uint8_t*>(wprep + W.w2f),
                            reinterpret_cast<uint32_t*>(wprep + W.w2f_sc), "quant_w2", s)))
      return rc;
  }
  if ((rc = quant_weights(d, w2, D, F, true, mx, reinterpret_cast<uint8_t*>(wprep + W.w2t),
                          reinterpret_cast<uint32_t*>(wprep + W.w2t_sc), "quant_w2_t", s)))
    return rc;
  return quant_weights(d, w1, 2 * F, D, true, mx, reinterpret_cast<uint8_t*>(wprep + W.w1t),
                       reinterpret_cast<uint32_t*>(wprep + W.w1t_sc), "quant_w1_t", s);
}

// Pointers to the FP8 regions of one scratch buffer.
struct F8Scratch {
  uint8_t *qrow, *qt1, *qt2, *qta, *qt3;
  uint32_t *qrow_sc, *qt1_sc, *qt2_sc, *qta_sc, *qt3_sc;
  size_t qrow_sc_bytes, qt_sc_bytes, qta_sc_bytes;
};

static F8Scratch f8scratch(const moe_desc& d, const Layout& L, char* scratch) {
  const F8Offsets o = f8offsets(d);
  char* b = scratch + L.fp8;
  auto u8 = [&](size_t off) { return reinterpret_cast<uint8_t*>(b + off); };
  auto u32 = [&](size_t off) { return reinterpret_cast<uint32_t*>(b + off); };
  F8Scratch f{};
  f.qrow = u8(o.qrow);
  f.qrow_sc = u32(o.qrow_sc);
  f.qt1 = u8(o.qt1);
  f.qt1_sc = u32(o.qt1_sc);
  f.qt2 = u8(o.qt2);
  f.qt2_sc = u32(o.qt2_sc);
  f.qta = u8(o.qta);
  f.qta_sc = u32(o.qta_sc);
  if (o.has_qt3) {
    f.qt3 = u8(o.qt3);
    f.qt3_sc = u32(o.qt3_sc);
  }
  f.qrow_sc_bytes = o.qrow_sc_bytes;
  f.qt_sc_bytes = o.qt_sc_bytes;
  f.qta_sc_bytes = o.qta_sc_bytes;
  return f;
}

int fp8_view(const moe_desc& d, const Layout& L, char* scratch, int which, void** ptr,
             size_t* bytes) {
  const F8Scratch f = f8scratch(d, L, scratch);
  const size_t N = size_t(d.T) * d.K, C = d.D > 2 * d.F ? d.D : 2 * d.F;
  const size_t npad = size_t(max_steps128(d)) * 128;
  switch (which) {
    case MOE_VIEW_Q_ROWS: *ptr = f.qrow; *bytes = N * C; return MOE_OK;
    case MOE_VIEW_Q_ROWS_SCALE: *ptr = f.qrow_sc; *bytes = f.qrow_sc_bytes; return MOE_OK;
    case MOE_VIEW_Q_TOK_A: *ptr = f.qt1; *bytes = C * npad; return MOE_OK;
    case MOE_VIEW_Q_TOK_A_SCALE: *ptr = f.qt1_sc; *bytes = f.qt_sc_bytes; return MOE_OK;
    case MOE_VIEW_Q_TOK_B: *ptr = f.qt2; *bytes = C * npad; return MOE_OK;
    case MOE_VIEW_Q_TOK_B_SCALE: *ptr = f.qt2_sc; *bytes = f.qt_sc_bytes; return MOE_OK;
    default: return MOE_EINVAL;
  }
}

// Expert linear 1 + SwiGLU on the quantised x rows: stores H into `h` and A
// into `act` (either may be null, as in the bf16 path).  A's codes come from a
// pass over the stored A (fp8_fwd_gemms): the epilogue runs while the matrix
// cores idle, so quantising there costs more than that pass (30B MXFP8: the
// epilogue 36 us slower, against a pass that also writes A's token codes).
static int fp8_w1_swiglu(const moe_desc& d, const Layout& L, const char* wprep, uint16_t* h,
                         uint16_t* act, const char* name, char* scratch, hipStream_t s,
                         bool x_quantised = false) {
  const WLayout W = wlayout(d);
  const F8Scratch f = f8scratch(d, L, scratch);
  const bool mx = d.mode == MOE_MXFP8;
  const int D = d.D, F = d.F, N = d.T * d.K;
  int rc;
  if (!x_quantised &&
      (rc = quant_rows(d, reinterpret_cast<const uint16_t*>(scratch + L.xperm), D, mx, f.qrow,
                       f.qrow_sc, "quant_x_rows", s)))
    return rc;
  F8Args a{};
  a.K = D;
  a.A = f.qrow;
  a.SA = f.qrow_sc;
  a.sa_ld = N;
  a.sa_bytes = uint32_t(f.qrow_sc_bytes);
  a.B = reinterpret_cast<const uint8_t*>(wprep + W.w1f);
  a.b_bstride = int64_t(2) * F * D;
  a.SB = reinterpret_cast<const uint32_t*>(wprep + W.w1f_sc);
  a.sb_ld = 2 * F;
  a.sb_bstride = int64_t(D / 128) * 2 * F;
  a.sb_bytes = uint32_t(size_t(D / 128) * 2 * F * 4);
  a.F = F;
  a.epi = EpiArgs{h, 0, act, nullptr, F};
  return mx ? run_f8_grouped<true, EPI_SWIGLU>(d, L, a, 2 * F, name, scratch, s)
            : run_f8_grouped<false, EPI_SWIGLU>(d, L, a, 2 * F, name, scratch, s);
}

int fp8_recompute_h(const moe_desc& d, const Layout& L, const char* wprep, char* scratch,
                    hipStream_t s) {
  return fp8_w1_swiglu(d, L, wprep, reinterpret_cast<uint16_t*>(scratch + L.h), nullptr,
                       "gemm_w1_recompute", scratch, s);
}

int fp8_fwd_gemms(const moe_desc& d, const Layout& L, const char* wprep, char* scratch,
                  hipStream_t s, bool x_quantised) {
  const WLayout W = wlayout(d);
  const F8Scratch f = f8scratch(d, L, scratch);
  const bool mx = d.mode == MOE_MXFP8;
  const int D = d.D, F = d.F, N = d.T * d.K;
  int rc = fp8_w1_swiglu(d, L, wprep,
                         L.recompute ? nullptr : reinterpret_cast<uint16_t*>(scratch + L.h),
                         reinterpret_cast<uint16_t*>(scratch + L.a), "gemm_w1_swiglu", scratch, s,
                         x_quantised);
  if (rc) return rc;
  // expert linear 2, on A's row codes: one pass over A writes them and A's
  // token codes for the W2 weight gradient (into their own buffer, which the
  // backward leaves alone)
  if ((rc = quant_tokens(d, L, reinterpret_cast<const uint16_t*>(scratch + L.a), F, mx, f.qta,
                         f.qta_sc, "quant_a", scratch, s, TOK_PERM, nullptr, f.qt1, f.qt1_sc)))
    return rc;
  F8Args b{};
  b.K = F;
  b.A = f.qt1;
  b.SA = f.qt1_sc;
  b.sa_ld = N;
  b.sa_bytes = uint32_t(size_t(F / 128) * N * 4);
  b.B = reinterpret_cast<const uint8_t*>(wprep + W.w2f);
  b.b_bstride = int64_t(D) * F;
  b.SB = reinterpret_cast<const uint32_t*>(wprep + W.w2f_sc);
  b.sb_ld = D;
  b.sb_bstride = int64_t(F / 128) * D;
  b.sb_bytes = uint32_t(size_t(F / 128) * D * 4);
  b.F = F;
  b.epi = EpiArgs{reinterpret_cast<uint16_t*>(scratch + L.o), D, nullptr, nullptr, F};
  return mx ? run_f8_grouped<true, EPI_STORE>(d, L, b, D, "gemm_w2", scratch, s)
            : run_f8_grouped<false, EPI_STORE>(d, L, b, D, "gemm_w2", scratch, s);
}

void fp8_row_codes(const moe_desc& d, const Layout& L, char* scratch, uint8_t** codes,
                   uint32_t** scales) {
  const F8Scratch f = f8scratch(d, L, scratch);
  *codes = f.qrow;
  *scales = f.qrow_sc;
}

// dYw's row codes live in the first token-code buffer: the W2 dgrad reads them
// before the W2 weight gradient quantises dYw over tokens into that buffer.
void fp8_dyw_codes(const moe_desc& d, const Layout& L, char* scratch, uint8_t** codes,
                   uint32_t** scales) {
  const F8Scratch f = f8scratch(d, L, scratch);
  *codes = f.qt1;
  *scales = f.qt1_sc;
}

int fp8_x_tokens(const moe_desc& d, const Layout& L, const void* x, bool rows, char* scratch,
                 hipStream_t s) {
  const F8Scratch f = f8scratch(d, L, scratch);
  return quant_tokens(d, L, static_cast<const uint16_t*>(x), d.D, d.mode == MOE_MXFP8, f.qt2,
                      f.qt2_sc, rows ? "quant_x" : "quant_x_tokens", scratch, s, TOK_GATHER,
                      nullptr, rows ? f.qrow : nullptr, rows ? f.qrow_sc : nullptr);
}

int fp8_bwd_gemms(const moe_desc& d, const Layout& L, const char* wprep, const void* dy,
                  const float* topk_w, void* dw1, void* dw2, char* scratch, hipStream_t s) {
  const WLayout W = wlayout(d);
  const F8Scratch f = f8scratch(d, L, scratch);
  const bool mx = d.mode == MOE_MXFP8;
  const bool paired = pair_capable(d);
  // MXFP8 and FP8: the forward already wrote x's token codes (fp8_x_tokens);
  // FP8 also A's (beside A's row codes)
  const bool x_tokens = !fp8_fwd(d.mode);
  const bool a_tokens = !fp8_fwd(d.mode);
  const int D = d.D, F = d.F, N = d.T * d.K;
  const int64_t npad = int64_t(max_steps128(d)) * 128;
  const auto* dyg = static_cast<const uint16_t*>(dy);
  const auto* act = reinterpret_cast<const uint16_t*>(scratch + L.a);
  const auto* dh = reinterpret_cast<const uint16_t*>(scratch + L.dh);
  const auto* xp = reinterpret_cast<const uint16_t*>(scratch + L.xperm);
  int rc;
  // W2 dgrad + SwiGLU-backward on dYw's row codes, in the first token-code
  // buffer (written by the combine-backward, or in MXFP8 by the pass below
  // that also writes dYw's token codes).  dH's row codes for the W1 dgrad
  // come from the pass that quantises the stored dH over tokens: quantising in
  // the epilogue, which runs while the matrix cores idle, cost more (blockwise
  // 0.16 ms at the 30B shape and 0.33 ms at 235B; MXFP8 62 us against the
  // pass's 40 us more)
  uint8_t* dh_rows = f.qrow;
  uint32_t* dh_rows_sc = f.qrow_sc;
  F8Args a{};
  a.K = D;
  a.A = f.qt1;
  a.SA = f.qt1_sc;
  a.sa_ld = N;
  a.sa_bytes = uint32_t(size_t(D / 128) * N * 4);
  a.B = reinterpret_cast<const uint8_t*>(wprep + W.w2t);
  a.b_bstride = int64_t(F) * D;
  a.SB = reinterpret_cast<const uint32_t*>(wprep + W.w2t_sc);
  a.sb_ld = F;
  a.sb_bstride = int64_t(D / 128) * F;
  a.sb_bytes = uint32_t(size_t(D / 128) * F * 4);
  a.F = F;
  a.epi = EpiArgs{reinterpret_cast<uint16_t*>(scratch + L.dh), 0, nullptr,
                  reinterpret_cast<const uint16_t*>(scratch + L.h), F};
  // W2 wgrad over tokens: dYw's token codes (in the first buffer once the W2
  // dgrad is done with the row codes there; in the third when both run in one
  // launch) and A's.  dYw's are gathered from dy (the combine-backward stores
  // no bf16 dYw rows in the FP8 modes).
  uint8_t* dyt = paired || mx ? f.qt3 : f.qt1;
  uint32_t* dyt_sc = paired || mx ? f.qt3_sc : f.qt1_sc;
  F8Args w{};
  w.M = D;
  w.N = F;
  w.A = dyt;
  w.lda = npad;
  w.SA = dyt_sc;
  w.sa_ld = D;
  w.sa_bytes = uint32_t(f.qt_sc_bytes);
  w.B = f.qta;
  w.ldb = npad;
  w.SB = f.qta_sc;
  w.sb_ld = F;
  w.sb_bytes = uint32_t(f.qta_sc_bytes);
  w.C = dw2;
  // W1 wgrad over tokens: dH's token codes (first buffer) and x_perm's (second)
  F8Args v{};
  v.M = 2 * F;
  v.N = D;
  v.A = f.qt1;
  v.lda = npad;
  v.SA = f.qt1_sc;
  v.sa_ld = 2 * F;
  v.sa_bytes = uint32_t(f.qt_sc_bytes);
  v.B = f.qt2;
  v.ldb = npad;
  v.SB = f.qt2_sc;
  v.sb_ld = D;
  v.sb_bytes = uint32_t(f.qt_sc_bytes);
  v.C = dw1;
  // W1 dgrad on dH's row codes
  F8Args b{};
  b.K = 2 * F;
  b.A = f.qrow;
  b.SA = f.qrow_sc;
  b.sa_ld = N;
  b.sa_bytes = uint32_t(size_t(2 * F / 128) * N * 4);
  b.B = reinterpret_cast<const uint8_t*>(wprep + W.w1t);
  b.b_bstride = int64_t(D) * 2 * F;
  b.SB = reinterpret_cast<const uint32_t*>(wprep + W.w1t_sc);
  b.sb_ld = D;
  b.sb_bstride = int64_t(2 * F / 128) * D;
  b.sb_bytes = uint32_t(size_t(2 * F / 128) * D * 4);
  b.F = F;
  b.epi = EpiArgs{reinterpret_cast<uint16_t*>(scratch + L.dxperm), D, nullptr, nullptr, F};

  // MXFP8: one pass gathered from dy and the routing weights writes dYw's row
  // codes (the W2 dgrad's operand, in the first buffer) and its token codes
  // (the W2 weight gradient's, in the third); the combine-backward computed
  // only dtopk_w
  if (mx && (rc = quant_tokens(d, L, dyg, D, true, f.qt3, f.qt3_sc, "quant_dyw", scratch, s,
                               TOK_GATHER_W, topk_w, f.qt1, f.qt1_sc)))
    return rc;
  if (paired) {  // each dgrad beside its weight gradient, one launch per pair
    int* ctr = reinterpret_cast<int*>(scratch + L.pair);
    if ((rc = launch_zero(ctr, 2 * kPairQueues * sizeof(int), s))) return rc;
    if (!mx && (rc = quant_tokens(d, L, dyg, D, mx, f.qt3, f.qt3_sc, "quant_dyw_tokens", scratch, s,
                                  TOK_GATHER_W, topk_w)))
      return rc;
    if (a_tokens &&
        (rc = quant_tokens(d, L, act, F, mx, f.qta, f.qta_sc, "quant_a_tokens", scratch, s)))
      return rc;
    rc = mx ? run_f8_pair<true, EPI_DSWIGLU>(d, L, a, F, w, ctr, "pair_w2", scratch, s)
            : run_f8_pair<false, EPI_DSWIGLU>(d, L, a, F, w, ctr, "pair_w2", scratch, s);
    if (rc) return rc;
    if ((rc = quant_tokens(d, L, dh, 2 * F, mx, f.qt1, f.qt1_sc, "quant_dh_tokens", scratch, s,
                           TOK_PERM, nullptr, dh_rows, dh_rows_sc)))
      return rc;
    if (x_tokens &&
        (rc = quant_tokens(d, L, xp, D, mx, f.qt2, f.qt2_sc, "quant_x_tokens", scratch, s)))
      return rc;
    return mx ? run_f8_pair<true, EPI_STORE>(d, L, b, D, v, ctr + kPairQueues, "pair_w1", scratch, s)
              : run_f8_pair<false, EPI_STORE>(d, L, b, D, v, ctr + kPairQueues, "pair_w1", scratch, s);
  }

  rc = mx ? run_f8_grouped<true, EPI_DSWIGLU>(d, L, a, F, "gemm_w2_dgrad_dswiglu", scratch, s)
          : run_f8_grouped<false, EPI_DSWIGLU>(d, L, a, F, "gemm_w2_dgrad_dswiglu", scratch, s);
  if (rc) return rc;
  if (!mx && (rc = quant_tokens(d, L, dyg, D, mx, f.qt1, f.qt1_sc, "quant_dyw_tokens", scratch, s,
                                TOK_GATHER_W, topk_w)))
    return rc;
  if (a_tokens &&
      (rc = quant_tokens(d, L, act, F, mx, f.qta, f.qta_sc, "quant_a_tokens", scratch, s)))
    return rc;
  rc = mx ? run_f8_wgrad<true>(d, L, w, "gemm_w2_wgrad", scratch, s)
          : run_f8_wgrad<false>(d, L, w, "gemm_w2_wgrad", scratch, s);
  if (rc) return rc;
  // W1 wgrad, then W1 dgrad: the wgrad's dH token pass also writes the row
  // codes the dgrad reads, and the un-permute then reads dX_perm right after
  // it is written.
  auto w1_wgrad = [&]() -> int {
    if ((rc = quant_tokens(d, L, dh, 2 * F, mx, f.qt1, f.qt1_sc, "quant_dh_tokens", scratch, s,
                           TOK_PERM, nullptr, dh_rows, dh_rows_sc)))
      return rc;
    if (x_tokens &&
        (rc = quant_tokens(d, L, xp, D, mx, f.qt2, f.qt2_sc, "quant_x_tokens", scratch, s)))
      return rc;
    return mx ? run_f8_wgrad<true>(d, L, v, "gemm_w1_wgrad", scratch, s)
              : run_f8_wgrad<false>(d, L, v, "gemm_w1_wgrad", scratch, s);
  };
  auto w1_dgrad = [&]() -> int {
    return mx ? run_f8_grouped<true, EPI_STORE>(d, L, b, D, "gemm_w1_dgrad", scratch, s)
              : run_f8_grouped<false, EPI_STORE>(d, L, b, D, "gemm_w1_dgrad", scratch, s);
  };
  if ((rc = w1_wgrad())) return rc;
  return w1_dgrad();
}

}  // namespace moe
