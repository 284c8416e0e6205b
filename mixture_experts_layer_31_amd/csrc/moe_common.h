// Internal definitions shared by the MI355X MoE layer's host code and kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming (nontemporal) load and store, for data touched once per
// pass: the access keeps it out of the caches' working set.
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_nt(const void* p) {
  const nt_u32x4 v = __builtin_nontemporal_load(static_cast<const nt_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store16_nt(void* p, const uint4& a) {
  const nt_u32x4 v = {a.x, a.y, a.z, a.w};
  __builtin_nontemporal_store(v, static_cast<nt_u32x4*>(p));
}

// Two floats rounded to bf16 (nearest, ties to even) in one packed word, low
// half first: one v_cvt_pk_bf16_f32.  Converting each value on its own took
// two conversions, a shift and an OR per pair.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Bits of the device error word kept in scratch.
enum : uint32_t { kErrIndex = 1u, kErrTimeout = 2u };

// Routing processes the flat pair list in chunks of this many pairs per block.
constexpr int kRouteChunk = 2048;
constexpr int kRouteThreads = 1024;  // 256 measured 9.1 + 16.4 us for count + scatter
                                     // at 30B against 6.4 + 12.2

// Byte offsets of the regions of the caller's scratch buffer.  Every region
// starts on a 256-byte boundary.  The layout depends only on the descriptor.
struct Layout {
  size_t err, counts, offsets, tiles[3], eorder, chunk_cnt, chunk_bad, pos, src, wperm;
  size_t xperm, h, a, o, dyperm, dh, dxperm, dpart, fp8, queue, pair, total;
  bool recompute;   // MOE_FLAG_RECOMPUTE: no H region; H is rebuilt in the dH region
  int nchunks;      // routing chunks
  int act_bytes;    // bytes per intermediate element
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// A bf16 forward (MOE_BF16, MOE_FP8_BWD) at the shapes whose W1 GEMM takes the
// 128-byte-row loop (2F % 256 == 0, D % 64 == 0): the W1 GEMM gathers x's rows
// itself (no dispatch kernel) and writes x_perm for the backward.
inline bool w1_gathers(const moe_desc& d) {
  return (d.mode == MOE_BF16 || d.mode == MOE_FP8_BWD) && (2 * d.F) % 256 == 0 &&
         d.D % 64 == 0;
}
// MOE_BF16 at those shapes: the GEMMs also carry the routing weights.
// - the W1 GEMM's SwiGLU epilogue stores A_w = w * A, so W2 yields O_w = w * O
//   and the combine is an unweighted sum;
// - the backward dispatches dy unscaled, the W2 dgrad's epilogue applies w and
//   writes dProb partials (its accumulators G = dy W2^T against the SwiGLU
//   output recomputed from H), and the W2 weight gradient pairs dy with A_w.
inline bool bf16_wide(const moe_desc& d) { return d.mode == MOE_BF16 && w1_gathers(d); }
// dProb partials per routed row: one per 64 columns of F
inline int dprob_parts(const moe_desc& d) { return d.F / 64; }

// FP8 modes (moe_fp8.hip): extra scratch for quantised operands, prepared
// weight sizes, weight preparation and the quantised GEMM sequences.
bool fp8_mode(int mode);
size_t fp8_scratch_bytes(const moe_desc& d);
size_t queue_scratch_bytes(const moe_desc& d);  // ticket tables and counters of the persistent forward
size_t fp8_wprep_bytes(const moe_desc& d);

inline Layout make_layout(const moe_desc& d) {
  Layout L{};
  const size_t N = size_t(d.T) * d.K, E = d.E, D = d.D, F = d.F;
  L.act_bytes = d.mode == MOE_FP32 ? 4 : 2;
  L.nchunks = int((N + kRouteChunk - 1) / kRouteChunk);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
  L.err = take(256);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  for (int i = 0; i < 3; ++i) L.tiles[i] = take((E + 1) * 4);
  L.eorder = take((E + 1) * 4);  // experts by descending count, then the skew flag
  L.chunk_cnt = take(size_t(L.nchunks) * E * 4);
  L.chunk_bad = take(size_t(L.nchunks) * 4);  // per-chunk flag: an index outside [0, E)
  L.pos = take(N * 4);
  L.src = take(N * 4);
  L.wperm = take(N * 4);
  const size_t ab = L.act_bytes;
  L.xperm = take(N * D * ab);
  L.recompute = (d.flags & MOE_FLAG_RECOMPUTE) != 0;
  L.h = L.recompute ? 0 : take(N * 2 * F * ab);
  L.a = take(N * F * ab);
  L.o = take(N * D * ab);
  L.dyperm = take(N * D * ab);
  L.dh = take(N * 2 * F * ab);
  L.dxperm = take(N * D * ab);
  L.dpart = bf16_wide(d) ? take(N * size_t(dprob_parts(d)) * 4) : 0;
  if (L.recompute) L.h = L.dh;  // written by the backward's recompute, then overwritten by dH
  L.fp8 = take(fp8_scratch_bytes(d));
  L.queue = take(queue_scratch_bytes(d));
  L.pair = take(2 * 8 * 4);  // ticket counters of the paired backward launches
  L.total = o;
  return L;
}

// Tile heights for which the routing step writes per-expert m-tile prefix sums.
constexpr int kTileRows[3] = {64, 128, 256};

// The whole forward (validation, routing, dispatch, GEMMs, combine) into the
// given scratch; moe_fwd and moe_fwd_noalloc (moe_noalloc.hip) call it.
int forward(const moe_desc* d, const void* x, const int32_t* topk_idx, const float* topk_w,
            const void* w1, const void* w2, const void* wprep, void* y, void* scratch,
            size_t scratch_bytes, hipStream_t s);

// ---- launch helpers (host), implemented in moe_api.hip ----
// Every kernel launch goes through these so the opt-in profiler can bracket it.
void prof_begin(const char* name, hipStream_t s);
void prof_end(hipStream_t s);

// ---- kernel launchers (host) ----
// topk_w (optional): also w_perm[pos[p]] = topk_w[p]
int launch_route(const moe_desc& d, const Layout& L, const int32_t* idx, char* scratch,
                 hipStream_t s, const float* topk_w = nullptr);
int launch_clear_err(char* scratch, const Layout& L, hipStream_t s);

// Row gathers/scatters: dispatch (x -> expert-contiguous rows), combine and the
// un-permute reduction.  `in_f32`/`out_f32` select fp32 instead of bf16 I/O.
// With qmode (FP8 forward modes) the dispatch also writes the rows' e4m3
// quantisation along D; store_rows = false then skips the bf16 rows themselves.
int launch_dispatch(const moe_desc& d, const Layout& L, const void* rows, bool in_f32,
                    char* scratch, size_t dst_off, hipStream_t s, int qmode = 0,
                    uint8_t* qcodes = nullptr, uint32_t* qsc = nullptr, bool store_rows = true,
                    const char* name = "dispatch");
// weighted = false: y_t = sum_k O[pos] (the rows already carry their weights)
int launch_combine(const moe_desc& d, const Layout& L, const float* topk_w, void* y,
                   bool out_f32, const char* scratch, hipStream_t s, bool weighted = true);
// dtopk_w[p] = sum of row pos[p]'s dProb partials, in column order (0 for pairs
// without a row); offsets[E] rows hold partials
int launch_dprob_reduce(const moe_desc& d, const Layout& L, float* dtopk_w, const char* scratch,
                        hipStream_t s);
int launch_unpermute(const moe_desc& d, const Layout& L, void* dx, bool out_f32,
                     const char* scratch, hipStream_t s);
// Combine-backward: dYw_perm rows (w * dy, bf16) and dtopk_w = <dy, o>.  With
// qmode 1 (MX) or 2 (blockwise) it also writes the rows' e4m3 quantisation
// along D (codes [N, D], scale entries [D/128][N]); bf16 rows only.
// store_rows = false skips the bf16 dYw rows (with qmode 0: dtopk_w only).
int launch_dispatch_dy(const moe_desc& d, const Layout& L, const void* dy, bool in_f32,
                       const float* topk_w, float* dtopk_w, char* scratch, hipStream_t s,
                       int qmode = 0, uint8_t* qcodes = nullptr, uint32_t* qsc = nullptr,
                       bool store_rows = true);
int launch_zero(void* p, size_t bytes, hipStream_t s);  // bytes % 16 == 0
int launch_convert_bf16(const float* in, uint16_t* out, size_t n, hipStream_t s);
// Router ahead of the layer (moe_router.hip): softmax -> top-K -> renormalise,
// and its backward to the logits.  Requires 1 <= K <= min(E, 64), E <= 512.
int launch_router_fwd(int T, int E, int K, const float* logits, int32_t* topk_idx, float* topk_w,
                      hipStream_t s);
int launch_router_bwd(int T, int E, int K, const int32_t* topk_idx, const float* topk_w,
                      const float* dtopk_w, float* dlogits, hipStream_t s);

// Grouped GEMMs (MFMA).  See moe_gemm.hip.
// fp32 GEMMs of mode MOE_FP32 (moe_f32.hip).
int launch_fwd_gemms_f32(const moe_desc& d, const Layout& L, const float* w1, const float* w2,
                         char* scratch, hipStream_t s);
int launch_bwd_gemms_f32(const moe_desc& d, const Layout& L, const float* w1, const float* w2,
                         float* dw1, float* dw2, char* scratch, hipStream_t s);
// Backward GEMMs in pairs (each dgrad beside its weight gradient in one
// launch, moe_pair.h): when the descriptor and shapes allow it.
bool pair_capable(const moe_desc& d);
// Persistent forward (dispatch + W1 + SwiGLU + W2 in one launch); see moe_queue.hip.
bool queue_capable(const moe_desc& d);
int launch_fwd_queue(const moe_desc& d, const Layout& L, const void* x, bool in_f32,
                     const uint16_t* w1, const uint16_t* w2, char* scratch, hipStream_t s);
// x: the token rows when w1_gathers(d), else null.
int launch_fwd_gemms(const moe_desc& d, const Layout& L, const uint16_t* w1, const uint16_t* w2,
                     char* scratch, hipStream_t s, const uint16_t* x = nullptr);
// MOE_FLAG_RECOMPUTE: the forward's W1 GEMM again, storing only H (into L.h,
// the dH region), with the same kernels and operands as the forward.
int launch_recompute_h(const moe_desc& d, const Layout& L, const uint16_t* w1, char* scratch,
                       hipStream_t s);
int launch_recompute_h_f32(const moe_desc& d, const Layout& L, const float* w1, char* scratch,
                           hipStream_t s);
int fp8_recompute_h(const moe_desc& d, const Layout& L, const char* wprep, char* scratch,
                    hipStream_t s);
int fp8_prepare_weights(const moe_desc& d, const uint16_t* w1, const uint16_t* w2, char* wprep,
                        hipStream_t s);
// x_quantised: the dispatch already wrote x_perm's row quantisation (fp8_row_codes).
int fp8_fwd_gemms(const moe_desc& d, const Layout& L, const char* wprep, char* scratch,
                  hipStream_t s, bool x_quantised = false);
// MXFP8 and FP8 forward: x's token codes for the W1 weight gradient, gathered
// from x; with rows, also x's row codes for the W1 GEMM (what the dispatch
// writes in these modes, which then need no dispatch).
int fp8_x_tokens(const moe_desc& d, const Layout& L, const void* x, bool rows, char* scratch,
                 hipStream_t s);
// The FP8 backward, after the combine-backward wrote dYw's row codes
// (fp8_dyw_codes) and no bf16 dYw rows: dYw's token codes are gathered from dy
// (bf16 [T, D]) and topk_w.
int fp8_bwd_gemms(const moe_desc& d, const Layout& L, const char* wprep, const void* dy,
                  const float* topk_w, void* dw1, void* dw2, char* scratch, hipStream_t s);
// Where the dispatch writes x_perm's row codes, and the combine-backward dYw's.
void fp8_row_codes(const moe_desc& d, const Layout& L, char* scratch, uint8_t** codes,
                   uint32_t** scales);
void fp8_dyw_codes(const moe_desc& d, const Layout& L, char* scratch, uint8_t** codes,
                   uint32_t** scales);
int fp8_view(const moe_desc& d, const Layout& L, char* scratch, int which, void** ptr,
             size_t* bytes);
int launch_bwd_gemms(const moe_desc& d, const Layout& L, const uint16_t* w1, const uint16_t* w2,
                     void* dw1, void* dw2, bool dw_f32, char* scratch, hipStream_t s);

}  // namespace moe
