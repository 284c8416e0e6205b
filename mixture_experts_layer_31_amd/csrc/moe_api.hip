// Host side of the MoE layer's C ABI: argument validation, scratch layout,
// launch sequencing and the opt-in kernel profiler.  The declarations and the
// contract of every entry point are in include/moe.h.
#include <mutex>
#include <string>
#include <vector>

#include "moe_common.h"

namespace moe {
namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Descriptor checks shared by every entry point.
int check_desc(const moe_desc* d) {
  if (d == nullptr) return MOE_EINVAL;
  if (d->T < 0 || d->D <= 0 || d->F <= 0 || d->E <= 0 || d->K <= 0) return MOE_EINVAL;
  if (d->K > d->E || d->E > 1024) return MOE_EINVAL;
  if (d->mode < MOE_FP32 || d->mode > MOE_FP8) return MOE_EINVAL;
  if ((d->flags & ~int32_t(MOE_FLAG_OVERLAP | MOE_FLAG_QUEUE_TIMEOUT_TEST | MOE_FLAG_RECOMPUTE |
                           MOE_FLAG_OVERLAP_BWD | MOE_FLAG_SERIAL_BWD)) != 0)
    return MOE_EINVAL;
  if ((d->flags & MOE_FLAG_OVERLAP_BWD) && (d->flags & MOE_FLAG_SERIAL_BWD)) return MOE_EINVAL;
  const long long N = (long long)d->T * d->K;
  const long long widest = d->D > 2 * d->F ? d->D : 2 * d->F;
  if (N >= (1LL << 31) || N * widest >= (1LL << 46)) return MOE_EINVAL;
  if (d->D % 64 != 0 || d->F % 64 != 0) return MOE_EUNSUPPORTED;
  // The GEMMs address one expert's rows, and one expert's weight matrix,
  // through 32-bit buffer resources with int byte offsets.  An expert can hold
  // every routed pair (ids need not be distinct for the kernels to stay in
  // bounds), so every [N, widest] intermediate and every [2F, D] weight must
  // stay below 2 GiB; larger shapes are refused rather than wrapped.
  const long long eb = d->mode == MOE_FP32 ? 4 : 2;
  if (N * widest * eb >= (1LL << 31) || 2LL * d->F * d->D * eb >= (1LL << 31))
    return MOE_EUNSUPPORTED;
  if (d->mode == MOE_FP8_BWD || d->mode == MOE_MXFP8 || d->mode == MOE_FP8) {
    // token-quantised operands: [widest, npad] codes, read by the weight
    // gradients with 256-row buffer ranges, and [npad / 128, widest] scales
    const long long npad = (N + 127LL * d->E) / 128 * 128;
    if (256 * npad >= (1LL << 31) || npad / 128 * widest * 4 >= (1LL << 31))
      return MOE_EUNSUPPORTED;
  }
  return MOE_OK;
}

// Modes whose kernels exist in this library, and their shape requirements.
int check_built(const moe_desc* d) {
  if (fp8_mode(d->mode) && (d->D % 256 != 0 || d->F % 256 != 0)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

int check_scratch(const moe_desc* d, const void* scratch, size_t bytes) {
  if (scratch == nullptr) return MOE_EINVAL;
  if (!aligned(scratch, 16)) return MOE_EALIGN;
  if (bytes < make_layout(*d).total) return MOE_ESCRATCH;
  return MOE_OK;
}

size_t wprep_size(const moe_desc& d) {
  if (d.mode == MOE_FP32_BF16GEMM)  // bf16 copies of W1 and W2
    return align256(size_t(d.E) * 2 * d.F * d.D * 2) + align256(size_t(d.E) * d.D * d.F * 2);
  return fp8_wprep_bytes(d);  // quantised copies (0 for the bf16 mode)
}

// ---- profiler state (only touched while enabled) ----
struct ProfPending {
  const char* name;
  hipEvent_t a, b;
};
struct ProfTotal {
  std::string name;
  double ms;
  int64_t n;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
const char* g_prof_name = nullptr;
hipEvent_t g_prof_start = nullptr;
std::vector<ProfPending> g_prof_pending;
std::vector<hipEvent_t> g_prof_pool;
std::vector<ProfTotal> g_prof_totals;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Weight pointers the GEMMs read (bf16): the caller's, or the bf16 copies in wprep.
int gemm_weights(const moe_desc& d, const void* w1, const void* w2, const void* wprep,
                 const uint16_t** g1, const uint16_t** g2) {
  if (fp8_mode(d.mode) && wprep == nullptr) return MOE_EINVAL;
  if (d.mode == MOE_FP32_BF16GEMM) {
    if (wprep == nullptr) return MOE_EINVAL;
    const char* base = static_cast<const char*>(wprep);
    *g1 = reinterpret_cast<const uint16_t*>(base);
    *g2 = reinterpret_cast<const uint16_t*>(base + align256(size_t(d.E) * 2 * d.F * d.D * 2));
  } else {
    *g1 = static_cast<const uint16_t*>(w1);
    *g2 = static_cast<const uint16_t*>(w2);
  }
  return MOE_OK;
}

}  // namespace

void prof_begin(const char* name, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) return;
  g_prof_name = name;
  g_prof_start = prof_event();
  if (g_prof_start) (void)hipEventRecord(g_prof_start, s);
}

void prof_end(hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on || g_prof_start == nullptr) return;
  hipEvent_t b = prof_event();
  if (b == nullptr) return;
  (void)hipEventRecord(b, s);
  g_prof_pending.push_back({g_prof_name, g_prof_start, b});
  g_prof_start = nullptr;
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null pointer, bad sizes, bad mode or flags)";
    case MOE_ESCRATCH: return "scratch or wprep buffer smaller than required";
    case MOE_EALIGN: return "buffer not 16-byte aligned";
    case MOE_EUNSUPPORTED: return "mode or shape not supported by this library";
    case MOE_EHIP: return "HIP launch or runtime error";
    case MOE_EINDEX: return "topk_idx entry outside [0, E)";
    case MOE_ETIMEOUT: return "bounded wait in a persistent kernel expired";
    default: return "unknown status";
  }
}

size_t moe_scratch_bytes(const moe_desc* d) {
  if (check_desc(d) != MOE_OK) return 0;
  return make_layout(*d).total;
}

size_t moe_wprep_bytes(const moe_desc* d) {
  if (check_desc(d) != MOE_OK) return 0;
  return wprep_size(*d);
}

int moe_prepare_weights(const moe_desc* d, const void* w1, const void* w2, void* wprep,
                        size_t wprep_bytes, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if ((rc = check_built(d))) return rc;
  const size_t need = wprep_size(*d);
  if (need == 0) return MOE_OK;
  if (w1 == nullptr || w2 == nullptr || wprep == nullptr) return MOE_EINVAL;
  if (!aligned(w1, 16) || !aligned(w2, 16) || !aligned(wprep, 16)) return MOE_EALIGN;
  if (wprep_bytes < need) return MOE_ESCRATCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fp8_mode(d->mode))
    return fp8_prepare_weights(*d, static_cast<const uint16_t*>(w1),
                               static_cast<const uint16_t*>(w2), static_cast<char*>(wprep), s);
  const size_t n1 = size_t(d->E) * 2 * d->F * d->D, n2 = size_t(d->E) * d->D * d->F;
  char* base = static_cast<char*>(wprep);
  rc = launch_convert_bf16(static_cast<const float*>(w1), reinterpret_cast<uint16_t*>(base), n1, s);
  if (rc) return rc;
  return launch_convert_bf16(static_cast<const float*>(w2),
                             reinterpret_cast<uint16_t*>(base + align256(n1 * 2)), n2, s);
}

int moe_route(const moe_desc* d, const int32_t* topk_idx, void* scratch, size_t scratch_bytes,
              void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (topk_idx == nullptr && d->T > 0) return MOE_EINVAL;
  if (!aligned(topk_idx, 4)) return MOE_EALIGN;
  if ((rc = check_scratch(d, scratch, scratch_bytes))) return rc;
  const Layout L = make_layout(*d);
  return launch_route(*d, L, topk_idx, static_cast<char*>(scratch), static_cast<hipStream_t>(stream));
}

int moe_routing_view(const moe_desc* d, const void* scratch, size_t scratch_bytes,
                     int32_t** counts, int32_t** offsets, int32_t** pos, int32_t** src) {
  int rc = check_desc(d);
  if (rc) return rc;
  if ((rc = check_scratch(d, scratch, scratch_bytes))) return rc;
  const Layout L = make_layout(*d);
  char* b = const_cast<char*>(static_cast<const char*>(scratch));
  if (counts) *counts = reinterpret_cast<int32_t*>(b + L.counts);
  if (offsets) *offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  if (pos) *pos = reinterpret_cast<int32_t*>(b + L.pos);
  if (src) *src = reinterpret_cast<int32_t*>(b + L.src);
  return MOE_OK;
}

int moe_scratch_view(const moe_desc* d, const void* scratch, size_t scratch_bytes, int which,
                     void** ptr, size_t* bytes) {
  int rc = check_desc(d);
  if (rc) return rc;
  if ((rc = check_scratch(d, scratch, scratch_bytes))) return rc;
  if (ptr == nullptr) return MOE_EINVAL;
  const Layout L = make_layout(*d);
  const size_t N = size_t(d->T) * d->K, ab = L.act_bytes;
  size_t off, n;
  switch (which) {
    case MOE_VIEW_XPERM: off = L.xperm; n = N * d->D * ab; break;
    case MOE_VIEW_H:
      if (L.recompute) return MOE_EINVAL;  // the forward keeps no H
      off = L.h;
      n = N * 2 * d->F * ab;
      break;
    case MOE_VIEW_A: off = L.a; n = N * d->F * ab; break;
    case MOE_VIEW_O: off = L.o; n = N * d->D * ab; break;
    case MOE_VIEW_DYPERM: off = L.dyperm; n = N * d->D * ab; break;
    case MOE_VIEW_DH: off = L.dh; n = N * 2 * d->F * ab; break;
    case MOE_VIEW_DXPERM: off = L.dxperm; n = N * d->D * ab; break;
    case MOE_VIEW_WPERM: off = L.wperm; n = N * 4; break;
    case MOE_VIEW_QUEUE: off = L.queue; n = queue_scratch_bytes(*d); break;
    default:
      if (!fp8_mode(d->mode) || which < MOE_VIEW_Q_ROWS || which > MOE_VIEW_Q_TOK_B_SCALE)
        return MOE_EINVAL;
      return fp8_view(*d, L, const_cast<char*>(static_cast<const char*>(scratch)), which, ptr,
                      bytes ? bytes : &n);
  }
  *ptr = const_cast<char*>(static_cast<const char*>(scratch)) + off;
  if (bytes) *bytes = n;
  return MOE_OK;
}

int moe_fwd(const moe_desc* d, const void* x, const int32_t* topk_idx, const float* topk_w,
            const void* w1, const void* w2, const void* wprep, void* y, void* scratch,
            size_t scratch_bytes, void* stream) {
  return forward(d, x, topk_idx, topk_w, w1, w2, wprep, y, scratch, scratch_bytes,
                 static_cast<hipStream_t>(stream));
}

}  // extern "C"

// The forward behind moe_fwd and moe_fwd_noalloc (which passes the library's
// own scratch).
int moe::forward(const moe_desc* d, const void* x, const int32_t* topk_idx, const float* topk_w,
                 const void* w1, const void* w2, const void* wprep, void* y, void* scratch,
                 size_t scratch_bytes, hipStream_t s) {
  int rc = check_desc(d);
  if (rc) return rc;
  if ((rc = check_built(d))) return rc;
  // with no tokens the [T, ...] buffers are empty and may be null
  if (!w1 || !w2 || (d->T > 0 && (!x || !topk_idx || !topk_w || !y))) return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(w1, 16) || !aligned(w2, 16) ||
      !aligned(topk_idx, 4) || !aligned(topk_w, 4) || (wprep && !aligned(wprep, 16)))
    return MOE_EALIGN;
  if ((rc = check_scratch(d, scratch, scratch_bytes))) return rc;
  const uint16_t *g1, *g2;
  if ((rc = gemm_weights(*d, w1, w2, wprep, &g1, &g2))) return rc;
  const Layout L = make_layout(*d);
  char* sc = static_cast<char*>(scratch);
  const bool io_f32 = d->mode == MOE_FP32 || d->mode == MOE_FP32_BF16GEMM;
  if ((rc = launch_route(*d, L, topk_idx, sc, s, topk_w))) return rc;
  if (d->T == 0) return MOE_OK;  // routing metadata of no pairs; y is empty
  if (queue_capable(*d)) {
    if ((rc = launch_fwd_queue(*d, L, x, io_f32, g1, g2, sc, s))) return rc;
    return launch_combine(*d, L, topk_w, y, io_f32, sc, s, !bf16_wide(*d));
  }
  const bool fwd_q = fp8_mode(d->mode) && d->mode != MOE_FP8_BWD;
  if (fwd_q) {
    // Nothing stores the dispatched bf16 rows (except under recompute, whose
    // backward quantises them again): x's token codes (the W1 weight gradient's
    // operand) come from a pass gathered from x.  In MXFP8 that pass also writes
    // x's row codes (the W1 GEMM's operand), and no dispatch runs
    // (30B: 0.17 ms against 0.09 + 0.12); blockwise, whose row quotients cost
    // that pass more than the dispatch (0.31 against 0.09 + 0.17 ms), the
    // dispatch writes them.
    const bool mx = d->mode == MOE_MXFP8;
    const bool rows_in_pass = mx && !L.recompute;
    if (!rows_in_pass) {
      uint8_t* qc;
      uint32_t* qs;
      fp8_row_codes(*d, L, sc, &qc, &qs);
      if ((rc = launch_dispatch(*d, L, x, io_f32, sc, L.xperm, s, mx ? 1 : 2, qc, qs,
                                L.recompute)))
        return rc;
    }
    if ((rc = fp8_x_tokens(*d, L, x, rows_in_pass, sc, s))) return rc;
  } else if (!w1_gathers(*d) && (rc = launch_dispatch(*d, L, x, io_f32, sc, L.xperm, s))) {
    return rc;
  }
  if (d->mode == MOE_FP32)
    rc = launch_fwd_gemms_f32(*d, L, static_cast<const float*>(w1), static_cast<const float*>(w2),
                              sc, s);
  else if (fp8_mode(d->mode) && d->mode != MOE_FP8_BWD)
    rc = fp8_fwd_gemms(*d, L, static_cast<const char*>(wprep), sc, s, true);
  else
    rc = launch_fwd_gemms(*d, L, g1, g2, sc, s,
                          w1_gathers(*d) ? static_cast<const uint16_t*>(x) : nullptr);
  if (rc) return rc;
  return launch_combine(*d, L, topk_w, y, io_f32, sc, s, !bf16_wide(*d));
}

extern "C" {

int moe_bwd(const moe_desc* d, const void* dy, const float* topk_w, const void* w1,
            const void* w2, const void* wprep, void* dx, void* dw1, void* dw2, float* dtopk_w,
            void* scratch, size_t scratch_bytes, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if ((rc = check_built(d))) return rc;
  if (!w1 || !w2 || !dw1 || !dw2 || (d->T > 0 && (!dy || !topk_w || !dx || !dtopk_w)))
    return MOE_EINVAL;
  if (!aligned(dy, 16) || !aligned(dx, 16) || !aligned(w1, 16) || !aligned(w2, 16) ||
      !aligned(dw1, 16) || !aligned(dw2, 16) || !aligned(topk_w, 4) || !aligned(dtopk_w, 4) ||
      (wprep && !aligned(wprep, 16)))
    return MOE_EALIGN;
  if ((rc = check_scratch(d, scratch, scratch_bytes))) return rc;
  const uint16_t *g1, *g2;
  if ((rc = gemm_weights(*d, w1, w2, wprep, &g1, &g2))) return rc;
  const Layout L = make_layout(*d);
  char* sc = static_cast<char*>(scratch);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool io_f32 = d->mode == MOE_FP32 || d->mode == MOE_FP32_BF16GEMM;
  if (d->T == 0) {  // no tokens: every expert's weight gradient is zero; dx, dtopk_w are empty
    const size_t es = io_f32 ? 4 : 2, n1 = size_t(d->E) * 2 * d->F * d->D * es;
    if ((rc = launch_zero(dw1, n1, s))) return rc;
    return launch_zero(dw2, n1 / 2, s);
  }
  if (L.recompute) {  // H again, by the forward's own W1 GEMM (before the combine-backward,
                      // whose fused FP8 row codes the FP8 recompute's x codes would overwrite)
    if (d->mode == MOE_FP32)
      rc = launch_recompute_h_f32(*d, L, static_cast<const float*>(w1), sc, s);
    else if (fp8_mode(d->mode) && d->mode != MOE_FP8_BWD)
      rc = fp8_recompute_h(*d, L, static_cast<const char*>(wprep), sc, s);
    else
      rc = launch_recompute_h(*d, L, g1, sc, s);
    if (rc) return rc;
  }
  if (d->mode == MOE_MXFP8) {  // dtopk_w only: the pass gathered from dy writes dYw's codes
    if ((rc = launch_dispatch_dy(*d, L, dy, io_f32, topk_w, dtopk_w, sc, s, 0, nullptr, nullptr,
                                 false)))
      return rc;
  } else if (fp8_mode(d->mode)) {  // the combine-backward quantises dYw's rows for the W2
                                   // dgrad, without storing them in bf16
    uint8_t* qc;
    uint32_t* qs;
    fp8_dyw_codes(*d, L, sc, &qc, &qs);
    if ((rc = launch_dispatch_dy(*d, L, dy, io_f32, topk_w, dtopk_w, sc, s, 2, qc, qs, false)))
      return rc;
  } else if (bf16_wide(*d)) {  // dy unscaled: w and dtopk_w come from the W2 dgrad
    if ((rc = launch_dispatch(*d, L, dy, false, sc, L.dyperm, s, 0, nullptr, nullptr, true,
                              "dispatch_dy")))
      return rc;
  } else if ((rc = launch_dispatch_dy(*d, L, dy, io_f32, topk_w, dtopk_w, sc, s))) {
    return rc;
  }
  if (d->mode == MOE_FP32)
    rc = launch_bwd_gemms_f32(*d, L, static_cast<const float*>(w1), static_cast<const float*>(w2),
                              static_cast<float*>(dw1), static_cast<float*>(dw2), sc, s);
  else if (fp8_mode(d->mode))
    rc = fp8_bwd_gemms(*d, L, static_cast<const char*>(wprep), dy, topk_w, dw1, dw2, sc, s);
  else
    rc = launch_bwd_gemms(*d, L, g1, g2, dw1, dw2, io_f32, sc, s);
  if (rc) return rc;
  if (bf16_wide(*d) && (rc = launch_dprob_reduce(*d, L, dtopk_w, sc, s))) return rc;
  return launch_unpermute(*d, L, dx, io_f32, sc, s);
}

// The router reads only T, E and K of the descriptor.
static int check_router_desc(const moe_desc* d) {
  if (d == nullptr) return MOE_EINVAL;
  if (d->T < 0 || d->E <= 0 || d->K <= 0 || d->K > d->E) return MOE_EINVAL;
  if (d->E > 512 || d->K > 64) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

int moe_router_fwd(const moe_desc* d, const float* logits, int32_t* topk_idx, float* topk_w,
                   void* stream) {
  const int rc = check_router_desc(d);
  if (rc) return rc;
  if (d->T == 0) return MOE_OK;  // no tokens: nothing to route
  if (logits == nullptr || topk_idx == nullptr || topk_w == nullptr) return MOE_EINVAL;
  if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4)) return MOE_EALIGN;
  return launch_router_fwd(d->T, d->E, d->K, logits, topk_idx, topk_w,
                           static_cast<hipStream_t>(stream));
}

int moe_router_bwd(const moe_desc* d, const int32_t* topk_idx, const float* topk_w,
                   const float* dtopk_w, float* dlogits, void* stream) {
  const int rc = check_router_desc(d);
  if (rc) return rc;
  if (d->T == 0) return MOE_OK;
  if (topk_idx == nullptr || topk_w == nullptr || dtopk_w == nullptr || dlogits == nullptr)
    return MOE_EINVAL;
  if (!aligned(topk_idx, 4) || !aligned(topk_w, 4) || !aligned(dtopk_w, 4) || !aligned(dlogits, 4))
    return MOE_EALIGN;
  return launch_router_bwd(d->T, d->E, d->K, topk_idx, topk_w, dtopk_w, dlogits,
                           static_cast<hipStream_t>(stream));
}

int moe_check(const moe_desc* d, void* scratch, size_t scratch_bytes, void* stream) {
  int rc = check_desc(d);
  if (rc) return rc;
  if ((rc = check_scratch(d, scratch, scratch_bytes))) return rc;
  const Layout L = make_layout(*d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t word = 0;
  if (hipStreamSynchronize(s) != hipSuccess) return MOE_EHIP;
  if (hipMemcpy(&word, static_cast<char*>(scratch) + L.err, 4, hipMemcpyDeviceToHost) != hipSuccess)
    return MOE_EHIP;
  if ((rc = launch_clear_err(static_cast<char*>(scratch), L, s))) return rc;
  if (hipStreamSynchronize(s) != hipSuccess) return MOE_EHIP;
  if (word & kErrIndex) return MOE_EINDEX;
  if (word & kErrTimeout) return MOE_ETIMEOUT;
  return MOE_OK;
}

int moe_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return MOE_OK;
}

int moe_profile_collect(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (const ProfPending& p : g_prof_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.b) != hipSuccess) return MOE_EHIP;
    if (hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess) return MOE_EHIP;
    ProfTotal* t = nullptr;
    for (ProfTotal& q : g_prof_totals)
      if (q.name == p.name) t = &q;
    if (t == nullptr) {
      g_prof_totals.push_back({p.name, 0.0, 0});
      t = &g_prof_totals.back();
    }
    t->ms += ms;
    t->n += 1;
    g_prof_pool.push_back(p.a);
    g_prof_pool.push_back(p.b);
  }
  g_prof_pending.clear();
  return int(g_prof_totals.size());
}

int moe_profile_get(int i, const char** name, double* total_ms, int64_t* launches) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (i < 0 || i >= int(g_prof_totals.size())) return MOE_EINVAL;
  if (name) *name = g_prof_totals[i].name.c_str();
  if (total_ms) *total_ms = g_prof_totals[i].ms;
  if (launches) *launches = g_prof_totals[i].n;
  return MOE_OK;
}

int moe_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_totals.clear();
  return MOE_OK;
}

}  // extern "C"
