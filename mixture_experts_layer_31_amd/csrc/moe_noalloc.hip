// moe_fwd_noalloc: the forward of moe_fwd run in scratch memory the library
// owns, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The scratch is a file-scope device array of kNoallocScratchBytes.  Each GPU
// the library runs on holds its own copy from the first call on that device
// until the process ends.  Host code never passes the array's name to a kernel
// (on the host it is only a stand-in for the device symbol): the first call on
// each device resolves the array's device address with hipGetSymbolAddress,
// with that device current, and every call after that passes that address.
// Every call on a GPU shares that GPU's array: calls that overlap on one GPU
// (on different streams, or from different threads) race.  The forward writes
// every scratch word it later reads (the routing step starts its counts and
// the error word afresh), so nothing has to be cleared between calls.
#include <mutex>

#include "moe_common.h"

namespace moe {
namespace {

constexpr size_t kNoallocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char noalloc_scratch[kNoallocScratchBytes];

std::mutex g_noalloc_mu;
void* g_noalloc_ptr[kMaxDevices] = {};

// Device address of this device's copy of the array, resolved once per device.
int noalloc_base(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
  std::lock_guard<std::mutex> lk(g_noalloc_mu);
  if (g_noalloc_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch)) != hipSuccess || p == nullptr)
      return MOE_EHIP;
    g_noalloc_ptr[dev] = p;
  }
  *out = g_noalloc_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" {

int moe_fwd_noalloc(const moe_desc* d, const void* x, const int32_t* topk_idx,
                    const float* topk_w, const void* w1, const void* w2, const void* wprep,
                    void* y, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t need = moe_scratch_bytes(d);
  if (need == 0)  // an invalid or refused descriptor: moe_fwd's validation names the error
    return moe::forward(d, x, topk_idx, topk_w, w1, w2, wprep, y, nullptr, 0, s);
  if (need > moe::kNoallocScratchBytes) return MOE_ESCRATCH;
  void* base = nullptr;
  if (int rc = moe::noalloc_base(&base)) return rc;
  return moe::forward(d, x, topk_idx, topk_w, w1, w2, wprep, y, base, moe::kNoallocScratchBytes, s);
}

}  // extern "C"
