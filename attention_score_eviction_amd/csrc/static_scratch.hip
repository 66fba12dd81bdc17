// kvsel_score_static: kvsel_score with its scratch in a file-scope device
// array instead of a caller workspace, for callers that cannot allocate
// device memory (code under graph capture, tight serving loops, harnesses
// that forbid allocation).
//
// The array `scratch` below is a device symbol: in host code its name is a
// host-side stand-in, not a device address.  Its device address is looked up
// once per device, with that device current, by hipGetSymbolAddress on the
// first call on that device, and only that address is ever handed to a
// kernel.  Each device holds its own copy of the array for the life of the
// process.  Every call on one device shares that device's copy, so calls
// that overlap on one device (two streams, two threads) race; calls on one
// stream are ordered and safe.  Nothing in the scratch must start at zero:
// every scratch byte a kernel of the score path reads was written earlier in
// the same call.
#include <mutex>

#include "common.h"

namespace kvsel {
namespace {

constexpr size_t kStaticScratchBytes = KVSEL_STATIC_SCRATCH_BYTES;
static_assert(kStaticScratchBytes % 256 == 0, "scratch size must keep 256-byte alignment");

static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
char* g_ptr[kMaxDevices] = {};   // device address of `scratch` per device, once looked up

// Device address of this device's scratch array (NULL on failure).
char* scratch_ptr(int* err) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = 1;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *err = 1;
      return nullptr;
    }
    g_ptr[dev] = (char*)p;
  }
  return g_ptr[dev];
}

}  // namespace
}  // namespace kvsel

using namespace kvsel;

extern "C" {

kvsel_status kvsel_score_static(const kvsel_desc* desc, const void* q_obs, const void* k,
                                float* raw_scores, float* pooled, int32_t pool_kernel,
                                void* stream) {
  // The argument checks of kvsel_score, with the static scratch as the
  // workspace: a problem needing more than the array holds is refused before
  // any device call.
  const size_t need = kvsel_score_workspace(desc);
  if (need == 0) return kvsel_score(desc, q_obs, k, raw_scores, pooled, pool_kernel, nullptr, 0,
                                    stream);
  if (need > kStaticScratchBytes) return KVSEL_ERR_WORKSPACE;
  int err = 0;
  char* ws = scratch_ptr(&err);
  if (err || !ws) return KVSEL_ERR_DEVICE;
  return kvsel_score(desc, q_obs, k, raw_scores, pooled, pool_kernel, ws, kStaticScratchBytes,
                     stream);
}

}  // extern "C"
