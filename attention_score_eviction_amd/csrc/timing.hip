// Optional per-kernel timing for benchmarks (kvsel_timing_start /
// kvsel_timing_read).  While a kernel-name prefix is set, every launch of a
// matching kernel carries a start and a stop event that its dispatch stamps
// with the kernel's begin and end (hipExtLaunchKernelGGL); reading waits for
// the pairs and sums their durations per kernel name.  This is the only process-wide mutable state of the library
// and is off unless a caller turns it on.
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace kvsel {
namespace {

struct Pending {
  std::string name;
  hipEvent_t a, b;
};

std::mutex g_mu;
std::string g_prefix;            // "" = off, "*" = every kernel
bool g_on = false;               // read without the lock on the launch path
std::vector<Pending> g_pending;

}  // namespace

bool timing_wanted(const char* kernel_name) {
  if (!__atomic_load_n(&g_on, __ATOMIC_ACQUIRE)) return false;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_prefix.empty()) return false;
  if (g_prefix == "*") return true;
  return strncmp(kernel_name, g_prefix.c_str(), g_prefix.size()) == 0;
}

bool timing_events(hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  if (hipEventCreate(start) != hipSuccess) return false;
  if (hipEventCreate(stop) != hipSuccess) {
    (void)hipEventDestroy(*start);
    *start = nullptr;
    return false;
  }
  return true;
}

void timing_record(const char* kernel_name, hipEvent_t start, hipEvent_t stop) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_pending.push_back({kernel_name, start, stop});
}

}  // namespace kvsel

using namespace kvsel;

extern "C" {

kvsel_status kvsel_timing_start(const char* kernel_prefix) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_prefix = kernel_prefix ? kernel_prefix : "";
  __atomic_store_n(&g_on, !g_prefix.empty(), __ATOMIC_RELEASE);
  return KVSEL_OK;
}

int32_t kvsel_timing_read(char* names, int32_t name_bytes, double* total_ms, int32_t* launches,
                          int32_t max_kernels) {
  if (max_kernels < 0 || name_bytes < 0 || (max_kernels > 0 && (!names || !total_ms || !launches)))
    return -1;
  std::vector<Pending> pend;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    pend.swap(g_pending);
  }
  std::vector<std::string> seen;
  std::vector<double> ms;
  std::vector<int32_t> cnt;
  int32_t failed = 0;
  for (Pending& p : pend) {
    float t = 0.f;
    const bool ok = hipEventSynchronize(p.b) == hipSuccess &&
                    hipEventElapsedTime(&t, p.a, p.b) == hipSuccess;
    (void)hipEventDestroy(p.a);
    (void)hipEventDestroy(p.b);
    if (!ok) {
      ++failed;
      continue;
    }
    size_t i = 0;
    while (i < seen.size() && seen[i] != p.name) ++i;
    if (i == seen.size()) {
      seen.push_back(p.name);
      ms.push_back(0.0);
      cnt.push_back(0);
    }
    ms[i] += t;
    cnt[i] += 1;
  }
  if (failed) return -2;
  const int32_t n = (int32_t)seen.size();
  for (int32_t i = 0; i < n && i < max_kernels; ++i) {
    if (name_bytes > 0) {
      char* dst = names + (size_t)i * name_bytes;
      strncpy(dst, seen[i].c_str(), (size_t)name_bytes - 1);
      dst[name_bytes - 1] = '\0';
    }
    total_ms[i] = ms[i];
    launches[i] = cnt[i];
  }
  return n;
}

}  // extern "C"
