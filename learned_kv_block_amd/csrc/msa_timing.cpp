// msa_timing.cpp — kernel timing hook of the measurement build (libmsa_timed.so):
// records a HIP event pair on the launch stream around the launches of one
// chosen kernel. See include/msa_timing.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "msa_internal.hpp"
#include "msa_timing.h"

namespace {
constexpr int kOff = -2;  // not recording
struct Prof {
  std::mutex mu;
  std::atomic<int> kernel{kOff};  // the kernel recorded, MSA_K_ALL, or kOff
  int max = 0;
  int used = 0;
  std::vector<hipEvent_t> ev;  // 2 per launch
  std::vector<int> id;         // kernel of each launch
} g_prof;

bool wanted(int kernel) {
  const int k = g_prof.kernel.load();
  return k == kernel || (k == MSA_K_ALL && kernel >= 0);
}
}  // namespace

namespace msa {
void prof_before(int kernel, hipStream_t s) {
  if (!wanted(kernel)) return;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!wanted(kernel) || g_prof.used >= g_prof.max) return;
  (void)hipEventRecord(g_prof.ev[2 * g_prof.used], s);
  g_prof.id[g_prof.used] = kernel;
}
void prof_after(int kernel, hipStream_t s) {
  if (!wanted(kernel)) return;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!wanted(kernel) || g_prof.used >= g_prof.max || g_prof.id[g_prof.used] != kernel) return;
  (void)hipEventRecord(g_prof.ev[2 * g_prof.used + 1], s);
  ++g_prof.used;
}
}  // namespace msa

extern "C" {

msa_status msa_prof_begin(int kernel, int max_launches) {
  if ((kernel != MSA_K_ALL && (kernel < 0 || kernel >= MSA_K_COUNT)) || max_launches < 1 ||
      max_launches > 100000)
    return MSA_ERR_SHAPE;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.kernel = kOff;
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.assign(2 * (size_t)max_launches, nullptr);
  g_prof.id.assign((size_t)max_launches, -1);
  // timing-only events: no system-scope fence (cache writeback and invalidate)
  // when a record completes, so the records do not slow the kernels they time
  for (auto& e : g_prof.ev)
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess)
      return MSA_ERR_DEVICE;
  g_prof.max = max_launches;
  g_prof.used = 0;
  g_prof.kernel = kernel;
  return MSA_OK;
}

msa_status msa_prof_end(float* ms, int* launches) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.kernel = kOff;
  if (ms)
    for (int x = 0; x < MSA_K_COUNT; ++x) ms[x] = 0.0f;
  if (launches)
    for (int x = 0; x < MSA_K_COUNT; ++x) launches[x] = 0;
  msa_status st = MSA_OK;
  for (int x = 0; x < g_prof.used; ++x) {
    if (hipEventSynchronize(g_prof.ev[2 * x + 1]) != hipSuccess) { st = MSA_ERR_DEVICE; break; }
    float t = 0.0f;
    if (hipEventElapsedTime(&t, g_prof.ev[2 * x], g_prof.ev[2 * x + 1]) != hipSuccess) {
      st = MSA_ERR_DEVICE;
      break;
    }
    const int k = g_prof.id[x];
    if (ms) ms[k] += t;
    if (launches) ++launches[k];
  }
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.id.clear();
  g_prof.max = g_prof.used = 0;
  return st;
}

}  // extern "C"
