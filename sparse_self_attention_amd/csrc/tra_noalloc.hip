// Plan drift without any device allocation, for callers that cannot allocate
// (code under stream capture, tight serving loops, harnesses that forbid
// hipMalloc).  Same computation as tra_plan_drift, with its scratch (pooled
// keys of k, levels of (q, k), one counter) in a static device array instead
// of the plan's own scratch.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "tra.h"
#include "tra_internal.h"

namespace {

constexpr size_t SCRATCH_BYTES = size_t(32) << 20;  // TRA_DRIFT_NOALLOC_MAX_BYTES in tra.h

// One copy per device, alive until the process ends.
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};  // device address of `scratch`, per device

// Device address of this device's `scratch`, looked up once per device (the
// host-side symbol is only a stand-in and must never reach a kernel).
tra_status scratch_on(int device, unsigned char** out) {
  if (device < 0 || device >= MAX_DEVICES) return tra::report(TRA_ERR_HIP, "device index out of range");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch_ptr[device]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return tra::report(TRA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[device] = ptr;
  }
  *out = static_cast<unsigned char*>(g_scratch_ptr[device]);
  return TRA_OK;
}

}  // namespace

extern "C" {

size_t tra_drift_noalloc_max_bytes(void) { return SCRATCH_BYTES; }

tra_status tra_plan_drift_noalloc(const tra_plan* plan, const void* q, const void* k, int64_t* changed,
                                  void* stream) {
  if (!plan || !changed) return tra::report(TRA_ERR_INVALID_ARG, "plan and changed must not be NULL");
  const size_t need = tra::drift_scratch_bytes(plan);
  if (need > SCRATCH_BYTES)
    return tra::report(TRA_ERR_SHAPE, "tra_plan_drift_noalloc: the plan needs " + std::to_string(need) +
                                          " bytes of scratch; the static buffer holds " +
                                          std::to_string(SCRATCH_BYTES));
  int device = -1;
  const hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return tra::report(TRA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (device != tra::plan_device(plan))
    return tra::report(TRA_ERR_INVALID_ARG, "the current device is not the plan's device");
  unsigned char* base = nullptr;
  const tra_status st = scratch_on(device, &base);
  if (st != TRA_OK) return st;
  // Pooled keys | levels | counter; the drift clears the counter before its
  // kernels run.  Calls that overlap on one device share this memory and race.
  void* kbar = nullptr;
  int16_t* lv = nullptr;
  unsigned long long* counter = nullptr;
  tra::drift_scratch_layout(plan, base, &kbar, &lv, &counter);
  return tra::drift_with_scratch(plan, q, k, kbar, lv, counter, changed, stream);
}

}  // extern "C"
