// sa_noalloc.hip -- sa_decode_step_noalloc: the decode step of sa_decode_step
// with its workspace in a scratch array the library holds on each GPU, for
// callers that cannot allocate device memory.
//
// The array is a file-scope device variable (kNoAllocScratchBytes, one copy
// per GPU the library runs on, held until the process ends).  Its address on
// a device comes from hipGetSymbolAddress, looked up once per device with that
// device current and kept; host code never passes the variable's name itself
// (a host-side stand-in, not a device address).  Every call first zeroes, on
// its stream, the scratch words the step needs at zero (a fill kernel), so the
// calls may change shapes from one to the next.  Calls on one GPU share the
// array: calls that overlap in time there (other streams, other threads)
// race.
#include <mutex>

#include "sa_internal.h"

namespace sa {
namespace {

constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
constexpr int kNoAllocMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_mu;
void* g_scratch[kNoAllocMaxDevices] = {};

// The scratch array's address on the current device.
hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kNoAllocMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace sa

using namespace sa;

extern "C" sa_status sa_decode_step_noalloc(const void* Q, const void* K, const void* V, int dtype,
                                            int B, int Hq, int Hkv, int N, int D, int block,
                                            float* ksketch, int update_block, int k, float scale,
                                            int32_t* idx, int32_t* count, float* score, void* O,
                                            int out_dtype, float* lse, void* stream) {
  // host-side checks first, against the scratch size; an aligned stand-in
  // address takes the workspace's place (checks never dereference it)
  void* const stand_in = reinterpret_cast<void*>(uintptr_t(256));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  sa_status s = decode_step(Q, K, V, dtype, B, Hq, Hkv, N, D, block, ksketch, update_block, k,
                            scale, idx, count, score, O, out_dtype, lse, stand_in,
                            kNoAllocScratchBytes, st, StepPhase::kCheck);
  if (s == SA_ERR_WORKSPACE)
    return report(s, "sa_decode_step_noalloc: this shape needs more workspace than the 16 MiB "
                     "scratch the library holds per GPU (use sa_decode_step)");
  if (s) return s;
  void* ws = nullptr;
  const hipError_t e = scratch_on_current_device(&ws);
  if (e != hipSuccess) return report(SA_ERR_HIP, hipGetErrorString(e));
  return decode_step(Q, K, V, dtype, B, Hq, Hkv, N, D, block, ksketch, update_block, k, scale,
                     idx, count, score, O, out_dtype, lse, ws, kNoAllocScratchBytes, st,
                     StepPhase::kClearAndLaunch);
}
