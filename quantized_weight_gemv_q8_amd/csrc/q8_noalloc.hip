// q8_noalloc.hip -- the library's own scratch memory for the entry points
// that allocate nothing (for callers that cannot call hipMalloc or hand
// over a workspace: code under graph capture, tight serving loops).
//
// The scratch is one file-scope device array, allocated with the code
// object on every GPU the library runs on and held until the process ends.
// Host code must not pass the array's name to a kernel (on the host it is
// a stand-in, not a device address): its address on each device is taken
// once, with hipGetSymbolAddress while that device is current, and only
// that address is used afterwards. All calls on one GPU share the array,
// so calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "q8_internal.h"

namespace q8 {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_rc[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[device], [device]() {
    g_rc[device] = hipGetSymbolAddress(&g_ptr[device], HIP_SYMBOL(scratch));
  });
  *ptr = g_rc[device] == hipSuccess ? g_ptr[device] : nullptr;
  return g_rc[device];
}

}  // namespace q8
