// Fixed device scratch for bpt_layer_fwd_noalloc, the entry point that allocates
// nothing: the layer's workspace is carved from a file-scope device array instead
// of caller memory.
//
// The array's name is a host-side stand-in in host code; the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is ever handed to kernels or copies.
// Every GPU keeps its copy until the process ends. All calls on one GPU share its
// copy, so calls that overlap on one GPU race (the caller serialises them, e.g.
// on one stream).
#include <mutex>

#include "bpt_launch.hpp"

namespace bpt {
namespace {

__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_status[kMaxDevices];

}  // namespace

int noalloc_scratch(void** ptr, char* err, size_t n) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_err(err, n, "hipGetDevice: %s", hipGetErrorString(e));
    return 1;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_err(err, n, "device %s%d is past the scratch table", "", dev);
    return 1;
  }
  // device dev is current here: its copy of the array is the one resolved
  std::call_once(g_once[dev], [dev]() {
    g_status[dev] = hipGetSymbolAddress(&g_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_status[dev] != hipSuccess || !g_ptr[dev]) {
    set_err(err, n, "hipGetSymbolAddress(scratch): %s",
            g_status[dev] != hipSuccess ? hipGetErrorString(g_status[dev]) : "null address");
    return 1;
  }
  *ptr = g_ptr[dev];
  return 0;
}

}  // namespace bpt
