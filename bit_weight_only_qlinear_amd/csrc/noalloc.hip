// Static device scratch for the allocation-free forward entry point
// (qlinear_forward_static): the staged activations of the qGEMM's 224-row
// tiling live in a fixed array of this file instead of a workspace that the
// caller allocates.
//
// Each GPU that loads the library holds its own copy of the array until the
// process ends.  Host code never passes the array's name to a kernel (in
// host code it names a host-side stand-in): the device address is taken
// once per device with hipGetSymbolAddress, with that device current, and
// kept here.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qp_internal.hpp"

namespace qp {
namespace {

constexpr size_t kScratchBytes = size_t(40) << 20;   // 40 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];

}  // namespace

size_t static_scratch_bytes() { return kScratchBytes; }

hipError_t static_scratch(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace qp
