// The workspace of ecc_hard_3d_static (include/ecc.h): a file-scope device
// array, so that the entry point allocates nothing.  Every GPU the library
// runs on holds its own copy until the process ends.  Host code never uses
// the array's name as an address: the device address on each device comes
// from hipGetSymbolAddress, once per device, and is kept in g_ptr.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "ecc_internal.hpp"

namespace ecc {
namespace {

// the ticket and accumulators of one hard call, any H <= 8192
static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_ptr[kMaxDevices];
std::mutex g_mu;

__global__ void zero_words(unsigned long long* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0ull;
}

}  // namespace

// Device address of this device's array; the first call for a device looks it
// up and clears it with a fill kernel on `stream` (not a memset, so that the
// call can be captured into a graph).  The hard kernels leave it zero.
hipError_t static_workspace(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_mu);
    p = g_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      hipLaunchKernelGGL(zero_words, dim3(64), dim3(256), 0, stream, reinterpret_cast<unsigned long long*>(p),
                         kStaticWorkspaceBytes / sizeof(unsigned long long));
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      g_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace ecc
