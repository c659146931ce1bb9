// Stand-ins for the HIP runtime calls and the kernel launchers that the C ABI
// layer (ecc_api.cpp) reaches, so that the layer can be built and run on the
// CPU under AddressSanitizer / UndefinedBehaviorSanitizer with no GPU.  Each
// launcher records the arguments it was given for the contract checks.

#include <hip/hip_runtime_api.h>

#include "ecc_internal.hpp"

namespace stub {
ecc::HardArgs hard{};
ecc::SoftArgs soft{};
ecc::GradArgs grad{};
ecc::HeightArgs height{};
int hard_calls = 0, soft_calls = 0, grad_calls = 0, height_calls = 0, height_bwd_calls = 0, static_calls = 0;
hipError_t next_error = hipSuccess;  // returned once by the next launcher
extern void* const kStaticWs = reinterpret_cast<void*>(0x5000);

hipError_t take() {
  const hipError_t e = next_error;
  next_error = hipSuccess;
  return e;
}
}  // namespace stub

hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
  *value = 256;
  return hipSuccess;
}

const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stubbed HIP error"; }

namespace ecc {
hipError_t launch_hard(const HardArgs& a, hipStream_t) {
  stub::hard = a;
  ++stub::hard_calls;
  return stub::take();
}
hipError_t launch_soft(const SoftArgs& a, hipStream_t) {
  stub::soft = a;
  ++stub::soft_calls;
  return stub::take();
}
hipError_t launch_soft_grad(const GradArgs& a, hipStream_t) {
  stub::grad = a;
  ++stub::grad_calls;
  return stub::take();
}
hipError_t launch_height(const HeightArgs& a, hipStream_t) {
  stub::height = a;
  ++stub::height_calls;
  return stub::take();
}
hipError_t launch_height_bwd(const HeightArgs& a, hipStream_t) {
  stub::height = a;
  ++stub::height_bwd_calls;
  return stub::take();
}
hipError_t static_workspace(hipStream_t, void** p) {
  ++stub::static_calls;
  *p = stub::kStaticWs;
  return hipSuccess;
}
}  // namespace ecc
