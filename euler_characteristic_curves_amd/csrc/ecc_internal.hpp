// Internal declarations shared by the HIP translation units of libecc_mi355.
// Not part of the public ABI (that is include/ecc.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ecc {

constexpr int kBlock = 256;        // threads per workgroup (4 waves of 64)
constexpr int kWavesPerBlock = kBlock / 64;
constexpr int kAccCopies = 8;      // global accumulator copies, picked by blockIdx % kAccCopies

// Bins of the global accumulators: hard uint8 grids histogram their raw byte
// value (256 keys), everything else threshold indices (H keys).
__host__ __device__ inline int acc_bins(int H) { return H > 256 ? H : 256; }

// Workspace: [ticket + padding | kAccCopies x acc_bins(H) int64 accumulators].
// All of it must be zero between calls; the last workgroup of every launch
// leaves it zero.
constexpr size_t kWsHeader = 256;
inline size_t workspace_bytes(int H) {
  return kWsHeader + (size_t)kAccCopies * (size_t)acc_bins(H) * sizeof(long long);
}

struct HardArgs {
  const void* grid;
  int dtype;          // 0 = u8, 1 = f32
  int64_t nz, ny, nx; // nz = 1 for a 2D grid
  const float* tau;
  int H;
  int64_t* out;
  void* ws;
};

struct SoftArgs {
  const float* grid;
  int64_t nz, ny, nx;  // nz = 1 for 2D
  const float* tau;
  int H;
  float lambda;
  const float* grad_out;  // null for the forward pass
  float* out;             // S (forward) or grad_tau (backward)
  void* ws;
};

struct GradArgs {
  const float* grid;
  int64_t nz, ny, nx;  // nz = 1 for 2D
  const float* tau;
  int H;
  float lambda;
  const float* grad_out;
  float* out;  // grad_grid, one value per voxel
};

struct DeviceInfo {
  int cus;
  size_t lds_bytes;
};

// Per-device properties, cached (ecc_api.cpp).
hipError_t device_info(DeviceInfo* info);

hipError_t launch_hard(const HardArgs& a, hipStream_t stream);
hipError_t launch_soft(const SoftArgs& a, hipStream_t stream);
hipError_t launch_soft_grad(const GradArgs& a, hipStream_t stream);

}  // namespace ecc
