// Internal declarations shared by the HIP translation units of libecc_mi355.
// Not part of the public ABI (that is include/ecc.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ecc {

constexpr int kBlock = 256;        // threads per workgroup (4 waves of 64)
constexpr int kWavesPerBlock = kBlock / 64;
constexpr int kAccCopies = 8;      // global accumulator copies of one grid, picked by blockIdx % copies

// Bins of the global accumulators: hard uint8 grids histogram their raw byte
// value (256 keys), everything else threshold indices (H keys).
__host__ __device__ inline int acc_bins(int H) { return H > 256 ? H : 256; }

// Workspace of one grid: [ticket + padding | copies x acc_bins(H) int64
// accumulators | group tickets], the group tickets (one 128-byte line each,
// see grid_reduce) only in the workspace of a lone grid (copies ==
// kAccCopies).  All of it must be zero between calls; every launch leaves it
// zero.
constexpr size_t kWsHeader = 256;
constexpr int kTicketGroups = 32;
constexpr size_t kTicketLine = 128;
constexpr size_t kGroupTicketBytes = (size_t)kTicketGroups * kTicketLine;
inline size_t workspace_bytes(int H, int copies = kAccCopies) {
  return kWsHeader + (size_t)copies * (size_t)acc_bins(H) * sizeof(long long) +
         (copies == kAccCopies ? kGroupTicketBytes : 0);
}

// Accumulator copies per grid in a batch: the workgroups of a launch are
// shared among the grids, so fewer of them flush into each grid's totals.
inline int batch_copies(int64_t batch) {
  return batch >= kAccCopies ? 1 : (int)(kAccCopies / batch);
}

// A batch of `batch` grids of one shape, stored back to back.  Grid b reads
// tau + b * tau_stride (0: one threshold array for all), writes out + b * H and
// uses the workspace at ws + b * ws_stride.  Workgroup row blockIdx.y of a
// launch is grid blockIdx.y of the pointers it is given.
struct HardArgs {
  const void* grid;
  int dtype;          // 0 = u8, 1 = f32
  int64_t nz, ny, nx; // nz = 1 for a 2D grid
  const float* tau;
  int H;
  int64_t* out;
  void* ws;
  int64_t batch = 1;
  int64_t tau_stride = 0;
  size_t ws_stride = 0;
  int acc_copies = kAccCopies;
};

// Batches as for HardArgs; grad_out of grid b is grad_out + b * H.
struct SoftArgs {
  const float* grid;
  int64_t nz, ny, nx;  // nz = 1 for 2D
  const float* tau;
  int H;
  float lambda;
  const float* grad_out;  // null for the forward pass
  float* out;             // S (forward) or grad_tau (backward), H per grid
  void* ws;
  int64_t batch = 1;
  int64_t tau_stride = 0;
  size_t ws_stride = 0;
  int acc_copies = kAccCopies;
  // Backward with thresholds shared by the batch, summed over it: out is the
  // one float32[H] gradient of tau.  sum_batch = the whole batch (0: off),
  // ws_base = the workspace of grid 0, b_first = this launch's first grid.
  int64_t sum_batch = 0;
  void* ws_base = nullptr;
  int64_t b_first = 0;
};

// Grids per group of the two-level batch sum (soft backward, shared tau).
constexpr int64_t kSumGroup = 64;

struct GradArgs {
  const float* grid;
  int64_t nz, ny, nx;  // nz = 1 for 2D
  const float* tau;
  int H;
  float lambda;
  const float* grad_out;
  float* out;  // grad_grid, one value per voxel
  int64_t batch = 1;
  int64_t tau_stride = 0;
};

// Directional heights f_d = X + alpha_d <u_d, p> and their backward.
struct HeightArgs {
  const float* grid;   // forward input X
  int nd;              // 2 or 3
  int64_t nz, ny, nx;  // nz = 1 for 2D
  const float* dirs;   // [D][nd], axis order slowest first
  const float* alpha;  // [D]
  int D;
  float* out;          // forward: [D][voxels]
  const float* grad_h; // backward: dL/df, [D][voxels]
  float* grad_grid;    // [voxels] or null
  float* grad_dirs;    // [D][nd] (with grad_alpha) or null
  float* grad_alpha;   // [D]
  void* ws;
};

// Moments workspace: [D tickets, padded | D x blocks x nd float64 slots].
__host__ __device__ inline size_t height_ws_header(int D) {
  return ((size_t)D * sizeof(unsigned int) + 255) & ~(size_t)255;
}
__host__ __device__ inline int height_moment_blocks(int D) {
  const int b = (4096 + D - 1) / D;
  return b > 1024 ? 1024 : (b < 1 ? 1 : b);
}
inline size_t height_workspace_bytes(int nd, int D) {
  return height_ws_header(D) + (size_t)D * height_moment_blocks(D) * nd * sizeof(double);
}

// Largest number of grids in one launch (the workgroup grid's y extent).
constexpr int64_t kMaxBatchPerLaunch = 65535;

// Workspace stride between the grids of a batch.
inline size_t batch_ws_stride(int H, int64_t batch) {
  return (workspace_bytes(H, batch_copies(batch)) + 255) & ~(size_t)255;
}

struct DeviceInfo {
  int cus;
  size_t lds_bytes;
};

// Per-device properties, cached (ecc_api.cpp).
hipError_t device_info(DeviceInfo* info);

// The workspace of ecc_hard_3d_static: a static device array per GPU that
// holds the workspace of one hard call for any H <= 8192 (ecc_static.hip).
constexpr size_t kStaticWorkspaceBytes = kWsHeader + (size_t)kAccCopies * 8192 * sizeof(long long) + kGroupTicketBytes;
// Its address on the current device (looked up and cleared on `stream` by
// the first call for that device).
hipError_t static_workspace(hipStream_t stream, void** ptr);

hipError_t launch_hard(const HardArgs& a, hipStream_t stream);
hipError_t launch_soft(const SoftArgs& a, hipStream_t stream);
hipError_t launch_soft_grad(const GradArgs& a, hipStream_t stream);
hipError_t launch_height(const HeightArgs& a, hipStream_t stream);
hipError_t launch_height_bwd(const HeightArgs& a, hipStream_t stream);

}  // namespace ecc
