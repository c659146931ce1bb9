// C ABI of libecc_mi355: argument validation, error reporting, dispatch.
// The operations themselves are defined on the page "Scalable GPU-Accelerated
// Euler Characteristic Curves" (paper notes), "Method / Key designs"; see
// include/ecc.h for the contract of every entry point.

#include "../../include/ecc.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "ecc_internal.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, const char* detail = nullptr, long long a = 0, long long b = 0) {
  snprintf(g_err, sizeof(g_err), fmt, detail ? detail : "", a, b);
  return status;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

// Per-grid checks of the hard entry points; the workspace is checked only
// when `with_ws` (batched calls check it for the whole batch).
int check_hard(const void* grid, int dtype, int64_t nz, int64_t ny, int64_t nx, const float* tau,
               int32_t H, const int64_t* out, const void* ws, size_t ws_bytes, bool with_ws = true) {
  g_err[0] = 0;
  if (!grid) return fail(ECC_E_NULL, "%sgrid is NULL");
  if (!tau) return fail(ECC_E_NULL, "%stau is NULL");
  if (!out) return fail(ECC_E_NULL, "%sout is NULL");
  if (dtype != ECC_U8 && dtype != ECC_F32)
    return fail(ECC_E_DTYPE, "%sdtype %lld is neither ECC_U8 (0) nor ECC_F32 (1)", nullptr, dtype);
  if (nz < 1 || ny < 1 || nx < 1)
    return fail(ECC_E_SHAPE, "%severy dimension must be >= 1 (got ny=%lld nx=%lld)", nullptr, ny, nx);
  if (nx > ECC_MAX_VOXELS || ny > ECC_MAX_VOXELS / nx || nz > ECC_MAX_VOXELS / (nx * ny))
    return fail(ECC_E_SHAPE, "%sgrid has more than 2^40 voxels");
  if (H < 1 || H > ECC_MAX_THRESHOLDS)
    return fail(ECC_E_NTHRESH, "%sH=%lld outside [1, %lld]", nullptr, H, ECC_MAX_THRESHOLDS);
  if (!with_ws) return ECC_OK;
  if (!ws) return fail(ECC_E_WORKSPACE, "%sworkspace is NULL");
  const size_t need = ecc::workspace_bytes(H);
  if (ws_bytes < need)
    return fail(ECC_E_WORKSPACE, "%sworkspace has %lld bytes, needs %lld", nullptr, (long long)ws_bytes,
                (long long)need);
  return ECC_OK;
}

// Batch-specific checks: batch >= 1, tau_stride >= 0, all voxels within the
// ABI limit, and (when `with_ws`) a workspace slice for every grid.
int check_batch(int64_t batch, int64_t tau_stride, int64_t nvox, const void* ws, size_t ws_bytes,
                int32_t H, bool with_ws) {
  if (batch < 1) return fail(ECC_E_SHAPE, "%sbatch=%lld, must be >= 1", nullptr, batch);
  if (tau_stride < 0) return fail(ECC_E_SHAPE, "%stau_stride=%lld, must be >= 0", nullptr, tau_stride);
  if (batch > ECC_MAX_VOXELS / nvox) return fail(ECC_E_SHAPE, "%sbatch has more than 2^40 voxels");
  if (!with_ws) return ECC_OK;
  if (!ws) return fail(ECC_E_WORKSPACE, "%sworkspace is NULL");
  const size_t need = (size_t)batch * ecc::batch_ws_stride(H, batch);
  if (ws_bytes < need)
    return fail(ECC_E_WORKSPACE, "%sworkspace has %lld bytes, needs %lld", nullptr, (long long)ws_bytes,
                (long long)need);
  return ECC_OK;
}

// Checks shared by the soft entry points; the workspace is checked only when
// `with_ws` (the grid gradient needs none).
int check_soft(const float* grid, int32_t ndim, const int64_t* shape, const float* tau, int32_t H,
               float lambda, const void* out, const void* ws, size_t ws_bytes, int64_t dims[3],
               bool with_ws = true) {
  g_err[0] = 0;
  if (!grid) return fail(ECC_E_NULL, "%sgrid is NULL");
  if (!shape) return fail(ECC_E_NULL, "%sshape is NULL");
  if (!tau) return fail(ECC_E_NULL, "%stau is NULL");
  if (!out) return fail(ECC_E_NULL, "%soutput is NULL");
  if (ndim != 2 && ndim != 3) return fail(ECC_E_SHAPE, "%sndim=%lld, must be 2 or 3", nullptr, ndim);
  dims[0] = ndim == 3 ? shape[0] : 1;
  dims[1] = shape[ndim - 2];
  dims[2] = shape[ndim - 1];
  for (int i = 0; i < 3; ++i)
    if (dims[i] < 1) return fail(ECC_E_SHAPE, "%severy dimension must be >= 1");
  if (dims[2] > ECC_MAX_VOXELS || dims[1] > ECC_MAX_VOXELS / dims[2] ||
      dims[0] > ECC_MAX_VOXELS / (dims[1] * dims[2]))
    return fail(ECC_E_SHAPE, "%sgrid has more than 2^40 voxels");
  if (H < 1 || H > ECC_MAX_THRESHOLDS)
    return fail(ECC_E_NTHRESH, "%sH=%lld outside [1, %lld]", nullptr, H, ECC_MAX_THRESHOLDS);
  if (!(lambda > 0.0f) || !isfinite(lambda))
    return fail(ECC_E_LAMBDA, "%slambda must be finite and > 0");
  if (!with_ws) return ECC_OK;
  if (!ws) return fail(ECC_E_WORKSPACE, "%sworkspace is NULL");
  const size_t need = ecc::workspace_bytes(H);
  if (ws_bytes < need)
    return fail(ECC_E_WORKSPACE, "%sworkspace has %lld bytes, needs %lld", nullptr, (long long)ws_bytes,
                (long long)need);
  return ECC_OK;
}

// Checks of the height entry points; fills dims (nz = 1 in 2D).
int check_height(const void* grid, int32_t ndim, const int64_t* shape, const float* dirs, const float* alpha,
                 int32_t D, const void* out, int64_t dims[3]) {
  g_err[0] = 0;
  if (!grid) return fail(ECC_E_NULL, "%sgrid is NULL");
  if (!shape) return fail(ECC_E_NULL, "%sshape is NULL");
  if (!dirs) return fail(ECC_E_NULL, "%sdirs is NULL");
  if (!alpha) return fail(ECC_E_NULL, "%salpha is NULL");
  if (!out) return fail(ECC_E_NULL, "%soutput is NULL");
  if (ndim != 2 && ndim != 3) return fail(ECC_E_SHAPE, "%sndim=%lld, must be 2 or 3", nullptr, ndim);
  dims[0] = ndim == 3 ? shape[0] : 1;
  dims[1] = shape[ndim - 2];
  dims[2] = shape[ndim - 1];
  for (int i = 0; i < 3; ++i)
    if (dims[i] < 1 || dims[i] > ECC_MAX_AXIS)
      return fail(ECC_E_SHAPE, "%severy dimension must be in [1, 2^24]");
  if (D < 1 || D > ECC_MAX_DIRECTIONS)
    return fail(ECC_E_NDIRS, "%sD=%lld outside [1, %lld]", nullptr, D, ECC_MAX_DIRECTIONS);
  const int64_t nvox = dims[0] * dims[1] * dims[2];
  if (nvox > ECC_MAX_VOXELS / D) return fail(ECC_E_SHAPE, "%sD x voxels exceeds 2^40");
  return ECC_OK;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return ECC_OK;
  return fail(ECC_E_HIP, "HIP error: %s", hipGetErrorString(e));
}

}  // namespace

namespace ecc {

hipError_t device_info(DeviceInfo* info) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int cus = (dev >= 0 && dev < kMaxDevices) ? g_cus[dev].load(std::memory_order_relaxed) : 0;
  if (cus <= 0) {
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(cus, std::memory_order_relaxed);
  }
  info->cus = cus > 0 ? cus : 1;
  info->lds_bytes = 160 * 1024;
  return hipSuccess;
}

}  // namespace ecc

extern "C" {

int ecc_hard_2d(const void* grid, int dtype, int64_t ny, int64_t nx, const float* tau, int32_t H,
                int64_t* out, void* ws, size_t ws_bytes, void* stream) {
  int st = check_hard(grid, dtype, 1, ny, nx, tau, H, out, ws, ws_bytes);
  if (st != ECC_OK) return st;
  ecc::HardArgs a{grid, dtype, 1, ny, nx, tau, H, out, ws};
  return hip_status(ecc::launch_hard(a, reinterpret_cast<hipStream_t>(stream)));
}

int ecc_hard_3d(const void* grid, int dtype, int64_t nz, int64_t ny, int64_t nx, const float* tau,
                int32_t H, int64_t* out, void* ws, size_t ws_bytes, void* stream) {
  int st = check_hard(grid, dtype, nz, ny, nx, tau, H, out, ws, ws_bytes);
  if (st != ECC_OK) return st;
  ecc::HardArgs a{grid, dtype, nz, ny, nx, tau, H, out, ws};
  return hip_status(ecc::launch_hard(a, reinterpret_cast<hipStream_t>(stream)));
}

int ecc_hard_3d_static(const void* grid, int dtype, int64_t nz, int64_t ny, int64_t nx, const float* tau,
                       int32_t H, int64_t* out, void* stream) {
  int st = check_hard(grid, dtype, nz, ny, nx, tau, H, out, nullptr, 0, false);
  if (st != ECC_OK) return st;
  const size_t need = ecc::workspace_bytes(H);
  if (need > ecc::kStaticWorkspaceBytes)
    return fail(ECC_E_WORKSPACE, "%sH=%lld needs %lld bytes of scratch, more than the static array holds",
                nullptr, H, (long long)need);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  const hipError_t e = ecc::static_workspace(s, &ws);
  if (e != hipSuccess) return hip_status(e);
  ecc::HardArgs a{grid, dtype, nz, ny, nx, tau, H, out, ws};
  return hip_status(ecc::launch_hard(a, s));
}

int ecc_hard_2d_batched(const void* grid, int dtype, int64_t batch, int64_t ny, int64_t nx,
                        const float* tau, int64_t tau_stride, int32_t H, int64_t* out, void* ws,
                        size_t ws_bytes, void* stream) {
  return ecc_hard_3d_batched(grid, dtype, batch, 1, ny, nx, tau, tau_stride, H, out, ws, ws_bytes, stream);
}

int ecc_hard_3d_batched(const void* grid, int dtype, int64_t batch, int64_t nz, int64_t ny, int64_t nx,
                        const float* tau, int64_t tau_stride, int32_t H, int64_t* out, void* ws,
                        size_t ws_bytes, void* stream) {
  int st = check_hard(grid, dtype, nz, ny, nx, tau, H, out, ws, ws_bytes, false);
  if (st != ECC_OK) return st;
  st = check_batch(batch, tau_stride, nz * ny * nx, ws, ws_bytes, H, true);
  if (st != ECC_OK) return st;
  ecc::HardArgs a{grid, dtype, nz, ny, nx, tau, H, out, ws};
  a.batch = batch;
  a.tau_stride = tau_stride;
  a.ws_stride = ecc::batch_ws_stride(H, batch);
  a.acc_copies = ecc::batch_copies(batch);
  return hip_status(ecc::launch_hard(a, reinterpret_cast<hipStream_t>(stream)));
}

int ecc_soft_fwd(const float* grid, int32_t ndim, const int64_t* shape, const float* tau, int32_t H,
                 float lambda, float* out, void* ws, size_t ws_bytes, void* stream) {
  int64_t d[3];
  int st = check_soft(grid, ndim, shape, tau, H, lambda, out, ws, ws_bytes, d);
  if (st != ECC_OK) return st;
  ecc::SoftArgs a{grid, d[0], d[1], d[2], tau, H, lambda, nullptr, out, ws};
  return hip_status(ecc::launch_soft(a, reinterpret_cast<hipStream_t>(stream)));
}

int ecc_soft_bwd_tau(const float* grid, int32_t ndim, const int64_t* shape, const float* tau,
                     int32_t H, float lambda, const float* grad_out, float* grad_tau, void* ws,
                     size_t ws_bytes, void* stream) {
  int64_t d[3];
  int st = check_soft(grid, ndim, shape, tau, H, lambda, grad_tau, ws, ws_bytes, d);
  if (st != ECC_OK) return st;
  if (!grad_out) return fail(ECC_E_NULL, "%sgrad_out is NULL");
  ecc::SoftArgs a{grid, d[0], d[1], d[2], tau, H, lambda, grad_out, grad_tau, ws};
  return hip_status(ecc::launch_soft(a, reinterpret_cast<hipStream_t>(stream)));
}

int ecc_soft_bwd_grid(const float* grid, int32_t ndim, const int64_t* shape, const float* tau,
                      int32_t H, float lambda, const float* grad_out, float* grad_grid, void* stream) {
  int64_t d[3];
  int st = check_soft(grid, ndim, shape, tau, H, lambda, grad_grid, nullptr, 0, d, false);
  if (st != ECC_OK) return st;
  if (!grad_out) return fail(ECC_E_NULL, "%sgrad_out is NULL");
  ecc::GradArgs a{grid, d[0], d[1], d[2], tau, H, lambda, grad_out, grad_grid};
  return hip_status(ecc::launch_soft_grad(a, reinterpret_cast<hipStream_t>(stream)));
}

int ecc_soft_fwd_batched(const float* grid, int32_t ndim, const int64_t* shape, int64_t batch,
                         const float* tau, int64_t tau_stride, int32_t H, float lambda, float* out, void* ws,
                         size_t ws_bytes, void* stream) {
  int64_t d[3];
  int st = check_soft(grid, ndim, shape, tau, H, lambda, out, ws, ws_bytes, d, false);
  if (st != ECC_OK) return st;
  st = check_batch(batch, tau_stride, d[0] * d[1] * d[2], ws, ws_bytes, H, true);
  if (st != ECC_OK) return st;
  ecc::SoftArgs a{grid, d[0], d[1], d[2], tau, H, lambda, nullptr, out, ws};
  a.batch = batch;
  a.tau_stride = tau_stride;
  a.ws_stride = ecc::batch_ws_stride(H, batch);
  a.acc_copies = ecc::batch_copies(batch);
  return hip_status(ecc::launch_soft(a, reinterpret_cast<hipStream_t>(stream)));
}

int ecc_soft_bwd_tau_batched(const float* grid, int32_t ndim, const int64_t* shape, int64_t batch,
                             const float* tau, int64_t tau_stride, int32_t H, float lambda,
                             const float* grad_out, float* grad_tau, void* ws, size_t ws_bytes,
                             void* stream) {
  int64_t d[3];
  int st = check_soft(grid, ndim, shape, tau, H, lambda, grad_tau, ws, ws_bytes, d, false);
  if (st != ECC_OK) return st;
  if (!grad_out) return fail(ECC_E_NULL, "%sgrad_out is NULL");
  st = check_batch(batch, tau_stride, d[0] * d[1] * d[2], ws, ws_bytes, H, true);
  if (st != ECC_OK) return st;
  ecc::SoftArgs a{grid, d[0], d[1], d[2], tau, H, lambda, grad_out, grad_tau, ws};
  a.batch = batch;
  a.tau_stride = tau_stride;
  a.ws_stride = ecc::batch_ws_stride(H, batch);
  a.acc_copies = ecc::batch_copies(batch);
  return hip_status(ecc::launch_soft(a, reinterpret_cast<hipStream_t>(stream)));
}

int ecc_soft_bwd_tau_shared(const float* grid, int32_t ndim, const int64_t* shape, int64_t batch,
                            const float* tau, int32_t H, float lambda, const float* grad_out, float* grad_tau,
                            void* ws, size_t ws_bytes, void* stream) {
  int64_t d[3];
  int st = check_soft(grid, ndim, shape, tau, H, lambda, grad_tau, ws, ws_bytes, d, false);
  if (st != ECC_OK) return st;
  if (!grad_out) return fail(ECC_E_NULL, "%sgrad_out is NULL");
  st = check_batch(batch, 0, d[0] * d[1] * d[2], ws, ws_bytes, H, true);
  if (st != ECC_OK) return st;
  ecc::SoftArgs a{grid, d[0], d[1], d[2], tau, H, lambda, grad_out, grad_tau, ws};
  a.batch = batch;
  a.tau_stride = 0;
  a.ws_stride = ecc::batch_ws_stride(H, batch);
  a.acc_copies = ecc::batch_copies(batch);
  a.sum_batch = batch;
  return hip_status(ecc::launch_soft(a, reinterpret_cast<hipStream_t>(stream)));
}

int ecc_soft_bwd_grid_batched(const float* grid, int32_t ndim, const int64_t* shape, int64_t batch,
                              const float* tau, int64_t tau_stride, int32_t H, float lambda,
                              const float* grad_out, float* grad_grid, void* stream) {
  int64_t d[3];
  int st = check_soft(grid, ndim, shape, tau, H, lambda, grad_grid, nullptr, 0, d, false);
  if (st != ECC_OK) return st;
  if (!grad_out) return fail(ECC_E_NULL, "%sgrad_out is NULL");
  st = check_batch(batch, tau_stride, d[0] * d[1] * d[2], nullptr, 0, H, false);
  if (st != ECC_OK) return st;
  ecc::GradArgs a{grid, d[0], d[1], d[2], tau, H, lambda, grad_out, grad_grid};
  a.batch = batch;
  a.tau_stride = tau_stride;
  return hip_status(ecc::launch_soft_grad(a, reinterpret_cast<hipStream_t>(stream)));
}

int ecc_height(const float* grid, int32_t ndim, const int64_t* shape, const float* dirs, const float* alpha,
               int32_t D, float* out, void* stream) {
  int64_t d[3];
  int st = check_height(grid, ndim, shape, dirs, alpha, D, out, d);
  if (st != ECC_OK) return st;
  ecc::HeightArgs a{};
  a.grid = grid;
  a.nd = ndim;
  a.nz = d[0];
  a.ny = d[1];
  a.nx = d[2];
  a.dirs = dirs;
  a.alpha = alpha;
  a.D = D;
  a.out = out;
  return hip_status(ecc::launch_height(a, reinterpret_cast<hipStream_t>(stream)));
}

int ecc_height_bwd(const float* grad_h, int32_t ndim, const int64_t* shape, const float* dirs, const float* alpha,
                   int32_t D, float* grad_grid, float* grad_dirs, float* grad_alpha, void* ws, size_t ws_bytes,
                   void* stream) {
  int64_t d[3];
  int st = check_height(grad_h, ndim, shape, dirs, alpha, D, grad_grid ? (void*)grad_grid : (void*)grad_dirs, d);
  if (st != ECC_OK) return st;
  if ((grad_dirs == nullptr) != (grad_alpha == nullptr))
    return fail(ECC_E_NULL, "%sgrad_dirs and grad_alpha must both be given or both be NULL");
  if (grad_dirs) {
    if (!ws) return fail(ECC_E_WORKSPACE, "%sworkspace is NULL");
    const size_t need = ecc::height_workspace_bytes(ndim, D);
    if (ws_bytes < need)
      return fail(ECC_E_WORKSPACE, "%sworkspace has %lld bytes, needs %lld", nullptr, (long long)ws_bytes,
                  (long long)need);
  }
  ecc::HeightArgs a{};
  a.nd = ndim;
  a.nz = d[0];
  a.ny = d[1];
  a.nx = d[2];
  a.dirs = dirs;
  a.alpha = alpha;
  a.D = D;
  a.grad_h = grad_h;
  a.grad_grid = grad_grid;
  a.grad_dirs = grad_dirs;
  a.grad_alpha = grad_alpha;
  a.ws = ws;
  return hip_status(ecc::launch_height_bwd(a, reinterpret_cast<hipStream_t>(stream)));
}

size_t ecc_height_workspace_bytes(int32_t ndim, int32_t D) {
  if ((ndim != 2 && ndim != 3) || D < 1 || D > ECC_MAX_DIRECTIONS) return 0;
  return ecc::height_workspace_bytes(ndim, D);
}

size_t ecc_workspace_bytes(int op, int32_t ndim, const int64_t* shape, int32_t H) {
  (void)ndim;
  (void)shape;
  if (op != ECC_OP_HARD && op != ECC_OP_SOFT_FWD && op != ECC_OP_SOFT_BWD) return 0;
  if (H < 1 || H > ECC_MAX_THRESHOLDS) return 0;
  return ecc::workspace_bytes(H);
}

size_t ecc_workspace_bytes_batched(int op, int64_t batch, int32_t H) {
  if (op != ECC_OP_HARD && op != ECC_OP_SOFT_FWD && op != ECC_OP_SOFT_BWD) return 0;
  if (H < 1 || H > ECC_MAX_THRESHOLDS || batch < 1 || batch > ECC_MAX_VOXELS) return 0;
  return (size_t)batch * ecc::batch_ws_stride(H, batch);
}

const char* ecc_status_string(int status) {
  switch (status) {
    case ECC_OK: return "ok";
    case ECC_E_NULL: return "a required pointer is NULL";
    case ECC_E_SHAPE: return "invalid grid shape";
    case ECC_E_DTYPE: return "unsupported grid dtype";
    case ECC_E_NTHRESH: return "number of thresholds out of range";
    case ECC_E_LAMBDA: return "lambda must be finite and > 0";
    case ECC_E_WORKSPACE: return "workspace missing or too small";
    case ECC_E_HIP: return "HIP runtime error";
    case ECC_E_NDIRS: return "number of directions out of range";
    default: return "unknown status";
  }
}

const char* ecc_last_error(void) { return g_err; }

const char* ecc_version(void) { return "0.1.0"; }

}  // extern "C"
