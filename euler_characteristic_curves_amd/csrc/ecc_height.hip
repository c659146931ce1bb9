// Directional heights for the single- and multi-direction curves, gfx950.
//
// The page's differentiable layer adds a learnable direction u and scale
// alpha for its single-direction version, and names the multi-direction
// transform as the complete one (page "Scalable GPU-Accelerated Euler
// Characteristic Curves", "Method / Key designs / differentiable ECC layer",
// "Limitations and outlook").  The height of voxel p along direction d is
//     f_d(p) = X(p) + alpha_d * <u_d, p>,   p = integer voxel index,
// evaluated in float32 with every product and sum rounded in the order
//     h = (u_0 p_0 + u_1 p_1) [+ u_2 p_2],   f = X + alpha * h
// and nothing fused, so the values (and hence the hard curves of f) are
// reproducible bit for bit.  The curves of direction d are those of the grid
// f_d, computed by the batched entry points over the D height grids.
//
// Backward: with G_d = dL/df_d (the grid gradient of each height grid),
//     dL/dX = sum_d G_d,
//     M_d,i = sum_p G_d(p) p_i,  dL/du_d,i = alpha_d M_d,i,  dL/dalpha_d = sum_i u_d,i M_d,i.
// The moments are float64 per thread and workgroup; each workgroup adds its
// partial into its own zeroed workspace slot (one device-scope add, so the
// slot holds the partial exactly) and the last workgroup of the direction
// sums the slots in order: the result does not depend on scheduling.

#include <hip/hip_runtime.h>

#include "ecc_device.hpp"
#include "ecc_internal.hpp"

namespace ecc {
namespace {

constexpr int kHNT = 256;
constexpr int kHTileX = 4 * kHNT;  // columns per tile: 4 coalesced passes of the workgroup

// Tiles are (row, column block); rows are (z, y) in 3D and y in 2D.
struct HeightGeom {
  int64_t n1, nx, nrows, ntx, ntiles, nvox;
};

__host__ __device__ inline HeightGeom height_geom(const HeightArgs& a) {
  HeightGeom g;
  g.n1 = a.ny;
  g.nx = a.nx;
  g.nrows = a.nz * a.ny;
  g.ntx = (a.nx + kHTileX - 1) / kHTileX;
  g.ntiles = g.nrows * g.ntx;
  g.nvox = g.nrows * a.nx;
  return g;
}

// A voxel index as float32, rounded once: through float64, which holds any
// index exactly.  (The direct 64-bit-integer conversion that the compiler
// emits for this target, a normalising 64-bit shift and a 32-bit convert,
// gave wrong coordinates now and then for indices of 256 and up in the
// element-wise kernel below; the float64 route has no 64-bit shift.)
__device__ __forceinline__ float coord(int64_t i) { return (float)(double)i; }

// Height of one voxel, rounded step by step (no contraction into FMAs).
template <int ND>
__device__ __forceinline__ float height_of(float X, float alpha, const float* u, float pz, float py, float px) {
#pragma clang fp contract(off)
  float h;
  if constexpr (ND == 3) {
    const float a = u[0] * pz;
    const float b = u[1] * py;
    const float ab = a + b;
    const float c = u[2] * px;
    h = ab + c;
  } else {
    const float a = u[0] * py;
    const float c = u[1] * px;
    h = a + c;
  }
  const float s = alpha * h;
  return X + s;
}

template <int ND>
__global__ __launch_bounds__(kHNT) void height_kernel(HeightArgs a) {
  extern __shared__ float sd[];  // u[D][ND] then alpha[D]
  const int D = a.D;
  for (int i = threadIdx.x; i < D * (ND + 1); i += kHNT) sd[i] = i < D * ND ? a.dirs[i] : a.alpha[i - D * ND];
  __syncthreads();
  const HeightGeom g = height_geom(a);
  for (int64_t t = blockIdx.x; t < g.ntiles; t += gridDim.x) {
    const int64_t row = t / g.ntx, xc = t - row * g.ntx;
    const int64_t z = ND == 3 ? row / g.n1 : 0, y = row - z * g.n1;
    float X[4];
    int64_t xs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xs[j] = xc * kHTileX + j * kHNT + threadIdx.x;
      X[j] = xs[j] < g.nx ? a.grid[row * g.nx + xs[j]] : 0.0f;
    }
    for (int d = 0; d < D; ++d) {
      const float* u = sd + d * ND;
      const float al = sd[D * ND + d];
      float* out = a.out + (size_t)d * (size_t)g.nvox + row * g.nx;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (xs[j] < g.nx) out[xs[j]] = height_of<ND>(X[j], al, u, coord(z), coord(y), coord(xs[j]));
    }
  }
}

// Coordinates of a thread's current voxel along a grid-stride walk: one
// division at the start, then a mixed-radix add of the stride per step.
struct Walk {
  int64_t x, y, z, sx, sy, sz, nx, ny;
  __device__ void init(int64_t idx, int64_t stride, int64_t nx_, int64_t ny_) {
    nx = nx_;
    ny = ny_;
    const int64_t r = idx / nx, rs = stride / nx;
    x = idx - r * nx;
    z = r / ny;
    y = r - z * ny;
    sx = stride - rs * nx;
    sz = rs / ny;
    sy = rs - sz * ny;
  }
  __device__ void step() {
    x += sx;
    y += sy;
    if (x >= nx) {
      x -= nx;
      ++y;
    }
    z += sz;
    if (y >= ny) {
      y -= ny;
      ++z;
    }
  }
};

// Rows of a multiple of 4 voxels with 16-byte aligned grid and output:
// every thread takes 4 consecutive voxels of the flattened grid (one row, as
// nx is a multiple of 4) and writes one float4 per direction, so narrow rows
// keep every lane busy and stores are 16 bytes wide.
template <int ND>
__global__ __launch_bounds__(kHNT) void height_vec_kernel(HeightArgs a, int64_t nquads) {
  extern __shared__ float sd[];  // u[D][ND] then alpha[D]
  const int D = a.D;
  for (int i = threadIdx.x; i < D * (ND + 1); i += kHNT) sd[i] = i < D * ND ? a.dirs[i] : a.alpha[i - D * ND];
  __syncthreads();
  const int64_t nvox = a.nz * a.ny * a.nx;
  const int64_t stride = (int64_t)gridDim.x * kHNT;
  const int64_t q0 = (int64_t)blockIdx.x * kHNT + threadIdx.x;
  Walk w;
  w.init(4 * q0, 4 * stride, a.nx, a.ny);
  for (int64_t q = q0; q < nquads; q += stride, w.step()) {
    const int64_t idx = 4 * q, x0 = w.x;
    const float4 X = *reinterpret_cast<const float4*>(a.grid + idx);
    const float pz = coord(ND == 3 ? w.z : 0), py = coord(w.y);
    for (int d = 0; d < D; ++d) {
      const float* u = sd + d * ND;
      const float al = sd[D * ND + d];
      float4 f;
      f.x = height_of<ND>(X.x, al, u, pz, py, coord(x0 + 0));
      f.y = height_of<ND>(X.y, al, u, pz, py, coord(x0 + 1));
      f.z = height_of<ND>(X.z, al, u, pz, py, coord(x0 + 2));
      f.w = height_of<ND>(X.w, al, u, pz, py, coord(x0 + 3));
      *reinterpret_cast<float4*>(a.out + (size_t)d * (size_t)nvox + idx) = f;
    }
  }
}

// dL/dX = sum over directions, float32 in increasing d.
__global__ __launch_bounds__(kHNT) void height_grid_grad_kernel(HeightArgs a, int64_t nvox) {
  const int64_t stride = (int64_t)gridDim.x * kHNT;
  for (int64_t i = (int64_t)blockIdx.x * kHNT + threadIdx.x; i < nvox; i += stride) {
    float s = 0.0f;
    for (int d = 0; d < a.D; ++d) s += a.grad_h[(size_t)d * (size_t)nvox + i];
    a.grad_grid[i] = s;
  }
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Moments of direction blockIdx.y, then dL/du and dL/dalpha by its last
// workgroup.  VEC: rows of a multiple of 4 voxels, 16-byte aligned, read as
// float4 quads along a grid-stride walk; otherwise row tiles.
template <int ND, bool VEC>
__global__ __launch_bounds__(kHNT) void height_moments_kernel(HeightArgs a) {
  __shared__ double red[kHNT / 64][ND];
  __shared__ double Ms[ND];
  __shared__ int last;
  const int d = blockIdx.y;
  const HeightGeom g = height_geom(a);
  const float* G = a.grad_h + (size_t)d * (size_t)g.nvox;
  double m[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) m[i] = 0.0;
  // the voxels of one quad or one row share z and y
  auto add = [&](double s, double sx, int64_t z, int64_t y) {
    if constexpr (ND == 3) {
      m[0] = fma(s, (double)z, m[0]);
      m[1] = fma(s, (double)y, m[1]);
      m[2] += sx;
    } else {
      m[0] = fma(s, (double)y, m[0]);
      m[1] += sx;
    }
  };
  if constexpr (VEC) {
    const int64_t nquads = g.nvox / 4, stride = (int64_t)gridDim.x * kHNT;
    const int64_t q0 = (int64_t)blockIdx.x * kHNT + threadIdx.x;
    Walk w;
    w.init(4 * q0, 4 * stride, g.nx, g.n1);
    for (int64_t q = q0; q < nquads; q += stride, w.step()) {
      const float4 v = *reinterpret_cast<const float4*>(G + 4 * q);
      const double x = (double)w.x;
      const double s = ((double)v.x + (double)v.y) + ((double)v.z + (double)v.w);
      const double sx = fma((double)v.x, x, fma((double)v.y, x + 1.0, fma((double)v.z, x + 2.0, (double)v.w * (x + 3.0))));
      add(s, sx, w.z, w.y);
    }
  } else {
    for (int64_t t = blockIdx.x; t < g.ntiles; t += gridDim.x) {
      const int64_t row = t / g.ntx, xc = t - row * g.ntx;
      const int64_t z = ND == 3 ? row / g.n1 : 0, y = row - z * g.n1;
      double sx = 0.0, s = 0.0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t x = xc * kHTileX + j * kHNT + threadIdx.x;
        if (x < g.nx) {
          const double v = (double)G[row * g.nx + x];
          s += v;
          sx = fma(v, (double)x, sx);
        }
      }
      add(s, sx, z, y);
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    const double v = wave_sum(m[i]);
    if (lane == 0) red[wave][i] = v;
  }
  __syncthreads();
  double* part = reinterpret_cast<double*>(reinterpret_cast<char*>(a.ws) + height_ws_header(a.D)) +
                 ((size_t)d * gridDim.x + blockIdx.x) * ND;
  unsigned int* ticket = reinterpret_cast<unsigned int*>(a.ws) + d;
  if (threadIdx.x < ND) {
    double v = 0.0;
    for (int w = 0; w < kHNT / 64; ++w) v += red[w][threadIdx.x];
    // the slot is zero: this device-scope add leaves exactly v in it
    __hip_atomic_fetch_add(part + threadIdx.x, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's add is acknowledged
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned int prev = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = (prev == gridDim.x - 1);
    if (last) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last) return;
  double* slots = part - (size_t)blockIdx.x * ND;  // direction d's first slot
  if (threadIdx.x < ND) {
    double s = 0.0;
    for (unsigned int w = 0; w < gridDim.x; ++w) s += agent_load(slots + (size_t)w * ND + threadIdx.x);
    for (unsigned int w = 0; w < gridDim.x; ++w) agent_store(slots + (size_t)w * ND + threadIdx.x, 0.0);
    Ms[threadIdx.x] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double ga = 0.0;
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      ga += (double)a.dirs[d * ND + i] * Ms[i];
      a.grad_dirs[d * ND + i] = (float)((double)a.alpha[d] * Ms[i]);
    }
    a.grad_alpha[d] = (float)ga;
  }
}

int64_t height_blocks(const HeightGeom& g, int cus) {
  int64_t b = (int64_t)cus * 8;
  if (b > g.ntiles) b = g.ntiles;
  return b < 1 ? 1 : b;
}

}  // namespace

hipError_t launch_height(const HeightArgs& a, hipStream_t s) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  const HeightGeom g = height_geom(a);
  const size_t lds = (size_t)a.D * (a.nd + 1) * sizeof(float);
  const void* k = a.nd == 3 ? reinterpret_cast<const void*>(height_kernel<3>)
                            : reinterpret_cast<const void*>(height_kernel<2>);
  if (lds > 64 * 1024) {
    e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const bool vec = a.nx % 4 == 0 && reinterpret_cast<uintptr_t>(a.grid) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(a.out) % 16 == 0;
  if (vec) {
    const void* kv = a.nd == 3 ? reinterpret_cast<const void*>(height_vec_kernel<3>)
                               : reinterpret_cast<const void*>(height_vec_kernel<2>);
    if (lds > 64 * 1024) {
      e = hipFuncSetAttribute(kv, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    const int64_t nquads = g.nvox / 4;
    int64_t nb = (nquads + kHNT - 1) / kHNT;
    if (nb > (int64_t)di.cus * 8) nb = (int64_t)di.cus * 8;
    if (a.nd == 3)
      hipLaunchKernelGGL(height_vec_kernel<3>, dim3((unsigned)nb), dim3(kHNT), lds, s, a, nquads);
    else
      hipLaunchKernelGGL(height_vec_kernel<2>, dim3((unsigned)nb), dim3(kHNT), lds, s, a, nquads);
    return hipGetLastError();
  }
  const unsigned nb = (unsigned)height_blocks(g, di.cus);
  if (a.nd == 3)
    hipLaunchKernelGGL(height_kernel<3>, dim3(nb), dim3(kHNT), lds, s, a);
  else
    hipLaunchKernelGGL(height_kernel<2>, dim3(nb), dim3(kHNT), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_height_bwd(const HeightArgs& a, hipStream_t s) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  const HeightGeom g = height_geom(a);
  if (a.grad_grid) {
    int64_t nb = (g.nvox + kHNT - 1) / kHNT;
    if (nb > (int64_t)di.cus * 16) nb = (int64_t)di.cus * 16;
    hipLaunchKernelGGL(height_grid_grad_kernel, dim3((unsigned)nb), dim3(kHNT), 0, s, a, g.nvox);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.grad_dirs) {
    const dim3 grid((unsigned)height_moment_blocks(a.D), (unsigned)a.D);
    const bool vec = a.nx % 4 == 0 && reinterpret_cast<uintptr_t>(a.grad_h) % 16 == 0;
    if (a.nd == 3) {
      if (vec)
        hipLaunchKernelGGL((height_moments_kernel<3, true>), grid, dim3(kHNT), 0, s, a);
      else
        hipLaunchKernelGGL((height_moments_kernel<3, false>), grid, dim3(kHNT), 0, s, a);
    } else {
      if (vec)
        hipLaunchKernelGGL((height_moments_kernel<2, true>), grid, dim3(kHNT), 0, s, a);
      else
        hipLaunchKernelGGL((height_moments_kernel<2, false>), grid, dim3(kHNT), 0, s, a);
    }
    e = hipGetLastError();
  }
  return e;
}

}  // namespace ecc
