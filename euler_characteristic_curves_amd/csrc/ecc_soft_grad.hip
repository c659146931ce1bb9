// Gradient of the soft (sigmoid-relaxed) Euler characteristic curve with
// respect to the grid values, gfx950.
//
// Method: page "Scalable GPU-Accelerated Euler Characteristic Curves" (paper
// notes), "Method / Key designs / differentiable ECC layer":
//     S_k = sum_c (-1)^dim(c) s(lambda (tau_k - v_c)),  v_c = max of c's corners.
// For L = sum_k g_k S_k, dL/dv_c = -lambda (-1)^dim(c) h(v_c) with
//     h(v) = sum_k g_k s(x)(1 - s(x)),  x = lambda (tau_k - v),
// and dv_c/dX(p) = 1 for the corner p that holds the max (the first in index
// order among equal maxima), 0 for the others.  Every cell that sends its
// derivative to p has the value X(p), so
//     dL/dX(p) = -lambda c(p) h(X(p)),
// c(p) = signed count of those cells (ecc_star.hpp).  The result is a gather,
// not a scatter: one value per voxel, written once, no atomics, no workspace.
//
// Work split.  Every wave walks 64-voxel segments of the grid.  Phase A: each
// lane finds c(p) for its voxel from the 3x3(x3) block around it; voxels with
// c = 0 get 0 at once, the others go to the wave's queue in LDS (value, c,
// index).  Phase B, whenever the queue holds 256 voxels (and once at the
// end): every lane takes 4 queued voxels and sums h over all thresholds, read
// from a per-workgroup table in LDS (one broadcast read serves 2 thresholds
// x 4 voxels).  The sigmoid product uses the factored exponent of the soft
// forward kernel: with t = exp(lambda (v - tau)) = F E, F = 2^{L (v - c0)}
// per voxel and E = 2^{L (c0 - tau)} per threshold (L = lambda log2 e, c0
// the middle of the threshold range), s(1 - s) = t / (1 + t)^2, so
//     h(v) = F sum_k (g_k E_k) r_k^2,  r_k = 1 / (1 + F E_k),
// one FMA, one reciprocal, one multiply and one FMA per (voxel, threshold).
// Where the factors would leave the float range (very wide threshold span or
// huge upstream gradients) every pair takes exp2 directly.

#include <hip/hip_runtime.h>
#include <math.h>

#include "ecc_device.hpp"
#include "ecc_internal.hpp"
#include "ecc_star.hpp"

namespace ecc {
namespace {

constexpr int kGradNT = 256;
constexpr int kGradWaves = kGradNT / 64;
constexpr int kSlots = 4;                  // queued voxels per lane in one sweep
constexpr int kBatch = 64 * kSlots;        // voxels per sweep
constexpr int kQueueCap = kBatch + 64;     // a sweep starts once >= kBatch are queued

struct QEntry {
  float v;        // X(p)
  int c;          // c(p), non-zero
  long long idx;  // linear voxel index
};

struct GradCtx {
  const float2* T;  // per threshold: (E_k, g_k E_k) factored, (tau_k, g_k) direct
  int Hp;           // table length, H rounded up to even (pad entries are (0, 0))
  bool factored;
  double L64, cen;
  float Lf, lambda;
  float* out;
};

// Orders this wave's LDS accesses around it (queue writes by some lanes are
// read by other lanes of the same wave).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Phase B: sum h over all thresholds for queue entries q[0..n) (n <= kBatch),
// lane l taking entries l, l + 64, l + 128, l + 192; write the gradients.
__device__ __forceinline__ void sweep(const GradCtx& g, const QEntry* q, int n, int lane) {
  float a[kSlots];
  float wc[kSlots];
  long long id[kSlots];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int e = lane + 64 * j;
    const bool ok = e < n;
    const QEntry qe = q[ok ? e : 0];
    id[j] = ok ? qe.idx : -1;
    wc[j] = (float)qe.c;
    // F kept finite, so F E overflowing to inf only ever meets a 0 reciprocal
    a[j] = g.factored ? fminf(exp2_split(g.L64 * ((double)qe.v - g.cen)), 0x1p126f) : qe.v;
  }
  float acc[kSlots] = {0.0f, 0.0f, 0.0f, 0.0f};
  const float4* T4 = reinterpret_cast<const float4*>(g.T);
  const int n2 = g.Hp >> 1;
  if (g.factored) {
    for (int k = 0; k < n2; ++k) {
      const float4 t = T4[k];
#pragma unroll
      for (int j = 0; j < kSlots; ++j) {
        const float r0 = __builtin_amdgcn_rcpf(fmaf(a[j], t.x, 1.0f));
        acc[j] = fmaf(t.y * r0, r0, acc[j]);
        const float r1 = __builtin_amdgcn_rcpf(fmaf(a[j], t.z, 1.0f));
        acc[j] = fmaf(t.w * r1, r1, acc[j]);
      }
    }
  } else {
    for (int k = 0; k < n2; ++k) {
      const float4 t = T4[k];
#pragma unroll
      for (int j = 0; j < kSlots; ++j) {
        const float t0 = __builtin_amdgcn_exp2f(fminf(g.Lf * (a[j] - t.x), 126.0f));
        const float r0 = __builtin_amdgcn_rcpf(1.0f + t0);
        acc[j] = fmaf(t.y * (t0 * r0), r0, acc[j]);
        const float t1 = __builtin_amdgcn_exp2f(fminf(g.Lf * (a[j] - t.z), 126.0f));
        const float r1 = __builtin_amdgcn_rcpf(1.0f + t1);
        acc[j] = fmaf(t.w * (t1 * r1), r1, acc[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    if (id[j] < 0) continue;
    double h = (double)acc[j];
    if (g.factored) h *= (double)a[j];
    g.out[id[j]] = (float)(-(double)g.lambda * (double)wc[j] * h);
  }
}

// q = t / n and t - q n for 0 <= t < n + 64.
__device__ __forceinline__ int64_t div_near(int64_t t, int64_t n, int64_t* rem) {
  int64_t q;
  if (n > 64) {
    q = t >= n ? 1 : 0;
  } else {
    q = (int64_t)((unsigned)t / (unsigned)n);
  }
  *rem = t - q * n;
  return q;
}

template <bool D3>
__global__ __launch_bounds__(kGradNT) void soft_grad_kernel(GradArgs p, int64_t nseg) {
  extern __shared__ __align__(16) unsigned char smem[];
  {  // the grid of a batch that this workgroup row works on
    const int64_t b = blockIdx.y, nv = p.nz * p.ny * p.nx;
    p.grid += b * nv;
    p.out += b * nv;
    p.tau += b * p.tau_stride;
    p.grad_out += b * p.H;
  }
  QEntry* queues = reinterpret_cast<QEntry*>(smem);                     // kGradWaves x kQueueCap
  float2* T = reinterpret_cast<float2*>(queues + kGradWaves * kQueueCap);
  float* red = reinterpret_cast<float*>(smem);                          // setup only, 3 x kGradNT

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = p.H, Hp = (H + 1) & ~1;
  const float INF = __builtin_inff();

  // ---------------- threshold range, largest |g|: factored form or not
  {
    float lo = INF, hi = -INF, gm = 0.0f;
    for (int k = tid; k < H; k += kGradNT) {
      const float t = p.tau[k];
      lo = fminf(lo, t);
      hi = fmaxf(hi, t);
      gm = fmaxf(gm, fabsf(p.grad_out[k]));
    }
    red[tid] = lo;
    red[kGradNT + tid] = hi;
    red[2 * kGradNT + tid] = gm;
    __syncthreads();
    for (int off = kGradNT / 2; off > 0; off >>= 1) {
      if (tid < off) {
        red[tid] = fminf(red[tid], red[tid + off]);
        red[kGradNT + tid] = fmaxf(red[kGradNT + tid], red[kGradNT + tid + off]);
        red[2 * kGradNT + tid] = fmaxf(red[2 * kGradNT + tid], red[2 * kGradNT + tid + off]);
      }
      __syncthreads();
    }
  }
  const float tlo = red[0], thi = red[kGradNT], gmax = red[2 * kGradNT];
  GradCtx g;
  g.L64 = (double)p.lambda * 1.4426950408889634074;  // lambda * log2(e)
  g.cen = 0.5 * ((double)tlo + (double)thi);
  const double half_span = g.L64 * 0.5 * ((double)thi - (double)tlo);
  // E in [2^-100, 2^100] and |g E| <= 2^124; false for inf/NaN spans or gradients
  g.factored = (half_span >= 0.0) && (half_span <= 100.0) && (gmax <= 0x1p24f);
  g.Lf = (float)g.L64;
  g.lambda = p.lambda;
  g.out = p.out;
  g.T = T;
  g.Hp = Hp;
  for (int k = tid; k < Hp; k += kGradNT) {
    float2 e = make_float2(0.0f, 0.0f);
    if (k < H) {
      const float tk = p.tau[k], gk = p.grad_out[k];
      if (g.factored) {
        const float E = exp2_split(g.L64 * (g.cen - (double)tk));
        e = make_float2(E, gk * E);
      } else {
        e = make_float2(tk, gk);
      }
    }
    T[k] = e;
  }
  __syncthreads();

  // ---------------- segments of 64 voxels, one per wave at a time
  const float* grid = p.grid;
  const int64_t nz = p.nz, ny = p.ny, nx = p.nx;
  const int64_t plane = ny * nx, nvox = nz * plane;
  QEntry* q = queues + wave * kQueueCap;
  int count = 0;  // wave-uniform
  const int64_t wstride = (int64_t)gridDim.x * kGradWaves;
  // (z0, y0, x0) of the segment's first voxel, advanced by the grid stride
  // S = wstride * 64 voxels with a mixed-radix add (no division in the loop)
  int64_t seg = (int64_t)blockIdx.x * kGradWaves + wave;
  int64_t x0 = 0, y0 = 0, z0 = 0, sx = 0, sy = 0, sz = 0;
  if (seg < nseg) {
    const int64_t i0 = seg * 64, r0 = i0 / nx;
    x0 = i0 - r0 * nx;
    z0 = r0 / ny;
    y0 = r0 - z0 * ny;
    const int64_t S = wstride * 64, rs = S / nx;
    sx = S - rs * nx;
    sz = rs / ny;
    sy = rs - sz * ny;
  }
  for (; seg < nseg; seg += wstride) {
    const int64_t i0 = seg * 64;
    int64_t x, y;
    const int64_t qy = div_near(x0 + lane, nx, &x);
    const int64_t qz = div_near(y0 + qy, ny, &y);
    int64_t z = z0 + qz;
    const int64_t i = i0 + lane;
    const bool active = i < nvox;
    if (!active) x = y = z = 0;  // lanes past the end: every offset below is >= 0 and in the grid

    const bool xm = x > 0, xp = x + 1 < nx, ym = y > 0, yp = y + 1 < ny;
    const bool zm = D3 && z > 0, zp = D3 && z + 1 < nz;
    const int64_t ox[3] = {xm ? -1 : 0, 0, xp ? 1 : 0};
    const int64_t oy[3] = {ym ? -nx : 0, 0, yp ? nx : 0};
    const int64_t oz[3] = {zm ? -plane : 0, 0, zp ? plane : 0};
    const float* gp = grid + (active ? i : 0);
    const float pv = gp[0];
    uint32_t w = 0;
    constexpr int ZB = D3 ? 0 : 1, ZE = D3 ? 3 : 2;
#pragma unroll
    for (int dz = ZB; dz < ZE; ++dz)
#pragma unroll
      for (int dy = 0; dy < 3; ++dy)
#pragma unroll
        for (int dx = 0; dx < 3; ++dx) {
          const int b = (D3 ? 9 * dz : 0) + 3 * dy + dx;
          if (dz == 1 && dy == 1 && dx == 1) {
            w |= 1u << b;
            continue;
          }
          const float qv = gp[oz[dz] + oy[dy] + ox[dx]];
          const bool before = dz < 1 || (dz == 1 && (dy < 1 || (dy == 1 && dx < 1)));
          const bool ok = before ? (qv < pv) : (qv <= pv);
          w |= (uint32_t)ok << b;
        }
    // neighbours outside the grid: no cell through them exists
    if constexpr (D3) {
      if (!xm) w &= ~0x1249249u;
      if (!xp) w &= ~(0x1249249u << 2);
      if (!ym) w &= ~0x1C0E07u;
      if (!yp) w &= ~(0x1C0E07u << 6);
      if (!zm) w &= ~0x1FFu;
      if (!zp) w &= ~(0x1FFu << 18);
    } else {
      if (!xm) w &= ~0x49u;
      if (!xp) w &= ~(0x49u << 2);
      if (!ym) w &= ~0x7u;
      if (!yp) w &= ~(0x7u << 6);
    }
    const int c = active ? star_count<D3>(w) : 0;
    if (active && c == 0) p.out[i] = 0.0f;

    const bool push = c != 0;
    const uint64_t bal = __ballot(push);
    if (push) {
      const int pos = count + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
      QEntry e;
      e.v = pv;
      e.c = c;
      e.idx = i;
      q[pos] = e;
    }
    count += __popcll(bal);
    if (count >= kBatch) {
      wave_lds_sync();
      sweep(g, q + (count - kBatch), kBatch, lane);
      count -= kBatch;
      wave_lds_sync();
    }
    x0 += sx;
    y0 += sy;
    if (x0 >= nx) {
      x0 -= nx;
      ++y0;
    }
    z0 += sz;
    if (y0 >= ny) {
      y0 -= ny;
      ++z0;
    }
  }
  if (count > 0) {
    wave_lds_sync();
    sweep(g, q, count, lane);
  }
}

template <bool D3>
hipError_t launch_grad(const GradArgs& a, hipStream_t s, int64_t nseg, const DeviceInfo& di) {
  auto k = soft_grad_kernel<D3>;
  const size_t lds = (size_t)kGradWaves * kQueueCap * sizeof(QEntry) + (size_t)((a.H + 1) & ~1) * sizeof(float2);
  hipError_t e;
  if (lds > 64 * 1024) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k), kGradNT, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  // workgroups per grid: the launch's share of what fits on the chip
  int64_t g = ((int64_t)di.cus * per_cu + a.batch - 1) / a.batch;
  const int64_t need = (nseg + kGradWaves - 1) / kGradWaves;
  if (g > need) g = need;
  if (g < 1) g = 1;
  const int64_t nvox = a.nz * a.ny * a.nx;
  for (int64_t b0 = 0; b0 < a.batch; b0 += kMaxBatchPerLaunch) {
    const int64_t nb = a.batch - b0 < kMaxBatchPerLaunch ? a.batch - b0 : kMaxBatchPerLaunch;
    GradArgs c = a;
    c.grid = a.grid + b0 * nvox;
    c.out = a.out + b0 * nvox;
    c.tau = a.tau + b0 * a.tau_stride;
    c.grad_out = a.grad_out + b0 * a.H;
    hipLaunchKernelGGL(k, dim3((unsigned)g, (unsigned)nb), dim3(kGradNT), lds, s, c, nseg);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_soft_grad(const GradArgs& a, hipStream_t s) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  const int64_t nvox = a.nz * a.ny * a.nx;
  const int64_t nseg = (nvox + 63) / 64;
  return a.nz > 1 ? launch_grad<true>(a, s, nseg, di) : launch_grad<false>(a, s, nseg, di);
}

}  // namespace ecc
