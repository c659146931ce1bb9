// Soft (sigmoid-relaxed) Euler characteristic curve and its threshold
// gradient, gfx950.
//
// Method: page "Scalable GPU-Accelerated Euler Characteristic Curves"
// (paper notes), "Method / Key designs / differentiable ECC layer": the hard
// indicator of value <= tau becomes sigmoid(lambda (tau - value)), giving
//     S_k   = sum_c (-1)^dim(c) s(lambda (tau_k - v_c)),
//     dS/dtau_k = lambda sum_c (-1)^dim(c) s(x)(1 - s(x)),
// evaluated by custom forward / backward kernels.  Cells and values are those
// of the hard curve (max of corners, V-construction).
//
// Work split (cells x thresholds).  Each workgroup takes tiles of 512 voxels.
// Phase A turns a tile into a short list of (value, weight) terms: the same
// exact regrouping as the hard kernels (four row sequences per voxel,
// telescoped along x, equal values merged), so a term carries the summed sign
// of every cell that has that value.  Phase B sweeps the list in LDS against
// the thresholds: every wave takes a quarter of the terms, two at a time
// (one per half-wave), and every lane owns 8 thresholds of each
// 256-threshold chunk, so one broadcast LDS read of a term feeds 8 sigmoids
// per lane and the sweep's LDS traffic stays well below its VALU work.
// Tiles of 512 voxels and 8 thresholds per lane keep LDS and registers at
// 7 workgroups per CU, enough waves to hide the latency of the sweep.  The
// sigmoid costs one FMA and one
// reciprocal per (term, threshold) in the factored form
//     exp(lambda (v - tau)) = 2^{L (v - c)} * 2^{L (c - tau)},  L = lambda log2 e,
// with the first factor computed once per term and the second once per
// threshold (c is the middle of the threshold range; used when both factors
// stay inside the float range, else every pair takes exp2 directly).
// Sums are float64 per lane and per workgroup (LDS); workgroups combine in
// 64-bit fixed point, so the result is independent of scheduling.

#include <hip/hip_runtime.h>
#include <math.h>

#include "ecc_device.hpp"
#include "ecc_internal.hpp"

namespace ecc {
namespace {

constexpr int kTileVox = 512;           // voxels per tile
constexpr int kTermCap = 4 * kTileVox;  // at most 4 terms per voxel
constexpr int kChunk = 256;             // thresholds per sweep chunk
constexpr int kLaneGroups = 2;          // terms a wave sweeps at once
constexpr int kGroupLanes = 64 / kLaneGroups;
constexpr int kSlots = kChunk / kGroupLanes;  // thresholds per lane and chunk

__device__ void batch_sum(const SoftArgs& p, const long long* tot, double inv, int* flag);

struct Term {
  float a;  // F = 2^{L (v - c)} (factored) or the value v (direct)
  float w;  // summed sign
};

template <bool BWD>
__global__ __launch_bounds__(kBlock) void soft_kernel(SoftArgs p, int64_t ntiles, int fx_shift) {
  extern __shared__ __align__(16) unsigned char smem[];
  {  // the grid of a batch that this workgroup row works on
    const int64_t b = blockIdx.y;
    p.grid += b * (p.nz * p.ny * p.nx);
    p.tau += b * p.tau_stride;
    if (p.sum_batch == 0) p.out += b * p.H;
    if (BWD) p.grad_out += b * p.H;
    p.ws = reinterpret_cast<char*>(p.ws) + (size_t)b * p.ws_stride;
  }
  long long* tmp = reinterpret_cast<long long*>(smem);                 // 256
  int* misc = reinterpret_cast<int*>(tmp + kBlock);                    // [0]=count [1]=flag
  Term* terms = reinterpret_cast<Term*>(misc + 4);                     // kTermCap
  double* accS = reinterpret_cast<double*>(terms + kTermCap);          // H

  const int H = p.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* grid = p.grid;
  const int64_t nz = p.nz, ny = p.ny, nx = p.nx;
  const int64_t plane = ny * nx, nvox = nz * plane;
  const float INF = __builtin_inff();

  for (int k = tid; k < H; k += kBlock) accS[k] = 0.0;
  if (tid == 0) misc[0] = 0;

  // threshold range -> mode and centre
  float* ftmp = reinterpret_cast<float*>(tmp);
  {
    float lo = INF, hi = -INF;
    for (int k = tid; k < H; k += kBlock) {
      const float t = p.tau[k];
      lo = fminf(lo, t);
      hi = fmaxf(hi, t);
    }
    ftmp[tid] = lo;
    ftmp[kBlock + tid] = hi;
    __syncthreads();
    for (int off = kBlock / 2; off > 0; off >>= 1) {
      if (tid < off) {
        ftmp[tid] = fminf(ftmp[tid], ftmp[tid + off]);
        ftmp[kBlock + tid] = fmaxf(ftmp[kBlock + tid], ftmp[kBlock + tid + off]);
      }
      __syncthreads();
    }
  }
  const float tlo = ftmp[0], thi = ftmp[kBlock];
  const double L64 = (double)p.lambda * 1.4426950408889634074;  // lambda * log2(e)
  const double cen = 0.5 * ((double)tlo + (double)thi);
  const double half_span = L64 * 0.5 * ((double)thi - (double)tlo);
  // factored form needs 2^{L(c - tau)} inside [2^-100, 2^100] for every tau
  const bool factored = (half_span >= 0.0) && (half_span <= 100.0);  // false for inf/NaN spans
  const float Lf = (float)L64;
  __syncthreads();

  const int nchunks = (H + kChunk - 1) / kChunk;

  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    // ---------------- phase A: terms of this tile
    const int64_t base = t * kTileVox;
#pragma unroll 1
    for (int j = 0; j < kTileVox / kBlock; ++j) {
      const int64_t i = base + j * kBlock + tid;
      float sv[4] = {INF, INF, INF, INF};
      int wv[4] = {0, 0, 0, 0};
      if (i < nvox) {
        const int64_t x = i % nx;
        const int64_t yz = i / nx;
        const int64_t y = yz % ny, z = yz / ny;
        const bool y1 = y + 1 < ny, z1 = z + 1 < nz;
        // f[dz][dy][dx+1] for dx in {-1,0,1}
        float f[2][2][3];
#pragma unroll
        for (int dz = 0; dz < 2; ++dz)
#pragma unroll
          for (int dy = 0; dy < 2; ++dy)
#pragma unroll
            for (int dx = -1; dx <= 1; ++dx) {
              const bool in = (dz == 0 || z1) && (dy == 0 || y1) && (x + dx >= 0) && (x + dx < nx);
              f[dz][dy][dx + 1] = in ? grid[i + dz * plane + dy * nx + dx] : INF;
            }
        float s[4][3];
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          s[0][q] = f[0][0][q];
          s[1][q] = fmaxf(f[0][0][q], f[0][1][q]);
          s[2][q] = fmaxf(f[0][0][q], f[1][0][q]);
          s[3][q] = fmaxf(s[1][q], fmaxf(f[1][0][q], f[1][1][q]));
        }
        int w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = (int)(s[q][2] > s[q][1]) - (int)(s[q][1] > s[q][0]);
        w[1] = -w[1];
        w[2] = -w[2];
        const float v0 = s[0][1], v1 = s[1][1], v2 = s[2][1], v3 = s[3][1];
        if (v3 == v2) { w[2] += w[3]; w[3] = 0; }
        else if (v3 == v1) { w[1] += w[3]; w[3] = 0; }
        if (v2 == v1) { w[1] += w[2]; w[2] = 0; }
        if (v1 == v0) { w[0] += w[1]; w[1] = 0; }
        if (v2 == v0) { w[0] += w[2]; w[2] = 0; }
        sv[0] = v0; sv[1] = v1; sv[2] = v2; sv[3] = v3;
#pragma unroll
        for (int q = 0; q < 4; ++q) wv[q] = (sv[q] < INF) ? w[q] : 0;
      }
      int cnt = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) cnt += (wv[q] != 0);
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      const int total = __shfl(incl, 63);
      int wbase = 0;
      if (lane == 63 && total) wbase = atomicAdd(&misc[0], total);
      wbase = __shfl(wbase, 63);
      int pos = wbase + incl - cnt;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (wv[q] != 0) {
          Term tm;
          // F is kept finite so that F * E overflowing to inf only ever meets a 0 reciprocal
          tm.a = factored ? fminf(exp2_split(L64 * ((double)sv[q] - cen)), 0x1p126f) : sv[q];
          tm.w = (float)wv[q];
          terms[pos++] = tm;
        }
      }
    }
    __syncthreads();
    const int n = misc[0];

    // ---------------- phase B: sweep terms x thresholds
    // A wave works on kLaneGroups terms at once, one per group of
    // kGroupLanes lanes; a lane owns kSlots thresholds of the chunk, so each
    // broadcast read of a term serves kSlots sigmoids per lane.
    const int tb = (int)(((int64_t)n * wave) / kWavesPerBlock);
    const int te = (int)(((int64_t)n * (wave + 1)) / kWavesPerBlock);
    const int grp = lane / kGroupLanes, gl = lane % kGroupLanes;
    for (int c = 0; c < nchunks; ++c) {
      float e[kSlots];
      bool valid[kSlots];
#pragma unroll
      for (int r = 0; r < kSlots; ++r) {
        const int k = c * kChunk + r * kGroupLanes + gl;
        valid[r] = k < H;
        const float tk = valid[r] ? p.tau[k] : 0.0f;
        e[r] = factored ? (valid[r] ? exp2_split(L64 * (cen - (double)tk)) : 0.0f) : tk;
      }
      double acc[kSlots];
#pragma unroll
      for (int r = 0; r < kSlots; ++r) acc[r] = 0.0;
      // groups past the wave's last term take its first one with weight 0
      auto term = [&](int base) {
        const int ti = base + grp;
        Term tm = terms[ti < te ? ti : tb];
        if (ti >= te) tm.w = 0.0f;
        return tm;
      };
      if (factored) {
        for (int base = tb; base < te; base += kLaneGroups) {
          const Term tm = term(base);
          const double wd = (double)tm.w;
          const double wfd = wd * (double)tm.a;  // w F, once per term
#pragma unroll
          for (int r = 0; r < kSlots; ++r) {
            const float d = fmaf(tm.a, e[r], 1.0f);
            const float rr = __builtin_amdgcn_rcpf(d);
            if constexpr (!BWD) {
              acc[r] = fma(wd, (double)rr, acc[r]);
            } else {
              // w s (1 - s) = w t s^2 = (w F) (E s) s, t = F E
              const float q = (e[r] * rr) * rr;
              acc[r] = fma(wfd, (double)q, acc[r]);
            }
          }
        }
      } else {
        for (int base = tb; base < te; base += kLaneGroups) {
          const Term tm = term(base);
          const double wd = (double)tm.w;
#pragma unroll
          for (int r = 0; r < kSlots; ++r) {
            const float x = fminf(Lf * (tm.a - e[r]), 126.0f);  // L (v - tau), kept finite
            const float tt = __builtin_amdgcn_exp2f(x);
            const float rr = __builtin_amdgcn_rcpf(1.0f + tt);
            if constexpr (!BWD) {
              acc[r] = fma(wd, (double)rr, acc[r]);
            } else {
              const float q = (tt * rr) * rr;
              acc[r] = fma(wd, (double)q, acc[r]);
            }
          }
        }
      }
      // this wave's two lane groups, then the waves one after another: a
      // fixed order of additions, so the sums do not depend on scheduling
#pragma unroll
      for (int r = 0; r < kSlots; ++r) acc[r] += __shfl_down(acc[r], kGroupLanes);
      for (int w = 0; w < kWavesPerBlock; ++w) {
        if (wave == w && grp == 0) {
#pragma unroll
          for (int r = 0; r < kSlots; ++r)
            if (valid[r]) accS[c * kChunk + r * kGroupLanes + gl] += acc[r];
        }
        __syncthreads();
      }
    }
    __syncthreads();
    if (tid == 0) misc[0] = 0;
    __syncthreads();
  }

  // ---------------- combine workgroups in 64-bit fixed point (order-free)
  __syncthreads();
  const double scale = ldexp(1.0, fx_shift);
  long long* tot = reinterpret_cast<long long*>(terms);  // the term list is no longer needed
  if (!grid_reduce(p.ws, H, H, [&](int k) { return __double2ll_rn(accS[k] * scale); }, tot, &misc[1],
                   p.acc_copies))
    return;
  const double inv = ldexp(1.0, -fx_shift);
  if (!BWD || p.sum_batch == 0) {
    for (int k = tid; k < H; k += kBlock) {
      double v = (double)tot[k] * inv;
      if constexpr (BWD) v *= (double)p.lambda * (double)p.grad_out[k];
      p.out[k] = (float)v;
    }
    return;
  }
  if constexpr (BWD) batch_sum(p, tot, inv, &misc[1]);
}

// The shared-threshold gradient summed over the batch, in a fixed order.
// The last workgroup of grid b leaves its float64 values in the accumulator
// slots of its own workspace slice (grid_reduce has just cleared them).  Grids
// form groups of kSumGroup; the last grid of a group to finish (ticket in the
// header of the group's first slice) sums the group's slots in grid order into
// the group's first slot and clears the others; the last group (ticket in
// grid 0's header) sums the group totals in order, writes out and clears
// them, so the workspace is zero again.  Tickets and slots use device-scope
// atomics, ordered as in grid_reduce.
__device__ void batch_sum(const SoftArgs& p, const long long* tot, double inv, int* flag) {
  const int tid = threadIdx.x, H = p.H;
  const int64_t B = p.sum_batch, bg = p.b_first + blockIdx.y;
  char* const base = reinterpret_cast<char*>(p.ws_base);
  auto slot = [&](int64_t b) { return reinterpret_cast<double*>(base + (size_t)b * p.ws_stride + kWsHeader); };
  auto ticket = [&](int64_t b, int i) { return reinterpret_cast<unsigned int*>(base + (size_t)b * p.ws_stride) + i; };
  auto last_of = [&](unsigned int* t, int64_t n) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const unsigned int prev = __hip_atomic_fetch_add(t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = prev == (unsigned int)(n - 1);
      if (last) __hip_atomic_store(t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *flag = last;
    }
    __syncthreads();
    return *flag != 0;
  };
  // in-order sum of `n` slots starting at grid b0, stride `step` grids
  auto ordered_sum = [&](int64_t b0, int64_t n, int64_t step, int k) {
    double s = 0.0;
    int64_t i = 0;
    for (; i + 8 <= n; i += 8) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = agent_load(slot(b0 + (i + u) * step) + k);
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; i < n; ++i) s += agent_load(slot(b0 + i * step) + k);
    return s;
  };
  __syncthreads();
  double* mine = slot(bg);
  for (int k = tid; k < H; k += kBlock)
    agent_store(mine + k, (double)tot[k] * inv * (double)p.lambda * (double)p.grad_out[k]);
  const int64_t g0 = bg - bg % kSumGroup;
  const int64_t ng = B - g0 < kSumGroup ? B - g0 : kSumGroup;
  if (!last_of(ticket(g0, 1), ng)) return;
  for (int k = tid; k < H; k += kBlock) {
    const double s = ordered_sum(g0, ng, 1, k);
    agent_store(slot(g0) + k, s);
    for (int64_t b = g0 + 1; b < g0 + ng; ++b) agent_store(slot(b) + k, 0.0);
  }
  const int64_t ngroups = (B + kSumGroup - 1) / kSumGroup;
  if (!last_of(ticket(0, 2), ngroups)) return;
  for (int k = tid; k < H; k += kBlock) {
    p.out[k] = (float)ordered_sum(0, ngroups, kSumGroup, k);
    for (int64_t j = 0; j < ngroups; ++j) agent_store(slot(j * kSumGroup) + k, 0.0);
  }
}

}  // namespace

hipError_t launch_soft(const SoftArgs& a, hipStream_t s) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  const int64_t nvox = a.nz * a.ny * a.nx;
  const int64_t ntiles = (nvox + kTileVox - 1) / kTileVox;
  // workgroups per grid: the launch's share of 64 per CU.  Far more than fit
  // at once (7 per CU): tiles differ in how many terms they hold, and short
  // workgroups that the dispatcher keeps replacing balance the CUs better
  // than a few persistent ones (256^3: 64 per CU is 11 % faster than 4).
  int64_t g = ((int64_t)di.cus * 64 + a.batch - 1) / a.batch;
  if (g > ntiles) g = ntiles;
  if (g < 1) g = 1;
  // fixed point: |partial| and |total| <= #cells <= 8 * nvox, kept below 2^61;
  // the finest resolution that allows (small grids get more fraction bits:
  // the backward scales the sum by lambda g_k, and so its quantization)
  int bits = 0;
  while (bits < 62 && (((int64_t)1) << bits) < 8 * nvox + 8) ++bits;
  const int shift = 61 - bits;
  const size_t lds = kBlock * sizeof(long long) + 4 * sizeof(int) + kTermCap * sizeof(Term) +
                     (size_t)a.H * sizeof(double);
  auto k = a.grad_out ? soft_kernel<true> : soft_kernel<false>;
  if (lds > 64 * 1024) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds);
    if (e != hipSuccess) return e;
  }
  // one launch per run of at most kMaxBatchPerLaunch grids
  for (int64_t b0 = 0; b0 < a.batch; b0 += kMaxBatchPerLaunch) {
    const int64_t nb = a.batch - b0 < kMaxBatchPerLaunch ? a.batch - b0 : kMaxBatchPerLaunch;
    SoftArgs c = a;
    c.grid = a.grid + b0 * nvox;
    c.tau = a.tau + b0 * a.tau_stride;
    c.out = a.out + b0 * a.H;
    if (a.grad_out) c.grad_out = a.grad_out + b0 * a.H;
    c.ws = reinterpret_cast<char*>(a.ws) + (size_t)b0 * a.ws_stride;
    if (a.sum_batch) {
      c.out = a.out;
      c.ws_base = a.ws;
      c.b_first = b0;
    }
    hipLaunchKernelGGL(k, dim3((unsigned)g, (unsigned)nb), dim3(kBlock), lds, s, c, ntiles, shift);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ecc
