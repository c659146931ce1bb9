// Device-side building blocks shared by the hard and soft ECC kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ecc_internal.hpp"

namespace ecc {

// ---------------------------------------------------------------- exp2
// 2^a for |a| well inside the float range, accurate to ~1 ulp: split off the
// integer part in float64 so the float exp2 only sees [0, 1).
__device__ __forceinline__ float exp2_split(double a) {
  a = fmin(fmax(a, -300.0), 300.0);
  const double n = floor(a);
  const float f = (float)(a - n);
  return ldexpf(exp2f(f), (int)n);
}

// ---------------------------------------------------------------- atomics
__device__ __forceinline__ long long agent_load(const long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void agent_store(long long* p, long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ double agent_load(const double* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void agent_store(double* p, double v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Launches of at most this many workgroups per grid take one flat ticket
// (callers may raise it: see flush_and_finish).
constexpr unsigned int kFlatTicketMax = 64;

// Grid-wide reduction of per-workgroup rows of n int64 values, one launch.
//
// Every workgroup adds its non-zero values into one of `copies` int64
// accumulator rows with device-scope atomic adds, waits until all of its own
// memory operations are acknowledged, and only then takes a ticket.  On this
// GPU, device-scope atomics are performed at the point of coherence shared by
// all XCDs and a wave's vmcnt reaches zero only once they are, so a workgroup
// that draws the last ticket can read every other workgroup's contribution
// with device-scope atomic loads.  This replaces agent-scope fences, which
// write back and invalidate the issuing XCD's L2 and cost far more than the
// reduction itself when every workgroup issues them.  The last workgroup
// returns true with the totals in `tot` (LDS, n entries) and leaves the
// accumulators and the tickets zero for the next launch.  Integer addition is
// associative, so the totals do not depend on the order of arrival.
template <int NT = kBlock, typename Local>
__device__ bool grid_reduce(void* ws, int H, int n, Local local, long long* tot, int* lds_flag,
                            int copies = kAccCopies, unsigned int flat_max = kFlatTicketMax) {
  if (gridDim.x == 1) {  // a lone workgroup holds the totals already (tot must not alias local's data)
    for (int b = threadIdx.x; b < n; b += NT) tot[b] = local(b);
    __syncthreads();
    return true;
  }
  unsigned int* ticket = reinterpret_cast<unsigned int*>(ws);
  long long* acc = reinterpret_cast<long long*>(reinterpret_cast<char*>(ws) + kWsHeader);
  const int stride = acc_bins(H);
  long long* mine = acc + (size_t)(blockIdx.x % copies) * stride;
  for (int b = threadIdx.x; b < n; b += NT) {
    const long long v = local(b);
    if (v != 0) __hip_atomic_fetch_add(mine + b, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's atomics are acknowledged
  __syncthreads();                // ... and every other wave's of this workgroup
  if (threadIdx.x == 0) {
    int last = 0;
    if (copies == kAccCopies && gridDim.x > flat_max) {
      // Two-level ticket.  Atomics on one address are performed one after
      // another at the point of coherence, and when all workgroups finish
      // together a single ticket queues them all.  Workgroups count into
      // one of at most kTicketGroups group tickets (each on its own line);
      // the last of a group, having seen every member's increment (and so
      // every member's accumulator adds performed), counts into the main
      // ticket, whose last taker holds every contribution.
      unsigned int* groups =
          reinterpret_cast<unsigned int*>(reinterpret_cast<char*>(acc) + (size_t)copies * stride * sizeof(long long));
      const unsigned int gs = (gridDim.x + kTicketGroups - 1) / kTicketGroups;
      const unsigned int ng = (gridDim.x + gs - 1) / gs;
      const unsigned int g = blockIdx.x / gs;
      const unsigned int gsize = min(gs, gridDim.x - g * gs);
      unsigned int* gt = groups + (size_t)g * (kTicketLine / sizeof(unsigned int));
      const unsigned int p = __hip_atomic_fetch_add(gt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (p == gsize - 1) {
        __hip_atomic_store(gt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned int q = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = (q == ng - 1);
      }
    } else {
      const unsigned int prev = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = (prev == gridDim.x - 1);
    }
    if (last) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = last;
  }
  __syncthreads();
  if (!*lds_flag) return false;
  for (int b = threadIdx.x; b < n; b += NT) {
    long long s = 0;
#pragma unroll
    for (int c = 0; c < copies; ++c) s += agent_load(acc + (size_t)c * stride + b);
    tot[b] = s;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < copies * stride; i += NT) agent_store(acc + i, 0LL);
  return true;
}

// --------------------------------------------------------- block scans
// Inclusive scan of n values with NT threads, each thread owning one
// contiguous segment.  `get(i)` produces element i (called twice per
// element), `put(i, v)` receives the inclusive scan.  `tmp` holds NT T.
// `op` must be associative (integer adds, fmaxf).  256-thread workgroups scan
// the segment totals within each wave by lane shuffles, then across the four
// waves (two barriers).  512-thread workgroups (the 3D float kernel, which
// sits at its 128-register limit: the shuffle form makes it spill) scan
// them in LDS, two barriers per doubling step.
template <typename T, int NT = kBlock, typename Op, typename Get, typename Put>
__device__ void block_scan(int n, T identity, Op op, Get get, Put put, T* tmp) {
  const int t = threadIdx.x;
  const int seg = (n + NT - 1) / NT;
  const int b = t * seg;
  const int e = min(b + seg, n);
  T s = identity;
  for (int i = b; i < e; ++i) s = op(s, get(i));
  T run = identity;
  if constexpr (NT <= 256) {
    const int lane = t & 63, w = t >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const T v = __shfl_up(s, off);
      if (lane >= off) s = op(v, s);
    }
    if (lane == 63) tmp[w] = s;
    const T below = __shfl_up(s, 1);  // the scan over the lanes below this one
    __syncthreads();
    for (int j = 0; j < w; ++j) run = op(run, tmp[j]);
    if (lane > 0) run = op(run, below);
  } else {
    tmp[t] = s;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
      T v = t >= off ? tmp[t - off] : identity;
      __syncthreads();
      tmp[t] = op(tmp[t], v);
      __syncthreads();
    }
    if (t) run = tmp[t - 1];
  }
  for (int i = b; i < e; ++i) {
    run = op(run, get(i));
    put(i, run);
  }
  __syncthreads();
}

// Running maximum of the thresholds: R_k = max(tau_0..tau_k) with fmaxf, so a
// NaN threshold never admits a value.  min{k : v <= tau_k} equals
// min{k : v <= R_k}, and R is non-decreasing, which makes binning a search.
template <int NT = kBlock>
__device__ __forceinline__ void running_max_to_lds(const float* tau, int H, float* R, float* tmp) {
  block_scan<float, NT>(
      H, -__builtin_inff(), [](float a, float b) { return fmaxf(a, b); },
      [&](int i) { return tau[i]; }, [&](int i, float v) { R[i] = v; }, tmp);
}

// First k with v <= R[k] (R non-decreasing, in LDS), or H.  Exact fp32
// comparisons; the linear guess only picks the starting point.
__device__ __forceinline__ int bin_of(float v, const float* R, int H, float r0, float scale) {
  float g = (v - r0) * scale;
  g = fminf(fmaxf(g, 0.0f), (float)(H - 1));  // NaN guess -> 0
  int k = (int)g;
#pragma unroll
  for (int s = 0; s < 2; ++s)
    if (k > 0 && !(R[k - 1] < v)) --k;
#pragma unroll
  for (int s = 0; s < 2; ++s)
    if (k < H && !(v <= R[k])) ++k;
  const bool ok = (k == 0 || R[k - 1] < v) && (k == H || v <= R[k]);
  if (!ok) {
    int lo = 0, hi = H;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (v <= R[mid]) hi = mid; else lo = mid + 1;
    }
    k = lo;
  }
  return k;
}

// Linear-guess parameters for bin_of, from the running max in LDS.
__device__ __forceinline__ void guess_params(const float* R, int H, float* r0, float* scale) {
  const float a = R[0], b = R[H - 1];
  float s = 0.0f;
  if (H > 1) {
    const float span = b - a;
    if (span > 0.0f && span < __builtin_inff()) s = (float)(H - 1) / span;
  }
  if (!(s < __builtin_inff())) s = 0.0f;
  *r0 = a;
  *scale = s;
}

}  // namespace ecc
