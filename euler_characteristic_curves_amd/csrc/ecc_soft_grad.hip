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
// Where the factors would leave the float range (a threshold span much wider
// than 1 / lambda) every pair takes exp2 directly.
//
// Accuracy.  Terms are float32, summed in float32 over 8 thresholds and in
// float64 beyond.  The table holds the thresholds with g_k > 0 first and
// those with g_k < 0 after (g_k = 0 adds nothing and is left out), so the two
// partial sums give both h and m = sum_k |g_k| s(1 - s), the scale of the
// rounding error: every term is within a few float32 units of itself, so the
// error of h is below K u m (u = 2^-24; K derived at kFactoredK / kDirectK).
// Where h cancels (upstream gradients of both signs that are large, or a
// large lambda |c(p)|) that bound can exceed the accuracy the soft outputs
// are held to; such voxels are recomputed term by term in float64 from the
// defining formula, so every output is within kAbsTarget or kRelTarget of
// the exact value.  Upstream gradients enter the table scaled by a power of
// two, which is exact and keeps g_k E_k inside the float range.

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
constexpr int kBlk = 8;                    // thresholds per float32 partial sum
constexpr int kTablePad = 2 * kBlk;        // table entries beyond H (segment padding)

// Every output is within max(kAbsTarget, kRelTarget |exact|) of the exact
// value: 90 % of the soft tolerance (1e-3 absolute, 1e-4 relative), leaving
// the rest for the final rounding to float (below 6e-8 relative).
constexpr double kAbsTarget = 9e-4;
constexpr double kRelTarget = 9e-5;
constexpr double kU = 0x1p-24;  // float32 unit roundoff
// Factored terms gs E r r (r = 1 / (1 + F E), F applied in float64 after the
// sum).  E and F are float64 exp2 values rounded to float (u each); gs E and
// (gs E) r are rounded once each (u, u); 1 + F E is one FMA (u) and r one
// reciprocal (2 u).  With t = F E, a relative error e in F or E moves
// E r^2 F by e (1 - t) / (1 + t), at most e, so a term is within
// u + u + u + u + 2 (u + 2 u) = 10 u of itself; the float32 sum of 8
// same-signed terms adds 8 u of their sum: 18 u, taken as 20.
constexpr double kFactoredK = 20.0 * kU;
constexpr int kRefCap = 64;   // per-wave list of voxels for the float64 path
// Direct terms: the exponent x = L (v - tau) is three float32 roundings away
// from exact (3 u |x| in log2 units, 2.08 u |x| relative after exp2), then
// exp2 (2 u), 1 + t, the reciprocal and three multiplies: 2.08 u |x| + 11 u
// per term, + 8 u for the partial sums.  The bound K u m + Kx u sum |term| |x|
// with K = 24, Kx = 4.
constexpr double kDirectK = 24.0 * kU;
constexpr double kDirectKx = 4.0 * kU;

struct QEntry {
  float v;        // X(p)
  int c;          // c(p), non-zero
  long long idx;  // linear voxel index
};

struct GradCtx {
  // per threshold: (E_k, gs_k E_k) factored, (tau_k, gs_k) direct, gs = g / 2^s;
  // [0, nP): g > 0, [nP, nP + nN): g < 0, each padded with (0, 0) to kBlk
  const float2* T;
  int nP, nN;
  bool factored;
  double L64, cen;
  float Lf;
  double lam64;
  double gscale;  // 2^s
  double ginv;    // factored: sum_k |gs_k| / E_k
  double g1;      // sum_k |gs_k|
  const float* tau;   // the raw thresholds and upstream gradient (float64 path)
  const float* gout;
  int H;
  float* out;
};

// Wave-uniform copies (values read from LDS are uniform but would otherwise
// stay in vector registers for the whole kernel).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uni(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}
__device__ __forceinline__ double uni(double x) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_readfirstlane((int)(b & 0xffffffffLL));
  const int hi = __builtin_amdgcn_readfirstlane((int)(b >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Orders this wave's LDS accesses around it (queue writes by some lanes are
// read by other lanes of the same wave).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Table entries [k0, k1) (float4 units, 2 thresholds each, k1 - k0 a multiple
// of kBlk / 2), factored form: acc[j] += F-free sum of gs E r^2.
__device__ __forceinline__ void seg_factored(const float4* T4, int k0, int k1, const float* a, double* acc) {
  for (int k = k0; k < k1; k += kBlk / 2) {
    float blk[kSlots] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < kBlk / 2; ++u) {
      const float4 t = T4[k + u];
#pragma unroll
      for (int j = 0; j < kSlots; ++j) {
        const float r0 = __builtin_amdgcn_rcpf(fmaf(a[j], t.x, 1.0f));
        blk[j] = fmaf(t.y * r0, r0, blk[j]);
        const float r1 = __builtin_amdgcn_rcpf(fmaf(a[j], t.z, 1.0f));
        blk[j] = fmaf(t.w * r1, r1, blk[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < kSlots; ++j) acc[j] += (double)blk[j];
  }
}

// The same with exp2 per pair (a = v); mw[j] += |term| |x|, x the exponent.
__device__ __forceinline__ void seg_direct(const float4* T4, int k0, int k1, float Lf, const float* a,
                                           double* acc, float* mw) {
  for (int k = k0; k < k1; k += kBlk / 2) {
    float blk[kSlots] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < kBlk / 2; ++u) {
      const float4 t = T4[k + u];
#pragma unroll
      for (int j = 0; j < kSlots; ++j) {
        const float x0 = fmaxf(fminf(Lf * (a[j] - t.x), 126.0f), -150.0f);
        const float e0 = __builtin_amdgcn_exp2f(x0);
        const float r0 = __builtin_amdgcn_rcpf(1.0f + e0);
        const float s0 = (t.y * (e0 * r0)) * r0;
        blk[j] += s0;
        mw[j] = fmaf(fabsf(s0), fabsf(x0), mw[j]);
        const float x1 = fmaxf(fminf(Lf * (a[j] - t.z), 126.0f), -150.0f);
        const float e1 = __builtin_amdgcn_exp2f(x1);
        const float r1 = __builtin_amdgcn_rcpf(1.0f + e1);
        const float s1 = (t.w * (e1 * r1)) * r1;
        blk[j] += s1;
        mw[j] = fmaf(fabsf(s1), fabsf(x1), mw[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < kSlots; ++j) acc[j] += (double)blk[j];
  }
}

// h(v) term by term in float64, sum_k g_k e / (1 + e)^2 with
// e = exp(-|lambda (tau_k - v)|), for the m (wave-uniform) voxels listed in
// R: the wave takes one voxel at a time, lane l summing thresholds l, l + 64,
// ..., then a fixed-order butterfly (lane 0's total is written, so the
// result does not depend on scheduling).
__device__ __forceinline__ void refine_list(const GradCtx& g, const QEntry* R, int m, int lane) {
  for (int i = 0; i < m; ++i) {
    const QEntry e = R[i];
    const double vd = e.v;
    double h = 0.0;
    for (int k = lane; k < g.H; k += 64) {
      const double x = exp(-fabs(g.lam64 * ((double)g.tau[k] - vd)));
      const double r = 1.0 / (1.0 + x);
      h += (double)g.gout[k] * (x * r * r);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) h += __shfl_xor(h, off);
    if (lane == 0) g.out[e.idx] = (float)(-g.lam64 * (double)e.c * h);
  }
}

// Phase B: sum h over all thresholds for queue entries q[0..n) (n <= kBatch),
// lane l taking entries l, l + 64, l + 128, l + 192; write the gradients, or
// list the voxel in R for the float64 path (done before the next slot).
__device__ __forceinline__ void sweep(const GradCtx& g, const QEntry* q, int n, int lane, QEntry* R) {
  int rcount = 0;  // wave-uniform
  float a[kSlots];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int e = lane + 64 * j;
    const float v = q[e < n ? e : 0].v;
    // F rounded from float64 and kept finite, so F E overflowing to inf only
    // ever meets a 0 reciprocal (voxels with F > 2^126 are handled apart)
    a[j] = g.factored ? (float)fmin(exp2(g.L64 * ((double)v - g.cen)), 0x1p126) : v;
  }
  double accP[kSlots] = {0.0, 0.0, 0.0, 0.0};
  double accN[kSlots] = {0.0, 0.0, 0.0, 0.0};
  float mw[kSlots] = {0.0f, 0.0f, 0.0f, 0.0f};
  const float4* T4 = reinterpret_cast<const float4*>(g.T);
  const int eP = g.nP >> 1, eN = (g.nP + g.nN) >> 1;
  if (g.factored) {
    seg_factored(T4, 0, eP, a, accP);
    seg_factored(T4, eP, eN, a, accN);
  } else {
    seg_direct(T4, 0, eP, g.Lf, a, accP, mw);
    seg_direct(T4, eP, eN, g.Lf, a, accN, mw);
  }
  // the queue entries are still in place: reload them rather than hold them
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int e = lane + 64 * j;
    bool need = false;
    QEntry qe;
    if (e < n) {
      qe = q[e];
      const double lc = g.lam64 * fabs((double)qe.c);  // lambda |c(p)|
      double h, err;
      if (g.factored) {
        const double aF = g.L64 * ((double)qe.v - g.cen);
        if (aF > 126.0) {
          // above every threshold by more than 26 / L (F was clamped): s(1 - s)
          // <= 1 / t, so |h| <= 2^-aF sum_k |g_k| / E_k; take h = 0 with that error
          h = 0.0;
          err = exp2(-aF) * g.ginv * g.gscale;
        } else {
          // the float F of the sum, or float64 below the normal float range
          const double sc = (aF >= -126.0 ? (double)a[j] : exp2(aF)) * g.gscale;
          h = (accP[j] + accN[j]) * sc;
          // + underflow of g E below the float range: under 2^-147 per entry
          err = (kFactoredK * (accP[j] - accN[j]) + (double)(g.nP + g.nN) * 0x1p-147) * sc;
        }
      } else {
        h = (accP[j] + accN[j]) * g.gscale;
        // + the exponent clamps and underflow: under 2^-50 of sum |gs_k|
        err = (kDirectK * (accP[j] - accN[j]) + kDirectKx * (double)mw[j] + g.g1 * 0x1p-50) * g.gscale;
      }
      need = lc * err > fmax(kAbsTarget, kRelTarget * lc * fmax(fabs(h) - err, 0.0));
      if (!need) g.out[qe.idx] = (float)(-g.lam64 * (double)qe.c * h);
    }
    const uint64_t bal = __ballot(need);
    if (need) {
      R[rcount + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u))] = qe;
    }
    rcount += __popcll(bal);
    if (rcount > 0) {
      wave_lds_sync();
      refine_list(g, R, rcount, lane);
      rcount = 0;
      wave_lds_sync();
    }
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
  QEntry* rlists = queues + kGradWaves * kQueueCap;                     // kGradWaves x kRefCap
  float2* T = reinterpret_cast<float2*>(rlists + kGradWaves * kRefCap);  // H + kTablePad entries
  // set-up scratch, overlaying the queues: 3 x kGradNT floats + 2 x kGradNT
  // ints, then 2 x kGradWaves ints (table order), then 2 x kGradNT doubles
  float* red = reinterpret_cast<float*>(smem);
  int* redi = reinterpret_cast<int*>(red + 3 * kGradNT);
  int* cnt = reinterpret_cast<int*>(smem);
  double* redd = reinterpret_cast<double*>(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = p.H;
  const float INF = __builtin_inff();

  // ---------------- threshold range, largest |g|, how many g > 0 and g < 0
  {
    float lo = INF, hi = -INF, gm = 0.0f;
    int np = 0, nn = 0;
    for (int k = tid; k < H; k += kGradNT) {
      const float t = p.tau[k], gk = p.grad_out[k];
      lo = fminf(lo, t);
      hi = fmaxf(hi, t);
      gm = fmaxf(gm, fabsf(gk));
      np += gk > 0.0f;
      nn += gk < 0.0f;
    }
    red[tid] = lo;
    red[kGradNT + tid] = hi;
    red[2 * kGradNT + tid] = gm;
    redi[tid] = np;
    redi[kGradNT + tid] = nn;
    __syncthreads();
    for (int off = kGradNT / 2; off > 0; off >>= 1) {
      if (tid < off) {
        red[tid] = fminf(red[tid], red[tid + off]);
        red[kGradNT + tid] = fmaxf(red[kGradNT + tid], red[kGradNT + tid + off]);
        red[2 * kGradNT + tid] = fmaxf(red[2 * kGradNT + tid], red[2 * kGradNT + tid + off]);
        redi[tid] += redi[tid + off];
        redi[kGradNT + tid] += redi[kGradNT + tid + off];
      }
      __syncthreads();
    }
  }
  const float tlo = uni(red[0]), thi = uni(red[kGradNT]), gmax = uni(red[2 * kGradNT]);
  const int P = uni(redi[0]), N = uni(redi[kGradNT]);
  __syncthreads();  // the scratch is reused below

  GradCtx g;
  g.L64 = (double)p.lambda * 1.4426950408889634074;  // lambda * log2(e)
  g.cen = 0.5 * ((double)tlo + (double)thi);
  const double half_span = g.L64 * 0.5 * ((double)thi - (double)tlo);
  // E in [2^-100, 2^100]; false for inf/NaN spans
  g.factored = (half_span >= 0.0) && (half_span <= 100.0);
  g.Lf = (float)g.L64;
  g.lam64 = (double)p.lambda;
  g.out = p.out;
  g.T = T;
  g.tau = p.tau;
  g.gout = p.grad_out;
  g.H = H;
  g.nP = (P + kBlk - 1) & ~(kBlk - 1);
  g.nN = (N + kBlk - 1) & ~(kBlk - 1);
  // gs = g / 2^s with max |gs| in [1, 2): |gs E| <= 2^101
  int sh = gmax > 0.0f ? ilogbf(gmax) : 0;
  sh = sh < -200 ? -200 : (sh > 200 ? 200 : sh);
  g.gscale = ldexp(1.0, sh);

  // ---------------- the table: g > 0 in threshold order, then g < 0
  double ginv = 0.0, g1 = 0.0;
  {
    int runP = 0, runN = 0;
    for (int base = 0; base < H; base += kGradNT) {
      const int k = base + tid;
      float tk = 0.0f, gk = 0.0f;
      if (k < H) {
        tk = p.tau[k];
        gk = p.grad_out[k];
      }
      const bool pos = gk > 0.0f, neg = gk < 0.0f;
      const uint64_t bp = __ballot(pos), bn = __ballot(neg);
      if (lane == 0) {
        cnt[wave] = __popcll(bp);
        cnt[kGradWaves + wave] = __popcll(bn);
      }
      __syncthreads();
      int offP = runP, offN = runN;
      for (int w = 0; w < kGradWaves; ++w) {
        const int cp = cnt[w], cn = cnt[kGradWaves + w];
        if (w < wave) {
          offP += cp;
          offN += cn;
        }
        runP += cp;
        runN += cn;
      }
      if (pos || neg) {
        const uint64_t bal = pos ? bp : bn;
        const int below = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
        const int slot = pos ? offP + below : g.nP + offN + below;
        const float gs = ldexpf(gk, -sh);
        float2 e;
        if (g.factored) {
          const float E = (float)exp2(g.L64 * (g.cen - (double)tk));
          e = make_float2(E, gs * E);
          ginv += fabs((double)gs) / (double)E;
        } else {
          e = make_float2(tk, gs);
        }
        g1 += fabs((double)gs);
        T[slot] = e;
      }
      __syncthreads();  // cnt is rewritten by the next chunk
    }
  }
  for (int k = P + tid; k < g.nP; k += kGradNT) T[k] = make_float2(0.0f, 0.0f);
  for (int k = g.nP + N + tid; k < g.nP + g.nN; k += kGradNT) T[k] = make_float2(0.0f, 0.0f);
  redd[tid] = ginv;
  redd[kGradNT + tid] = g1;
  __syncthreads();
  for (int off = kGradNT / 2; off > 0; off >>= 1) {
    if (tid < off) {
      redd[tid] += redd[tid + off];
      redd[kGradNT + tid] += redd[kGradNT + tid + off];
    }
    __syncthreads();
  }
  g.ginv = uni(redd[0]);
  g.g1 = uni(redd[kGradNT]);
  // wave-uniform: scalar registers rather than vector pairs across the loop
  g.L64 = uni(g.L64);
  g.cen = uni(g.cen);
  g.lam64 = uni(g.lam64);
  g.gscale = uni(g.gscale);
  g.Lf = uni(g.Lf);
  __syncthreads();  // the queues overlay the scratch

  // ---------------- segments of 64 voxels, one per wave at a time
  const float* grid = p.grid;
  const int64_t nz = p.nz, ny = p.ny, nx = p.nx;
  const int64_t plane = ny * nx, nvox = nz * plane;
  QEntry* q = queues + wave * kQueueCap;
  QEntry* R = rlists + wave * kRefCap;
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
      sweep(g, q + (count - kBatch), kBatch, lane, R);
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
    sweep(g, q, count, lane, R);
  }
}

template <bool D3>
hipError_t launch_grad(const GradArgs& a, hipStream_t s, int64_t nseg, const DeviceInfo& di) {
  auto k = soft_grad_kernel<D3>;
  const size_t lds = (size_t)kGradWaves * (kQueueCap + kRefCap) * sizeof(QEntry) +
                     (size_t)(a.H + kTablePad) * sizeof(float2);
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
