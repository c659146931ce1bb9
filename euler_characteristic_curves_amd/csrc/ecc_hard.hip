// Hard Euler characteristic curve kernels for gfx950 (MI355X).
//
// Method: page "Scalable GPU-Accelerated Euler Characteristic Curves"
// (paper notes), "Method / Key designs": a single full sweep over the grid,
// per-workgroup histograms of H bins in on-chip memory, one global atomic per
// bin per workgroup, and the curve as the running sum of the histogram.  The
// per-voxel contribution is the "local Euler coefficient" of the same section,
// regrouped as below.
//
// Decomposition used here (exact).  Voxel p owns the cells reaching from p
// towards +x/+y(/+z).  Pair every cell without an x-extent with its
// x-extrusion: they have opposite signs and the extrusion's value is the max
// of the cell's value at x and at x+1.  Along each image row this leaves 2
// (2D) or 4 (3D) one-dimensional sequences
//     s1 = b(z,y,x)                                        sign +
//     s2 = max over {y, y+1}                               sign -
//     s3 = max over {z, z+1}                 (3D only)     sign -
//     s4 = max over {y, y+1} x {z, z+1}      (3D only)     sign +
// and each sequence contributes sum_x [ +s(x) - max(s(x), s(x+1)) ].  That
// telescopes along x to a weight (inc(x) - inc(x-1)) at s(x), with
// inc(x) = [s(x+1) > s(x)], which is non-zero only at local extrema.
// Weights of different sequences that land on the same bin at the same x are
// merged before they touch the histogram.  Cells that would reach outside the
// grid get the "trash" key (one past the last bin): out-of-range voxels read
// as +infinity, so such cells never enter a counted bin.
//
// Binning: bin(max of corners) = max of the corners' bins because bin() is
// monotone, so every voxel is binned once.  uint8 grids skip binning: they
// histogram raw byte values and the last workgroup maps values to thresholds.

#include <hip/hip_runtime.h>

#include "ecc_device.hpp"
#include "ecc_internal.hpp"

namespace ecc {
namespace {

template <int DT> struct Elem;
template <> struct Elem<0> { using T = uint8_t; };
template <> struct Elem<1> { using T = float; };

struct BinCtx {
  const float* R;  // running max of tau in LDS (f32 grids)
  int H;
  float r0, scale;
  int trash;       // key of "no threshold admits this cell"
};

template <int DT>
__device__ __forceinline__ int key_of(typename Elem<DT>::T v, const BinCtx& c) {
  if constexpr (DT == 0) {
    (void)c;
    return (int)v;
  } else {
    return bin_of(v, c.R, c.H, c.r0, c.scale);
  }
}

// VEC consecutive keys of one row starting at x0 (x0 is a multiple of VEC).
template <int DT, int VEC>
__device__ __forceinline__ void load_keys(const typename Elem<DT>::T* row, int64_t x0, int64_t nx,
                                          bool vec_ok, const BinCtx& c, int (&k)[VEC]) {
  using T = typename Elem<DT>::T;
  if (row == nullptr) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) k[j] = c.trash;
    return;
  }
  if (vec_ok && x0 + VEC <= nx) {
    if constexpr (DT == 0) {
      static_assert(VEC == 16 || VEC == 8, "u8 vector width");
      if constexpr (VEC == 16) {
        const uint4 w = *reinterpret_cast<const uint4*>(row + x0);
        const unsigned int ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 16; ++j) k[j] = (int)((ws[j >> 2] >> (8 * (j & 3))) & 0xffu);
      } else {
        const uint2 w = *reinterpret_cast<const uint2*>(row + x0);
        const unsigned int ws[2] = {w.x, w.y};
#pragma unroll
        for (int j = 0; j < 8; ++j) k[j] = (int)((ws[j >> 2] >> (8 * (j & 3))) & 0xffu);
      }
    } else {
      static_assert(VEC == 4, "f32 vector width");
      const float4 w = *reinterpret_cast<const float4*>(row + x0);
      k[0] = key_of<DT>(w.x, c);
      k[1] = key_of<DT>(w.y, c);
      k[2] = key_of<DT>(w.z, c);
      k[3] = key_of<DT>(w.w, c);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    const int64_t x = x0 + j;
    k[j] = x < nx ? key_of<DT>(row[x], c) : c.trash;
  }
  (void)sizeof(T);
}

template <int DT>
__device__ __forceinline__ int load_key1(const typename Elem<DT>::T* row, int64_t x, int64_t nx,
                                         const BinCtx& c) {
  return (row != nullptr && x >= 0 && x < nx) ? key_of<DT>(row[x], c) : c.trash;
}

// Weight of a sequence at one position: +1 at a start of a rise, -1 at its top.
__device__ __forceinline__ int tele(int prev, int cur, int next) {
  return (int)(next > cur) - (int)(cur > prev);
}

// ------------------------------------------------------------ shared tail
// Flush the workgroup histogram with one global atomic per non-zero bin, then
// let the last workgroup build the curve and re-zero the workspace.
template <int DT, int C>
__device__ void flush_and_finish(const HardArgs& a, int nbins, int* hist, long long* tmp,
                                 long long* ch, int* flag) {
  unsigned int* ticket = reinterpret_cast<unsigned int*>(a.ws);
  long long* acc = reinterpret_cast<long long*>(reinterpret_cast<char*>(a.ws) + kWsHeader);
  const int stride = acc_bins(a.H);
  __syncthreads();
  long long* mine = acc + (size_t)(blockIdx.x % kAccCopies) * stride;
  for (int b = threadIdx.x; b < nbins; b += kBlock) {
    int s = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) s += hist[b * C + c];
    if (s != 0) agent_add(mine + b, (long long)s);
  }
  if (!last_block_arrives(ticket, flag)) return;

  auto total = [&](int i) {
    long long s = 0;
#pragma unroll
    for (int c = 0; c < kAccCopies; ++c) s += agent_load(acc + (size_t)c * stride + i);
    return s;
  };
  if constexpr (DT == 0) {
    // per-value histogram -> cumulative count of values <= v
    block_scan<long long>(
        256, 0LL, [](long long x, long long y) { return x + y; }, total,
        [&](int i, long long v) { ch[i] = v; }, tmp);
    // out[k] = #(values <= R_k) weighted, R = running max of tau
    float* ftmp = reinterpret_cast<float*>(tmp);
    int64_t* out = a.out;
    block_scan<float>(
        a.H, -__builtin_inff(), [](float x, float y) { return fmaxf(x, y); },
        [&](int i) { return a.tau[i]; },
        [&](int i, float r) {
          long long v = 0;
          if (r >= 255.0f) v = ch[255];
          else if (r >= 0.0f) v = ch[(int)floorf(r)];
          out[i] = v;
        },
        ftmp);
  } else {
    int64_t* out = a.out;
    block_scan<long long>(
        a.H, 0LL, [](long long x, long long y) { return x + y; }, total,
        [&](int i, long long v) { out[i] = v; }, tmp);
  }
  for (int i = threadIdx.x; i < kAccCopies * stride; i += kBlock) agent_store(acc + i, 0LL);
}

template <int DT>
__device__ __forceinline__ void setup_bins(const HardArgs& a, float* R, long long* tmp, BinCtx& c,
                                           int nbins) {
  c.H = a.H;
  c.trash = nbins;
  c.R = R;
  c.r0 = 0.0f;
  c.scale = 0.0f;
  if constexpr (DT == 1) {
    running_max_to_lds(a.tau, a.H, R, reinterpret_cast<float*>(tmp));
    guess_params(R, a.H, &c.r0, &c.scale);
  }
}

// ------------------------------------------------------------------- 2D
// Workgroup tile: 4 waves stacked in y, each wave owns TH rows of a chunk of
// 64*VEC columns and marches down them, keeping the current row's keys in
// registers and loading the next.
template <int DT, int VEC, int C, int TH>
__global__ __launch_bounds__(kBlock) void hard2d_kernel(HardArgs a, int nbins, int64_t ntx,
                                                        int64_t ntiles, int vec_ok) {
  extern __shared__ __align__(16) unsigned char smem[];
  using T = typename Elem<DT>::T;
  long long* tmp = reinterpret_cast<long long*>(smem);            // 256
  long long* ch = tmp + kBlock;                                    // 256
  int* flag = reinterpret_cast<int*>(ch + kBlock);                 // 4 ints
  int* hist = flag + 4;                                            // (nbins+1)*C
  float* R = reinterpret_cast<float*>(hist + (nbins + 1) * C);     // H (f32)

  for (int i = threadIdx.x; i < (nbins + 1) * C; i += kBlock) hist[i] = 0;
  BinCtx bc;
  setup_bins<DT>(a, R, tmp, bc, nbins);
  __syncthreads();

  const T* grid = reinterpret_cast<const T*>(a.grid);
  const int64_t ny = a.ny, nx = a.nx;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lofs = lane & (C - 1);
  constexpr int64_t CHUNK = 64 * VEC;
  const bool vok = vec_ok != 0;

  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t tx = t % ntx, tyb = t / ntx;
    const int64_t ys = (tyb * kWavesPerBlock + wave) * TH;
    if (ys >= ny) continue;
    const int64_t ye = ys + TH < ny ? ys + TH : ny;
    const int64_t xb = tx * CHUNK, x0 = xb + lane * VEC;

    int cur[VEC], nxt[VEC];
    const T* row = grid + ys * nx;
    load_keys<DT, VEC>(row, x0, nx, vok, bc, cur);
    int curL = load_key1<DT>(row, xb - 1, nx, bc);
    int curR = load_key1<DT>(row, xb + CHUNK, nx, bc);

    for (int64_t y = ys; y < ye; ++y) {
      const T* nrow = (y + 1 < ny) ? grid + (y + 1) * nx : nullptr;
      load_keys<DT, VEC>(nrow, x0, nx, vok, bc, nxt);
      const int nxtL = load_key1<DT>(nrow, xb - 1, nx, bc);
      const int nxtR = load_key1<DT>(nrow, xb + CHUNK, nx, bc);

      int s1[VEC], s2[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        s1[j] = cur[j];
        s2[j] = max(cur[j], nxt[j]);
      }
      int s1l = __shfl_up(s1[VEC - 1], 1), s2l = __shfl_up(s2[VEC - 1], 1);
      int s1r = __shfl_down(s1[0], 1), s2r = __shfl_down(s2[0], 1);
      if (lane == 0) { s1l = curL; s2l = max(curL, nxtL); }
      if (lane == 63) { s1r = curR; s2r = max(curR, nxtR); }
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const int p1 = j ? s1[j - 1] : s1l, n1 = j + 1 < VEC ? s1[j + 1] : s1r;
        const int p2 = j ? s2[j - 1] : s2l, n2 = j + 1 < VEC ? s2[j + 1] : s2r;
        int w1 = tele(p1, s1[j], n1);
        int w2 = -tele(p2, s2[j], n2);
        if (s1[j] == s2[j]) { w1 += w2; w2 = 0; }
        if (w1) atomicAdd(&hist[s1[j] * C + lofs], w1);
        if (w2) atomicAdd(&hist[s2[j] * C + lofs], w2);
      }
#pragma unroll
      for (int j = 0; j < VEC; ++j) cur[j] = nxt[j];
      curL = nxtL;
      curR = nxtR;
    }
  }
  flush_and_finish<DT, C>(a, nbins, hist, tmp, ch, flag);
}

// ------------------------------------------------------------------- 3D
// Wave tile: a chunk of 64*VEC columns x TY rows x TZ planes.  The wave
// marches along z holding TY+1 rows (TY plus a one-row halo) of planes z and
// z+1 in registers; each step loads the TY+1 rows of the next plane.
template <int DT, int VEC, int C, int TY>
__global__ __launch_bounds__(kBlock) void hard3d_kernel(HardArgs a, int nbins, int64_t ntx,
                                                        int64_t nty4, int64_t TZ, int64_t ntiles,
                                                        int vec_ok) {
  extern __shared__ __align__(16) unsigned char smem[];
  using T = typename Elem<DT>::T;
  long long* tmp = reinterpret_cast<long long*>(smem);
  long long* ch = tmp + kBlock;
  int* flag = reinterpret_cast<int*>(ch + kBlock);
  int* hist = flag + 4;
  float* R = reinterpret_cast<float*>(hist + (nbins + 1) * C);

  for (int i = threadIdx.x; i < (nbins + 1) * C; i += kBlock) hist[i] = 0;
  BinCtx bc;
  setup_bins<DT>(a, R, tmp, bc, nbins);
  __syncthreads();

  const T* grid = reinterpret_cast<const T*>(a.grid);
  const int64_t nz = a.nz, ny = a.ny, nx = a.nx;
  const int64_t plane = ny * nx;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lofs = lane & (C - 1);
  constexpr int64_t CHUNK = 64 * VEC;
  const bool vok = vec_ok != 0;

  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t tx = t % ntx;
    const int64_t rest = t / ntx;
    const int64_t tyg = rest % nty4, tz = rest / nty4;
    const int64_t ys = (tyg * kWavesPerBlock + wave) * TY;
    if (ys >= ny) continue;
    const int64_t zs = tz * TZ;
    const int64_t ze = zs + TZ < nz ? zs + TZ : nz;
    const int64_t xb = tx * CHUNK, x0 = xb + lane * VEC;

    int A[TY + 1][VEC], B[TY + 1][VEC];
    int AL[TY + 1], AR[TY + 1], BL[TY + 1], BR[TY + 1];
#pragma unroll
    for (int r = 0; r <= TY; ++r) {
      const T* row = (ys + r < ny) ? grid + zs * plane + (ys + r) * nx : nullptr;
      load_keys<DT, VEC>(row, x0, nx, vok, bc, A[r]);
      AL[r] = load_key1<DT>(row, xb - 1, nx, bc);
      AR[r] = load_key1<DT>(row, xb + CHUNK, nx, bc);
    }
    for (int64_t z = zs; z < ze; ++z) {
      const bool zn = z + 1 < nz;
#pragma unroll
      for (int r = 0; r <= TY; ++r) {
        const T* row = (zn && ys + r < ny) ? grid + (z + 1) * plane + (ys + r) * nx : nullptr;
        load_keys<DT, VEC>(row, x0, nx, vok, bc, B[r]);
        BL[r] = load_key1<DT>(row, xb - 1, nx, bc);
        BR[r] = load_key1<DT>(row, xb + CHUNK, nx, bc);
      }
#pragma unroll
      for (int r = 0; r < TY; ++r) {
        if (ys + r < ny) {
          int s1[VEC], s2[VEC], s3[VEC], s4[VEC];
#pragma unroll
          for (int j = 0; j < VEC; ++j) {
            s1[j] = A[r][j];
            s2[j] = max(A[r][j], A[r + 1][j]);
            s3[j] = max(A[r][j], B[r][j]);
            s4[j] = max(s2[j], max(B[r][j], B[r + 1][j]));
          }
          const int e1l = AL[r], e2l = max(AL[r], AL[r + 1]), e3l = max(AL[r], BL[r]),
                    e4l = max(e2l, max(BL[r], BL[r + 1]));
          const int e1r = AR[r], e2r = max(AR[r], AR[r + 1]), e3r = max(AR[r], BR[r]),
                    e4r = max(e2r, max(BR[r], BR[r + 1]));
          int l1 = __shfl_up(s1[VEC - 1], 1), l2 = __shfl_up(s2[VEC - 1], 1);
          int l3 = __shfl_up(s3[VEC - 1], 1), l4 = __shfl_up(s4[VEC - 1], 1);
          int r1 = __shfl_down(s1[0], 1), r2 = __shfl_down(s2[0], 1);
          int r3 = __shfl_down(s3[0], 1), r4 = __shfl_down(s4[0], 1);
          if (lane == 0) { l1 = e1l; l2 = e2l; l3 = e3l; l4 = e4l; }
          if (lane == 63) { r1 = e1r; r2 = e2r; r3 = e3r; r4 = e4r; }
#pragma unroll
          for (int j = 0; j < VEC; ++j) {
            int w1 = tele(j ? s1[j - 1] : l1, s1[j], j + 1 < VEC ? s1[j + 1] : r1);
            int w2 = -tele(j ? s2[j - 1] : l2, s2[j], j + 1 < VEC ? s2[j + 1] : r2);
            int w3 = -tele(j ? s3[j - 1] : l3, s3[j], j + 1 < VEC ? s3[j + 1] : r3);
            int w4 = tele(j ? s4[j - 1] : l4, s4[j], j + 1 < VEC ? s4[j + 1] : r4);
            // move weights between entries holding the same key
            if (s4[j] == s3[j]) { w3 += w4; w4 = 0; }
            else if (s4[j] == s2[j]) { w2 += w4; w4 = 0; }
            if (s3[j] == s2[j]) { w2 += w3; w3 = 0; }
            if (s2[j] == s1[j]) { w1 += w2; w2 = 0; }
            if (s3[j] == s1[j]) { w1 += w3; w3 = 0; }
            if (w1) atomicAdd(&hist[s1[j] * C + lofs], w1);
            if (w2) atomicAdd(&hist[s2[j] * C + lofs], w2);
            if (w3) atomicAdd(&hist[s3[j] * C + lofs], w3);
            if (w4) atomicAdd(&hist[s4[j] * C + lofs], w4);
          }
        }
      }
#pragma unroll
      for (int r = 0; r <= TY; ++r) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) A[r][j] = B[r][j];
        AL[r] = BL[r];
        AR[r] = BR[r];
      }
    }
  }
  flush_and_finish<DT, C>(a, nbins, hist, tmp, ch, flag);
}

// ------------------------------------------------------------- launcher
int copies_for(int nbins) {
  const int c = 9000 / (nbins + 1);
  if (c >= 32) return 32;
  if (c >= 16) return 16;
  if (c >= 8) return 8;
  if (c >= 4) return 4;
  if (c >= 2) return 2;
  return 1;
}

size_t lds_bytes(int DT, int nbins, int C, int H) {
  size_t b = 2 * kBlock * sizeof(long long) + 4 * sizeof(int) + (size_t)(nbins + 1) * C * sizeof(int);
  if (DT == 1) b += (size_t)H * sizeof(float);
  return b;
}

template <int DT, int VEC, int C, int TH>
hipError_t launch2d(const HardArgs& a, int nbins, hipStream_t s, const DeviceInfo& di) {
  constexpr int64_t CHUNK = 64 * VEC;
  const int64_t ntx = (a.nx + CHUNK - 1) / CHUNK;
  const int64_t nty = (a.ny + TH * kWavesPerBlock - 1) / (TH * kWavesPerBlock);
  const int64_t ntiles = ntx * nty;
  const size_t esz = DT == 0 ? 1 : 4;
  const int vec_ok = (reinterpret_cast<uintptr_t>(a.grid) % (VEC * esz) == 0) &&
                     ((a.nx * (int64_t)esz) % (int64_t)(VEC * esz) == 0);
  const size_t lds = lds_bytes(DT, nbins, C, a.H);
  int64_t g = (int64_t)di.cus * 4;
  if (g > ntiles) g = ntiles;
  if (g < 1) g = 1;
  auto k = hard2d_kernel<DT, VEC, C, TH>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3((unsigned)g), dim3(kBlock), lds, s, a, nbins, ntx, ntiles, vec_ok);
  return hipGetLastError();
}

template <int DT, int VEC, int C, int TY>
hipError_t launch3d(const HardArgs& a, int nbins, hipStream_t s, const DeviceInfo& di) {
  constexpr int64_t CHUNK = 64 * VEC;
  const int64_t ntx = (a.nx + CHUNK - 1) / CHUNK;
  const int64_t nty4 = (a.ny + TY * kWavesPerBlock - 1) / (TY * kWavesPerBlock);
  // split z so that there are enough tiles to fill the chip
  const int64_t want = (int64_t)di.cus * 4;
  int64_t ntz = (want + ntx * nty4 - 1) / (ntx * nty4);
  if (ntz < 1) ntz = 1;
  if (ntz > a.nz) ntz = a.nz;
  int64_t TZ = (a.nz + ntz - 1) / ntz;
  if (TZ < 8 && a.nz >= 8) TZ = 8;
  ntz = (a.nz + TZ - 1) / TZ;
  const int64_t ntiles = ntx * nty4 * ntz;
  const size_t esz = DT == 0 ? 1 : 4;
  const int vec_ok = (reinterpret_cast<uintptr_t>(a.grid) % (VEC * esz) == 0) &&
                     ((a.nx * (int64_t)esz) % (int64_t)(VEC * esz) == 0);
  const size_t lds = lds_bytes(DT, nbins, C, a.H);
  int64_t g = want;
  if (g > ntiles) g = ntiles;
  if (g < 1) g = 1;
  auto k = hard3d_kernel<DT, VEC, C, TY>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3((unsigned)g), dim3(kBlock), lds, s, a, nbins, ntx, nty4, TZ, ntiles,
                     vec_ok);
  return hipGetLastError();
}

template <int C>
hipError_t dispatch_f32(const HardArgs& a, int nbins, hipStream_t s, const DeviceInfo& di) {
  if (a.nz == 1) return launch2d<1, 4, C, 16>(a, nbins, s, di);
  return launch3d<1, 4, C, 4>(a, nbins, s, di);
}

}  // namespace

hipError_t launch_hard(const HardArgs& a, hipStream_t s) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  if (a.dtype == 0) {
    if (a.nz == 1) return launch2d<0, 16, 32, 16>(a, 256, s, di);
    return launch3d<0, 8, 32, 4>(a, 256, s, di);
  }
  const int nbins = a.H;
  switch (copies_for(nbins)) {
    case 32: return dispatch_f32<32>(a, nbins, s, di);
    case 16: return dispatch_f32<16>(a, nbins, s, di);
    case 8: return dispatch_f32<8>(a, nbins, s, di);
    case 4: return dispatch_f32<4>(a, nbins, s, di);
    case 2: return dispatch_f32<2>(a, nbins, s, di);
    default: return dispatch_f32<1>(a, nbins, s, di);
  }
}

}  // namespace ecc
