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

#include <mutex>
#include <type_traits>

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

// Exact bin of one float (slow path: edge tiles and unaligned grids), out of line.
__device__ __attribute__((noinline)) int bin_generic(float v, const float* R, int H, float r0, float scale) {
  return bin_of(v, R, H, r0, scale);
}

template <int DT>
__device__ __forceinline__ int key_of(typename Elem<DT>::T v, const BinCtx& c) {
  if constexpr (DT == 0) {
    (void)c;
    return (int)v;
  } else {
    return bin_generic(v, c.R, c.H, c.r0, c.scale);
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
      static_assert(VEC == 16 || VEC == 8 || VEC == 4, "u8 vector width");
      if constexpr (VEC == 16) {
        const uint4 w = *reinterpret_cast<const uint4*>(row + x0);
        const unsigned int ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 16; ++j) k[j] = (int)((ws[j >> 2] >> (8 * (j & 3))) & 0xffu);
      } else if constexpr (VEC == 4) {
        const unsigned int w = *reinterpret_cast<const unsigned int*>(row + x0);
#pragma unroll
        for (int j = 0; j < 4; ++j) k[j] = (int)((w >> (8 * j)) & 0xffu);
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

// ------------------------------------------------------- fast-path helpers
// Cross-lane neighbours with DPP wave shifts (no LDS traffic).  Lane i gets
// lane i-1's (from_left) / lane i+1's (from_right) value; the lane at the end
// of the wave, which has no source lane, gets `edge`.
__device__ __forceinline__ int from_left(int v, int edge) {
  return __builtin_amdgcn_update_dpp(edge, v, 0x138 /* wave_shr:1 */, 0xF, 0xF, false);
}
__device__ __forceinline__ int from_right(int v, int edge) {
  return __builtin_amdgcn_update_dpp(edge, v, 0x130 /* wave_shl:1 */, 0xF, 0xF, false);
}

// Telescoped weights of one row sequence over this lane's V positions and
// unconditional histogram updates (an update of 0 costs the same LDS time as
// a masked one, and needs no exec-mask branches).  sign is +1 or -1.
//
// With ADDR the keys are already the LDS byte addresses of the lane's
// counters (bin * 4C + 4 * copy + histogram base), so the update needs no
// address arithmetic.  Comparisons of such keys order different bins
// correctly (the copy offset is below one bin's stride) and break ties
// between equal bins arbitrarily, which the telescoped sum allows: an x-edge
// of two equal keys may go to either end, as long as both ends see the same
// choice, and they do, because both lanes compare the same two values.
typedef __attribute__((address_space(3))) int lds_int;

template <int V, int C, bool ADDR = false>
__device__ __forceinline__ void tele_add(const int (&s)[V], int left, int right, int sign, int* hist,
                                         int lofs) {
  // d = s(x) - s(x+1) is negative exactly when the sequence rises after x.
  // Keys are below 2^18, so |d| < 2^24 and d >> 24 (arithmetic) is -1 on a
  // rise and 0 otherwise: the weight inc(x) - inc(x-1) is then one
  // subtraction of the top bytes of two differences (a byte-select form of
  // the subtraction, no separate compare and select per update).
  int dprev = left - s[0];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int nxt = j + 1 < V ? s[j + 1] : right;
    const int d = s[j] - nxt;
    const int w = sign > 0 ? (dprev >> 24) - (d >> 24) : (d >> 24) - (dprev >> 24);
    dprev = d;
    if constexpr (ADDR)
      __hip_atomic_fetch_add((lds_int*)(size_t)(unsigned int)s[j], w, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
    else
      atomicAdd(&hist[s[j] * C + lofs], w);
  }
}

// Binning table for float grids: P[k] = (R[k-1], R[k]) with R[-1] = -inf and
// R[H] = +inf, so v belongs to bin k iff P[k].x < v <= P[k].y.
template <int NT>
__device__ __forceinline__ void build_pairs(const float* R, int H, float2* P) {
  for (int k = threadIdx.x; k <= H; k += NT)
    P[k] = make_float2(k > 0 ? R[k - 1] : -__builtin_inff(), k < H ? R[k] : __builtin_inff());
}

// ------------------------------------------------------------ shared tail
// Reduce the workgroup histograms over the grid and let the last workgroup
// turn the totals into the curve.  `tot`
// is LDS for nbins int64 that may alias the (no longer needed) histogram.
template <int DT, int C, int NT>
__device__ __forceinline__ void flush_and_finish(const HardArgs& a, int nbins, int* hist, long long* tmp,
                                                 long long* ch, int* flag, long long* tot) {
  __syncthreads();
  // per-bin sum of the C copies, starting at a lane-dependent copy so that
  // the lanes of a wave read different banks
  auto local = [&](int b) {
    long long s = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) s += hist[b * C + ((c + (int)threadIdx.x) & (C - 1))];
    return s;
  };
  if (gridDim.x == 1) {
    // A lone workgroup: no device atomics.  tot aliases the histogram, and
    // tot[b] covers the counters of bins near 2b/C: bins <= b for C >= 2,
    // bins 2b and 2b+1 for C == 1.  Chunks of NT bins are read into
    // registers and then written, bottom-up for C >= 2 and top-down for
    // C == 1, so no counter is overwritten before it is read.
    const int nch = (nbins + NT - 1) / NT;
    for (int jj = 0; jj < nch; ++jj) {
      const int b = (C >= 2 ? jj : nch - 1 - jj) * NT + (int)threadIdx.x;
      const long long v = b < nbins ? local(b) : 0;
      __syncthreads();
      if (b < nbins) tot[b] = v;
      __syncthreads();
    }
  } else if (!grid_reduce<NT>(a.ws, a.H, nbins, local, tot, flag, a.acc_copies,
                                 // float 2D workgroups finish spread out by their
                                 // binning: one ticket up to 256 of them measured
                                 // 0.3-0.45 us faster; uint8 ones finish together
                                 DT == 1 && NT == kBlock ? 256u : kFlatTicketMax)) {
    return;
  }
  int64_t* out = a.out;
  if constexpr (DT == 0) {
    // per-value histogram -> weighted count of values <= v
    block_scan<long long, NT>(
        256, 0LL, [](long long x, long long y) { return x + y; }, [&](int i) { return tot[i]; },
        [&](int i, long long v) { ch[i] = v; }, tmp);
    // out[k] = weighted count of values <= R_k, R = running max of tau
    float* ftmp = reinterpret_cast<float*>(tmp);
    block_scan<float, NT>(
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
    block_scan<long long, NT>(
        a.H, 0LL, [](long long x, long long y) { return x + y; }, [&](int i) { return tot[i]; },
        [&](int i, long long v) { out[i] = v; }, tmp);
  }
}

template <int DT, int NT>
__device__ __forceinline__ void setup_bins(const HardArgs& a, float* R, float* scan, BinCtx& c,
                                           int nbins) {
  c.H = a.H;
  c.trash = nbins;
  c.R = R;
  c.r0 = 0.0f;
  c.scale = 0.0f;
  if constexpr (DT == 1) {
    running_max_to_lds<NT>(a.tau, a.H, R, scan);
    guess_params(R, a.H, &c.r0, &c.scale);
  }
}

// ------------------------------------------------------------ raw rows
// One row slice of a wave: VEC elements per lane plus the two elements just
// outside the wave's column chunk (needed by lanes 0 and 63).
template <int DT, int VEC> struct RawRow;
template <> struct RawRow<0, 16> { uint4 v; uint8_t l, r; };
template <> struct RawRow<0, 8> { uint2 v; uint8_t l, r; };
template <> struct RawRow<0, 4> { unsigned int v; uint8_t l, r; };
template <> struct RawRow<1, 4> { float4 v; float l, r; };

// Loads are unconditional: callers clamp the row pointer to a valid row and
// the edge columns to valid columns, and apply validity when forming keys, so
// the compiler can keep several loads in flight across loop iterations.
// A 64-bit integer that is the same in every lane, moved to scalar registers
// (offsets only: a pointer round-tripped through an integer would lose its
// global address space and turn loads into flat loads).
__device__ __forceinline__ int64_t uni64(int64_t v) {
  const unsigned int lo = __builtin_amdgcn_readfirstlane((unsigned int)(unsigned long long)v);
  const unsigned int hi = __builtin_amdgcn_readfirstlane((unsigned int)((unsigned long long)v >> 32));
  return (int64_t)(((unsigned long long)hi << 32) | lo);
}

template <int DT, int VEC>
__device__ __forceinline__ void fetch_row(RawRow<DT, VEC>& raw, const typename Elem<DT>::T* row,
                                          int64_t xb, int lane, int64_t xl, int64_t xr) {
  using T = typename Elem<DT>::T;
  // wave-uniform base (scalar registers) + 32-bit per-lane byte offset, so the
  // load uses the saddr + voffset form instead of per-lane 64-bit adds
  const char* base = reinterpret_cast<const char*>(row + xb);
  const unsigned int off = (unsigned int)lane * (unsigned int)(VEC * sizeof(T));
  if constexpr (DT == 0 && VEC == 16) raw.v = *reinterpret_cast<const uint4*>(base + off);
  if constexpr (DT == 0 && VEC == 8) raw.v = *reinterpret_cast<const uint2*>(base + off);
  if constexpr (DT == 0 && VEC == 4) raw.v = *reinterpret_cast<const unsigned int*>(base + off);
  if constexpr (DT == 1) raw.v = *reinterpret_cast<const float4*>(base + off);
  raw.l = row[xl];
  raw.r = row[xr];
}

struct FastBin {
  const float2* P;
  const float* R;
  int H;
  float mul, add;
};

// Fast bin guess for one float (first k with v <= R[k] when the thresholds
// are close to uniform): 4 VALU ops, clamped to [0, H] (NaN -> 0).
__device__ __forceinline__ int bin_guess(float v, const FastBin& fb) {
  const int k = (int)ceilf(fmaf(v, fb.mul, fb.add));
  return min(max(k, 0), fb.H);
}

// Exact bin by binary search over the running max; reached only on the slow
// path of a wave in which some guess failed its check (nothing from the fast
// check is reused, so none of it is kept live for this path).
__device__ __forceinline__ int bin_fix(float v, const FastBin& fb) {
  int lo = 0, hi = fb.H;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (v <= fb.R[mid]) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// Keys of a fetched row.  The loaded registers are always consumed (validity
// is applied afterwards with selects), so no load is left pending on any
// path.  CHECK=false skips the selects for rows known to be inside the grid.
// Float rows: every value takes one pair-table read; if any guess of the wave
// is wrong, one branch fixes all six of the lane's keys.
template <int DT, int VEC, bool CHECK = true>
__device__ __forceinline__ void row_keys(const RawRow<DT, VEC>& raw, bool valid, bool has_l, bool has_r,
                                         int trash, const FastBin& fb, int (&k)[VEC], int& kl, int& kr) {
  if constexpr (DT == 0) {
    unsigned int w[VEC / 4];
    if constexpr (VEC == 16) { w[0] = raw.v.x; w[1] = raw.v.y; w[2] = raw.v.z; w[3] = raw.v.w; }
    else if constexpr (VEC == 8) { w[0] = raw.v.x; w[1] = raw.v.y; }
    else { w[0] = raw.v; }
#pragma unroll
    for (int j = 0; j < VEC; ++j) k[j] = (int)((w[j >> 2] >> (8 * (j & 3))) & 0xffu);
    kl = (int)raw.l;
    kr = (int)raw.r;
  } else {
    // the left edge value is only needed by lane 0 and the right one by lane
    // 63, so both share one binning slot
    const bool lane0 = (threadIdx.x & 63) == 0;
    const float v[5] = {raw.v.x, raw.v.y, raw.v.z, raw.v.w, lane0 ? raw.l : raw.r};
    // every check is evaluated (bitwise, not short-circuit) so the five
    // table reads issue back to back as 64-bit loads with one wait
    int g[5];
    bool ok = true;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      g[j] = bin_guess(v[j], fb);
      const float2 p = fb.P[g[j]];
      ok = ok & (p.x < v[j]) & (v[j] <= p.y);
    }
    if (!ok) {
#pragma unroll
      for (int j = 0; j < 5; ++j) g[j] = bin_fix(v[j], fb);
    }
    k[0] = g[0];
    k[1] = g[1];
    k[2] = g[2];
    k[3] = g[3];
    kl = g[4];
    kr = g[4];
  }
  if constexpr (CHECK) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) k[j] = valid ? k[j] : trash;
  }
  kl = (valid && has_l) ? kl : trash;
  kr = (valid && has_r) ? kr : trash;
}

// ------------------------------------------------------------------- 2D
// One row step of a 2D wave tile: cur/nxt keys of rows y and y+1
// (lane-local), edge keys from outside the chunk; two telescoped sequences
// (the row and the max of the two rows) go to the histogram.
template <int VEC, int C, bool ADDR = false>
__device__ __forceinline__ void row2d(const int (&cur)[VEC], int cl, int cr, const int (&nxt)[VEC], int nl,
                                      int nr, int* hist, int lofs) {
  int s2[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) s2[j] = max(cur[j], nxt[j]);
  tele_add<VEC, C, ADDR>(cur, from_left(cur[VEC - 1], cl), from_right(cur[0], cr), 1, hist, lofs);
  tele_add<VEC, C, ADDR>(s2, from_left(s2[VEC - 1], max(cl, nl)), from_right(s2[0], max(cr, nr)), -1,
                         hist, lofs);
}

// Wave tile of aligned rows.  Rows ys..ye-1 are processed, row ye is the
// halo.  Rows past the grid are loaded from the last row (always a valid
// address) and turned into trash keys.  PARTIAL: the column chunk runs past
// the row end (narrow grids, the last chunk of a row).  Aligned rows hold a
// whole number of lane vectors, so a lane is wholly inside or wholly past the
// row; lanes past it load the chunk's first vector and carry trash keys,
// which also makes them the out-of-grid right neighbour of the last real
// column.
template <int DT, int VEC, int C, bool PARTIAL = false>
__device__ __forceinline__ void tile2d_fast(const typename Elem<DT>::T* grid, int64_t ny, int64_t nx,
                                            int64_t ys, int64_t ye, int64_t xb, int lane, int lofs,
                                            int* hist, int trash, const FastBin& fb) {
  using T = typename Elem<DT>::T;
  constexpr int64_t CHUNK = 64 * VEC;
  // uint8 grids carry keys as LDS counter addresses (see tele_add): the
  // address is formed once per value instead of once per histogram update
  constexpr bool ADDR = DT == 0;
  const unsigned int abase = (unsigned int)(size_t)(lds_int*)hist + 4u * (unsigned int)lofs;
  auto to_addr = [&](int (&k)[VEC], int& kl, int& kr) {
    if constexpr (ADDR) {
#pragma unroll
      for (int j = 0; j < VEC; ++j) k[j] = (int)(abase + 4u * C * (unsigned int)k[j]);
      kl = (int)(abase + 4u * C * (unsigned int)kl);
      kr = (int)(abase + 4u * C * (unsigned int)kr);
    }
  };
  const bool has_l = xb > 0, has_r = xb + CHUNK < nx;
  // Keys of a fetched row as counter addresses.  For bytes the address
  // abase + 4C * byte is one unsigned byte dot product per value: the byte's
  // word against a word holding 4C in that byte's place, accumulated onto
  // abase.
  auto keys = [&](const RawRow<DT, VEC>& raw, bool valid, auto check, int (&k)[VEC], int& kl, int& kr) {
    if constexpr (ADDR && 4 * C <= 255 && VEC == 16) {
      const unsigned int w[4] = {raw.v.x, raw.v.y, raw.v.z, raw.v.w};
#pragma unroll
      for (int j = 0; j < VEC; ++j)
        k[j] = (int)__builtin_amdgcn_udot4(w[j >> 2], (4u * C) << (8 * (j & 3)), abase, false);
      const int ta = (int)(abase + 4u * C * (unsigned int)trash);
      kl = (valid && has_l) ? (int)(abase + 4u * C * (unsigned int)raw.l) : ta;
      kr = (valid && has_r) ? (int)(abase + 4u * C * (unsigned int)raw.r) : ta;
      if constexpr (decltype(check)::value) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) k[j] = valid ? k[j] : ta;
      }
    } else {
      row_keys<DT, VEC, decltype(check)::value>(raw, valid, has_l, has_r, trash, fb, k, kl, kr);
      to_addr(k, kl, kr);
    }
  };
  const int64_t xl = has_l ? xb - 1 : xb, xr = has_r ? xb + CHUNK : xb;
  const bool lane_in = !PARTIAL || xb + (int64_t)lane * VEC < nx;
  const int vlane = lane_in ? lane : 0;  // lanes past the row end load a valid vector
  const T* lastrow = grid + (ny - 1) * nx;
  auto rowp = [&](int64_t y) { return y < ny ? grid + y * nx : lastrow; };
  // D rows of loads in flight.  Prefetches past the tile's halo row reload
  // the halo row (a cache hit) instead of reading rows the tile never uses.
  constexpr int D = 4;
  auto ahead = [&](int64_t r) { return rowp(r < ye ? r : ye); };
  RawRow<DT, VEC> q[D];
  int cur[VEC], cl, cr;
  {
    RawRow<DT, VEC> r0;
    fetch_row<DT, VEC>(r0, rowp(ys), xb, vlane, xl, xr);
#pragma unroll
    for (int K = 0; K < D; ++K) fetch_row<DT, VEC>(q[K], ahead(ys + 1 + K), xb, vlane, xl, xr);
    keys(r0, lane_in, std::true_type{}, cur, cl, cr);
  }
  int nxt[VEC], nl, nr;
  auto step = [&]() {
    row2d<VEC, C, ADDR>(cur, cl, cr, nxt, nl, nr, hist, lofs);
#pragma unroll
    for (int j = 0; j < VEC; ++j) cur[j] = nxt[j];
    cl = nl;
    cr = nr;
  };
  // main loop: D rows per trip, every "next" row inside the grid; each
  // stage's load is consumed in place and refilled D rows ahead (a register
  // copy of an in-flight load would make the wave wait for it)
  int64_t y = ys;
  for (; y + D <= ye && y + D < ny; y += D) {
#pragma unroll
    for (int K = 0; K < D; ++K) {
      keys(q[K], lane_in, std::integral_constant<bool, PARTIAL>{}, nxt, nl, nr);
      fetch_row<DT, VEC>(q[K], ahead(y + K + D + 1), xb, vlane, xl, xr);
      step();
    }
  }
  // remainder: fewer than D rows, checked against the tile and grid ends
#pragma unroll
  for (int K = 0; K < D; ++K) {
    if (y + K < ye) {
      keys(q[K], lane_in && y + K + 1 < ny, std::true_type{}, nxt, nl, nr);
      step();
    }
  }
}

// Any wave tile (edges, unaligned rows): element loads with bounds checks.
template <int DT, int VEC, int C>
__device__ __forceinline__ void tile2d_generic(const typename Elem<DT>::T* grid, int64_t ny, int64_t nx,
                                               int64_t ys, int64_t ye, int64_t xb, int lane, int lofs,
                                               int* hist, bool vok, const BinCtx& bc) {
  using T = typename Elem<DT>::T;
  constexpr int64_t CHUNK = 64 * VEC;
  const int64_t x0 = xb + lane * VEC;
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
    int s2[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) s2[j] = max(cur[j], nxt[j]);
    tele_add<VEC, C>(cur, from_left(cur[VEC - 1], curL), from_right(cur[0], curR), 1, hist, lofs);
    tele_add<VEC, C>(s2, from_left(s2[VEC - 1], max(curL, nxtL)), from_right(s2[0], max(curR, nxtR)), -1,
                     hist, lofs);
#pragma unroll
    for (int j = 0; j < VEC; ++j) cur[j] = nxt[j];
    curL = nxtL;
    curR = nxtR;
  }
}

struct Lds {
  int* flag;       // [0] last-workgroup flag, [1] bucket table usable
  int* hist;       // sweep: C interleaved copies of nbins+1 int32 counters
  float* scan;     // setup: NT scratch values (over the histogram, before it is cleared)
  long long* tot;  // flush: nbins totals          } over everything after the flag,
  long long* tmp;  // flush: NT scratch values     } which is dead once the
  long long* ch;   // uint8 flush: NT value counts } sweep is over
  float* R;
  float2* P;       // pair table, or
  float2* lut;     // bucket table (same LDS)
};

__host__ __device__ inline size_t align16(size_t b) { return (b + 15) & ~(size_t)15; }

// LDS: flag (16 bytes, so the histogram sits at a compile-time offset that
// folds into every ds_add) | histogram | R | X.  X holds either the bucket
// table (nlut entries) or, when there is none or it cannot be used, the pair
// table P (H+1 entries).  Setup scratch overlays the histogram before it is
// cleared; the flush's totals and scratch overlay everything after the flag.
__host__ __device__ inline size_t lds_flush_offset(int nbins) {
  return 16 + align16((size_t)nbins * sizeof(long long));
}

__host__ __device__ inline size_t lds_layout(int DT, int nbins, int C, int H, int nlut, int NT,
                                             size_t* off_R, size_t* off_X) {
  size_t hist = (size_t)(nbins + 1) * C * sizeof(int);
  if (hist < (size_t)NT * sizeof(long long)) hist = (size_t)NT * sizeof(long long);
  size_t b = 16 + align16(hist);
  *off_R = b;
  if (DT == 1) b = align16(b + (size_t)H * sizeof(float));
  *off_X = b;
  if (DT == 1) b += (size_t)(nlut > H + 1 ? nlut : H + 1) * sizeof(float2);
  const size_t flush = lds_flush_offset(nbins) + 2 * (size_t)NT * sizeof(long long);
  return b > flush ? b : flush;
}

// ------------------------------------------------------------ bucket table
// Exact binning with one table read for float grids.  A monotone map
//     bucket(v) = clamp(round(v * mul + add), 0, n-1)
// splits the line into n buckets.  It is evaluated as one fma whose addend
// carries a bias of 2^23: the sum then lies where float32 holds exactly the
// integers, so the fma's own rounding is the round() above, the clamp is a
// med3 with biased bounds, and the bucket is the float's bit pattern minus
// that of 2^23 (no conversion instruction).  NaN clamps to the low bound.  If no two thresholds R_k share a bucket,
// then for v in bucket j every R_k in an earlier bucket is < v and every R_k
// in a later one is > v, so
//     bin(v) = #{k : R_k < v} = base[j] + [v > thr[j]],
// with base[j] = #{k : bucket(R_k) < j} and thr[j] the threshold in bucket j
// (+inf if none).  The table is built per workgroup from R with the same
// bucket() code the sweep uses; the flag says whether the thresholds met the
// one-per-bucket condition (with finite, increasing end points), otherwise
// the sweep takes the checked path.
struct LutBin {
  const float2* lut;  // (thr, LDS byte address of bin base's counters, as int bits)
  float mul, add, hi; // add and hi carry the 2^23 bias
  unsigned int tbase; // LDS byte address of the table minus 8 x (bit pattern of 2^23)
  int lo4, hi4;       // this lane's copy offset in bytes, and that plus one bin's stride
};

constexpr float kLutBias = 8388608.0f;        // 2^23
constexpr unsigned int kLutBiasBits = 0x4B000000u;

// Bit pattern of bias + bucket(v), in [bits(2^23), bits(2^23) + n - 1].
__device__ __forceinline__ unsigned int lut_bits(float v, const LutBin& lb) {
  return __float_as_uint(__builtin_amdgcn_fmed3f(fmaf(v, lb.mul, lb.add), kLutBias, lb.hi));
}

__device__ __forceinline__ int lut_bucket(float v, const LutBin& lb) {
  return (int)(lut_bits(v, lb) - kLutBiasBits);
}

typedef __attribute__((address_space(3))) const unsigned long long lds_u64;

// The table entry of v's bucket, addressed with one shift-add of the bits.
__device__ __forceinline__ float2 lut_entry(float v, const LutBin& lb) {
  const unsigned long long w = *(lds_u64*)(size_t)(lut_bits(v, lb) * 8u + lb.tbase);
  return make_float2(__uint_as_float((unsigned int)w), __uint_as_float((unsigned int)(w >> 32)));
}

// Key of v: the LDS byte address of this lane's counter for bin(v).
__device__ __forceinline__ int lut_key(float v, const LutBin& lb) {
  const float2 e = lut_entry(v, lb);
  return __float_as_int(e.y) + ((v > e.x) ? lb.hi4 : lb.lo4);
}

// Exact key by binary search over the running max R (any thresholds): the
// number of R_k below v, found with a fixed, wave-uniform number of steps.
struct SearchBin {
  const float* R;
  int H;
  int top;         // largest power of two <= H (0 if H == 0)
  int base;        // LDS byte address of bin 0 for this lane's copy
  int stride;      // bytes per bin (4 C)
};

__device__ __forceinline__ int search_key(float v, const SearchBin& sb) {
  int k = 0;
  for (int step = sb.top; step > 0; step >>= 1)
    if (k + step <= sb.H && sb.R[k + step - 1] < v) k += step;
  return sb.base + k * sb.stride;
}

// Table modes (left in the first flag word given): 0 none, 1 one threshold per bucket (entries (thr,
// address of bin base)), 2 at most kMaxPerBucket per bucket (entries (count,
// base index)): bin(v) = base + #{thresholds of v's bucket below v}, which is
// exact for the same reason.
constexpr int kMaxPerBucket = 8;

template <int NT>
__device__ __forceinline__ void build_lut(const float* R, int H, int n, float2* lut, int* flag,
                                          LutBin& lb, unsigned int hist_addr, unsigned int stride) {
  const float lo = R[0], hi = R[H - 1];
  const float INF = __builtin_inff();
  float mul = 0.0f, add = 0.0f;
  bool ok = H >= 2 && lo > -INF && hi < INF && hi > lo;
  if (ok) {
    mul = (float)(n - 1) / (hi - lo);
    add = -lo * mul;
    ok = mul > 0.0f && mul < INF && add > -INF && add < INF;
  }
  if (!ok) { mul = 0.0f; add = 0.0f; }
  lb.mul = mul;
  lb.add = add + kLutBias;
  lb.hi = kLutBias + (float)(n - 1);
  lb.lut = lut;
  lb.tbase = (unsigned int)(size_t)(lds_u64*)lut - 8u * kLutBiasBits;
  if (threadIdx.x == 0) { flag[0] = ok ? 1 : 0; flag[1] = 1; }
  __syncthreads();
  if (!flag[0]) return;  // uniform: every thread read the same flag
  // thresholds in the fullest bucket (counted from the first of each run, capped)
  auto run = [&](int k, int bk) {
    int c = 1;
    while (c <= kMaxPerBucket && k + c < H && lut_bucket(R[k + c], lb) == bk) ++c;
    return c;
  };
  int worst = 1;
  for (int k = threadIdx.x; k < H; k += NT) {
    const int bk = lut_bucket(R[k], lb);
    if (k == 0 || lut_bucket(R[k - 1], lb) < bk) worst = max(worst, run(k, bk));
  }
  if (worst > 1) atomicMax(&flag[1], worst);
  __syncthreads();
  const int mode = flag[1] == 1 ? 1 : (flag[1] <= kMaxPerBucket ? 2 : 0);
  __syncthreads();
  if (threadIdx.x == 0) flag[0] = mode;
  if (mode == 0) { __syncthreads(); return; }
  for (int k = threadIdx.x; k <= H; k += NT) {
    const int bprev = k > 0 ? lut_bucket(R[k - 1], lb) : -1;
    const int bk = k < H ? lut_bucket(R[k], lb) : n - 1;
    for (int j = bprev + 1; j <= bk; ++j) {
      const bool here = k < H && j == bk;  // threshold k is the first one of bucket j
      if (mode == 1)
        lut[j] = make_float2(here ? R[k] : INF, __int_as_float((int)(hist_addr + stride * (unsigned int)k)));
      else
        lut[j] = make_float2(__int_as_float(here ? run(k, bk) : 0), __int_as_float(k));
    }
  }
  __syncthreads();
}

template <int DT, int C, int NT>
__device__ __forceinline__ Lds setup_lds(unsigned char* smem, const HardArgs& a, int nbins, int nlut,
                                         BinCtx& bc, FastBin& fb, LutBin& lb) {
  size_t oR, oX;
  lds_layout(DT, nbins, C, a.H, nlut, NT, &oR, &oX);
  Lds L;
  L.flag = reinterpret_cast<int*>(smem);
  L.hist = reinterpret_cast<int*>(smem + 16);
  L.scan = reinterpret_cast<float*>(smem + 16);
  L.tot = reinterpret_cast<long long*>(smem + 16);
  L.tmp = reinterpret_cast<long long*>(smem + lds_flush_offset(nbins));
  L.ch = L.tmp + NT;
  L.R = reinterpret_cast<float*>(smem + oR);
  L.P = reinterpret_cast<float2*>(smem + oX);
  L.lut = reinterpret_cast<float2*>(smem + oX);
  if (threadIdx.x == 0) L.flag[1] = 0;
  setup_bins<DT, NT>(a, L.R, L.scan, bc, nbins);  // ends with a barrier
  for (int i = threadIdx.x; i < (nbins + 1) * C; i += NT) L.hist[i] = 0;
  fb.P = L.P;
  fb.R = L.R;
  fb.H = a.H;
  fb.mul = bc.scale;
  fb.add = -bc.r0 * bc.scale;
  if (!(fb.add > -__builtin_inff() && fb.add < __builtin_inff())) { fb.mul = 0.0f; fb.add = 0.0f; }
  lb.lut = L.lut;
  lb.mul = 0.0f;
  lb.add = lb.hi = kLutBias;
  lb.tbase = (unsigned int)(size_t)(lds_u64*)L.lut - 8u * kLutBiasBits;
  lb.lo4 = 4 * ((threadIdx.x & 63) & (C - 1));
  lb.hi4 = lb.lo4 + 4 * C;
  __syncthreads();
  if constexpr (DT == 1) {
    if (nlut > 0)
      build_lut<NT>(L.R, a.H, nlut, L.lut, L.flag + 1, lb, (unsigned int)(size_t)(lds_int*)L.hist,
                    4u * (unsigned int)C);  // leaves the table mode in flag[1]
    // the pair table is only needed when the bucket table is not used
    if (!L.flag[1]) build_pairs<NT>(L.R, a.H, L.P);
  }
  __syncthreads();
  return L;
}

// Tiles of this workgroup: t = first, first + step, ... while t < end.  The
// dispatcher hands workgroups to the chip's 8 XCDs in turn (linear id mod 8)
// and each XCD has its own L2.  With at least 8 workgroups, XCD x takes the
// x-th eighth of the tile range, split over its own workgroups, so tiles
// that are neighbours in x (and mostly in y and z) run on one XCD: the edge
// columns and halo rows that each reads from the other come from that XCD's
// L2 instead of HBM, and every XCD still gets an equal share of the tiles.
// (Tile counts are 32-bit: the launchers refuse 2^31 tiles or more, which only a
// grid of a few columns and more than 2^36 rows could need.)
struct TileRange {
  int first, end, step;
};

__device__ __forceinline__ TileRange tile_range(int64_t ntiles64) {
  constexpr int X = 8;
  const int b = (int)blockIdx.x, g = (int)gridDim.x, ntiles = (int)ntiles64;
  if (g < X) return TileRange{b, ntiles, g};
  const int x = b % X, j = b / X;
  const int nwg = g / X + (x < g % X ? 1 : 0);  // workgroups on this XCD
  const int lo = x * (ntiles / X) + (x < ntiles % X ? x : ntiles % X);
  const int hi = lo + ntiles / X + (x < ntiles % X ? 1 : 0);
  return TileRange{lo + j, hi, nwg};
}

// The grid of a batch that this workgroup row works on.
__device__ __forceinline__ void batch_slice(HardArgs& a) {
  const int64_t b = blockIdx.y;
  const size_t esz = a.dtype == 0 ? 1 : 4;
  a.grid = reinterpret_cast<const char*>(a.grid) + (size_t)b * (size_t)(a.nz * a.ny * a.nx) * esz;
  a.tau += b * a.tau_stride;
  a.out += b * a.H;
  a.ws = reinterpret_cast<char*>(a.ws) + (size_t)b * a.ws_stride;
}

template <int DT, int VEC, int C, int TH, int NT>
__global__ __launch_bounds__(NT) void hard2d_kernel(HardArgs a, int nbins, int64_t ntx, int64_t ntiles,
                                                    int vec_ok, int th) {
  extern __shared__ __align__(16) unsigned char smem[];
  using T = typename Elem<DT>::T;
  batch_slice(a);
  BinCtx bc;
  FastBin fb;
  LutBin lb;
  Lds L = setup_lds<DT, C, NT>(smem, a, nbins, 0, bc, fb, lb);

  const T* grid = reinterpret_cast<const T*>(a.grid);
  const int64_t ny = a.ny, nx = a.nx;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int lofs = lane & (C - 1);
  constexpr int64_t CHUNK = 64 * VEC;
  const bool vok = vec_ok != 0;

  // th == TH (large grids) keeps the tile height a compile-time constant,
  // which lets the compiler schedule the unrolled row loop as a whole
  auto sweep = [&](auto thc) {
    const int64_t h = thc.value > 0 ? (int64_t)thc.value : (int64_t)th;
    for (TileRange tr = tile_range(ntiles); tr.first < tr.end; tr.first += tr.step) {
      const int64_t t = tr.first;
      const int64_t tx = t % ntx, tyb = t / ntx;
      const int64_t ys = (tyb * (NT / 64) + wave) * h;
      if (ys >= ny) continue;
      const int64_t ye = ys + h < ny ? ys + h : ny;
      const int64_t xb = tx * CHUNK;
      if (vok && xb + CHUNK <= nx)
        tile2d_fast<DT, VEC, C>(grid, ny, nx, ys, ye, xb, lane, lofs, L.hist, nbins, fb);
      else if (vok)
        tile2d_fast<DT, VEC, C, true>(grid, ny, nx, ys, ye, xb, lane, lofs, L.hist, nbins, fb);
      else
        tile2d_generic<DT, VEC, C>(grid, ny, nx, ys, ye, xb, lane, lofs, L.hist, vok, bc);
    }
  };
  if (th == TH)
    sweep(std::integral_constant<int, TH>{});
  else
    sweep(std::integral_constant<int, 0>{});
  flush_and_finish<DT, C, NT>(a, nbins, L.hist, L.tmp, L.ch, L.flag, L.tot);
}

// ------------------------------------------------------------------- 3D
// Wave tile: a chunk of 64*VEC columns x TY rows x a range of planes.  The
// wave marches along z holding the keys of TY+1 rows (TY plus a one-row
// halo) of planes z and z+1; the raw rows of plane z+2 are in flight while
// plane z is processed.
template <int DT, int VEC, int C, int TY, bool ADDR = false>
__device__ __forceinline__ void rows3d(int (&A)[TY + 1][VEC], int (&AL)[TY + 1], int (&AR)[TY + 1],
                                       int (&B)[TY + 1][VEC], int (&BL)[TY + 1], int (&BR)[TY + 1],
                                       int64_t ys, int64_t ny, int* hist, int lofs) {
#pragma unroll
  for (int r = 0; r < TY; ++r) {
    if (ys + r < ny) {
      int s2[VEC], s3[VEC], s4[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        s2[j] = max(A[r][j], A[r + 1][j]);
        s3[j] = max(A[r][j], B[r][j]);
        s4[j] = max(s2[j], max(B[r][j], B[r + 1][j]));
      }
      const int e2l = max(AL[r], AL[r + 1]), e3l = max(AL[r], BL[r]), e4l = max(e2l, max(BL[r], BL[r + 1]));
      const int e2r = max(AR[r], AR[r + 1]), e3r = max(AR[r], BR[r]), e4r = max(e2r, max(BR[r], BR[r + 1]));
      tele_add<VEC, C, ADDR>(A[r], from_left(A[r][VEC - 1], AL[r]), from_right(A[r][0], AR[r]), 1, hist, lofs);
      tele_add<VEC, C, ADDR>(s2, from_left(s2[VEC - 1], e2l), from_right(s2[0], e2r), -1, hist, lofs);
      tele_add<VEC, C, ADDR>(s3, from_left(s3[VEC - 1], e3l), from_right(s3[0], e3r), -1, hist, lofs);
      tele_add<VEC, C, ADDR>(s4, from_left(s4[VEC - 1], e4l), from_right(s4[0], e4r), 1, hist, lofs);
    }
  }
}

template <int DT, int VEC, int C, int TY>
__device__ __forceinline__ void tile3d_fast(const typename Elem<DT>::T* grid, int64_t nz, int64_t ny,
                                            int64_t nx, int64_t zs, int64_t ze, int64_t ys, int64_t xb,
                                            int lane, int lofs, int* hist, int trash, const FastBin& fb) {
  constexpr int64_t CHUNK = 64 * VEC;
  const int64_t plane = ny * nx;
  const bool has_l = xb > 0, has_r = xb + CHUNK < nx;
  const int64_t xl = has_l ? xb - 1 : xb, xr = has_r ? xb + CHUNK : xb;
  using T = typename Elem<DT>::T;
  int64_t roff[TY + 1];  // element offsets of the rows in plane 0 (scalar registers)
#pragma unroll
  for (int r = 0; r <= TY; ++r) roff[r] = uni64((ys + r < ny ? ys + r : ny - 1) * nx);
  auto rowp = [&](int64_t z, int r) -> const T* {
    return grid + uni64((z < nz ? z : nz - 1) * plane + roff[r]);
  };
  RawRow<DT, VEC> raw[TY + 1];
  int A[TY + 1][VEC], AL[TY + 1], AR[TY + 1], B[TY + 1][VEC], BL[TY + 1], BR[TY + 1];
#pragma unroll
  for (int r = 0; r <= TY; ++r) fetch_row<DT, VEC>(raw[r], rowp(zs, r), xb, lane, xl, xr);
#pragma unroll
  for (int r = 0; r <= TY; ++r) row_keys<DT, VEC>(raw[r], ys + r < ny, has_l, has_r, trash, fb, A[r], AL[r], AR[r]);
#pragma unroll
  for (int r = 0; r <= TY; ++r) fetch_row<DT, VEC>(raw[r], rowp(zs + 1, r), xb, lane, xl, xr);
  const bool rows_in = ys + TY < ny;
  // One plane step: keys of plane z+1 into Y (from the raw rows fetched one
  // step earlier), fetch of plane z+2, then the rows of plane z (X) against
  // plane z+1 (Y).  (Unrolling twice to swap X and Y instead of copying was
  // measured slower: the doubled loop body costs more than the moves.)
#define ECC_PLANE_STEP(X, XL, XR, Y, YL, YR, ZZ)                                              \
  {                                                                                           \
    const bool zn = (ZZ) + 1 < nz;                                                            \
    if (zn && rows_in) {                                                                      \
      _Pragma("unroll") for (int r = 0; r <= TY; ++r)                                         \
        row_keys<DT, VEC, false>(raw[r], true, has_l, has_r, trash, fb, Y[r], YL[r], YR[r]);   \
    } else {                                                                                  \
      _Pragma("unroll") for (int r = 0; r <= TY; ++r)                                         \
        row_keys<DT, VEC, true>(raw[r], zn && ys + r < ny, has_l, has_r, trash, fb, Y[r],      \
                                YL[r], YR[r]);                                                \
    }                                                                                         \
    _Pragma("unroll") for (int r = 0; r <= TY; ++r)                                           \
      fetch_row<DT, VEC>(raw[r], rowp((ZZ) + 2, r), xb, lane, xl, xr);                        \
    rows3d<DT, VEC, C, TY>(X, XL, XR, Y, YL, YR, ys, ny, hist, lofs);                         \
  }
  for (int64_t z = zs; z < ze; ++z) {
    ECC_PLANE_STEP(A, AL, AR, B, BL, BR, z)
#pragma unroll
    for (int r = 0; r <= TY; ++r) {
#pragma unroll
      for (int j = 0; j < VEC; ++j) A[r][j] = B[r][j];
      AL[r] = BL[r];
      AR[r] = BR[r];
    }
  }
#undef ECC_PLANE_STEP
}

// Float tile with bucket-table binning (tile3d_lut below).  The wave holds the
// keys of TY+1 rows (TY plus the one-row y halo) of planes z and z+1 and
// marches along z; the raw rows of plane z+2 are in flight while plane z is
// processed.  The values just outside the wave's column chunk (one per row and
// side) are loaded and binned once per plane in a few edge lanes and moved to
// lanes 0 and 63 by DPP row shifts.  Row and plane validity is wave-uniform and
// handled by branches.  The z loop is unrolled twice so that planes z and z+1
// swap roles instead of being copied.
// Compile-time loop (DPP controls must be constants).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Value of lane R to lane 0 (row_shl:R, first row only) and of lane 63-R to
// lane 63 (row_shr:R, last row only); other lanes keep v.
template <int R>
__device__ __forceinline__ int edges_to_ends(int v) {
  const int l = __builtin_amdgcn_update_dpp(v, v, 0x100 + R, 0x1, 0xF, false);
  return __builtin_amdgcn_update_dpp(l, v, 0x110 + R, 0x8, 0xF, false);
}

template <int VEC>
struct RawLut {
  float v[VEC];
};

// SCALAR: element loads with the column clamped to the grid, and trash keys
// for columns past its end, for a chunk that sticks out of the grid or rows
// that are not 16-byte aligned.
// KEY maps a value to its key (the LDS address of this lane's counter for
// its bin): the bucket table, a per-bucket scan, or a binary search.
// With VEC = 8 a wave would cover a whole row of up to 512 values, with no
// neighbouring chunks and no edge values to load or bin.
// partial (wave-uniform; vector loads only): the chunk of aligned rows runs
// past the row end.  A lane then lies wholly inside or wholly past it (rows
// hold whole vectors); lanes past it load the chunk's first vector and carry
// trash keys, which also makes them the out-of-grid right neighbour of the
// last real column.  Callers pass a constant, so each call site inlines its
// own copy and full chunks carry no per-value select.
template <int VEC, int C, int TY, bool SCALAR, typename KEY>
__device__ __forceinline__ void tile3d_lut(const float* grid, int64_t nz, int64_t ny, int64_t nx, int64_t zs,
                                           int64_t ze, int64_t ys, int64_t xb, int lane, int lofs, int* hist,
                                           int trash_bin, const LutBin& lb, KEY key, bool partial = false) {
  static_assert(VEC == 4 || VEC == 8, "float rows are loaded as float4");
  constexpr bool EDGES = VEC == 4;
  // keys are LDS byte addresses of this lane's counters (see tele_add)
  const int trash = (int)((unsigned int)(size_t)(lds_int*)hist + 4u * (unsigned int)(C * trash_bin)) + lb.lo4;
  constexpr int64_t CHUNK = 64 * VEC;
  const int64_t plane = ny * nx;
  const bool has_l = xb > 0, has_r = xb + CHUNK < nx;
  // byte offset of the vector from the element just left of the chunk (lanes
  // past the row end of a partial chunk read lane 0's)
  const bool lane_in = !partial || xb + (int64_t)VEC * lane < nx;
  const unsigned int voff = 4u + 4u * VEC * (unsigned int)(lane_in ? lane : 0);
  // Edge values (the columns just outside the chunk, needed by lanes 0 and
  // 63) are loaded and binned once per plane for all TY+1 rows: lane r holds
  // row r's left edge, lane 63-r row r's right edge.  Their keys carry the
  // copy offset of the lane that uses them (0 or 63).  A missing edge (grid
  // border) reads a valid element and gets the trash key.
  const int erow = lane <= TY ? lane : (63 - lane <= TY ? 63 - lane : 0);
  const bool eleft = lane <= TY;
  const bool eok = eleft ? has_l : has_r;
  const int64_t ecol = eleft ? (has_l ? xb - 1 : xb) : (has_r ? xb + CHUNK : xb);
  const int64_t eoff64 = (ys + erow < ny ? ys + erow : ny - 1) * nx + ecol;  // element offset in a plane
  const int elo = 4 * ((eleft ? 0 : 63) & (C - 1));                         // user lane's copy offset
  const int etrash = trash - lb.lo4 + elo;
  int64_t roff[TY + 1];
#pragma unroll
  for (int r = 0; r <= TY; ++r) roff[r] = uni64((ys + r < ny ? ys + r : ny - 1) * nx + xb - 1);
  // SCALAR: last valid column relative to the chunk start; the clamped
  // offsets and column checks are recomputed where used (cheaper than
  // keeping more values live through the loop)
  const int lim = (int)(nx - 1 - xb < CHUNK ? nx - 1 - xb : CHUNK - 1);
  auto coff = [&](int j) { return 4u + 4u * (unsigned int)min(VEC * lane + j, lim); };
  auto cok = [&](int j) { return VEC * lane + j <= lim; };
  auto fetch = [&](RawLut<VEC>& q, int64_t z, int r) {
    const char* base = reinterpret_cast<const char*>(grid + uni64((z < nz ? z : nz - 1) * plane + roff[r]));
    if constexpr (SCALAR) {
#pragma unroll
      for (int j = 0; j < VEC; ++j) q.v[j] = *reinterpret_cast<const float*>(base + coff(j));
    } else {
#pragma unroll
      for (int h = 0; h < VEC / 4; ++h) {
        const float4 w = *reinterpret_cast<const float4*>(base + voff + 16u * h);
        q.v[4 * h] = w.x;
        q.v[4 * h + 1] = w.y;
        q.v[4 * h + 2] = w.z;
        q.v[4 * h + 3] = w.w;
      }
    }
  };
  auto fetch_edges = [&](float& e, int64_t z) {
    e = grid[(z < nz ? z : nz - 1) * plane + eoff64];
  };
  auto keys = [&](const RawLut<VEC>& q, bool row_ok, int (&k)[VEC]) {
    if (row_ok) {
#pragma unroll
      for (int j = 0; j < VEC; ++j) k[j] = key(q.v[j]);
      if constexpr (SCALAR) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) k[j] = cok(j) ? k[j] : trash;
      } else if (partial) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) k[j] = lane_in ? k[j] : trash;
      }
    } else {
#pragma unroll
      for (int j = 0; j < VEC; ++j) k[j] = trash;
    }
  };
  // edge keys of plane z for every row: one binning in the edge lanes, then
  // row-masked DPP row shifts bring row r's left edge to lane 0 (from lane r)
  // and its right edge to lane 63 (from lane 63-r)
  auto edge_keys = [&](float e, bool plane_ok, int (&E)[TY + 1]) {
    int ke = key(e) - lb.lo4 + elo;
    ke = (plane_ok && eok && ys + erow < ny) ? ke : etrash;
    E[0] = ke;
    static_for<1, TY + 1>([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      E[r] = edges_to_ends<r>(ke);
    });
  };
  RawLut<VEC> raw[TY + 1];
  float rawe = 0.0f;
  int A[TY + 1][VEC], AE[TY + 1], B[TY + 1][VEC], BE[TY + 1];
#pragma unroll
  for (int r = 0; r <= TY; ++r) fetch(raw[r], zs, r);
  if constexpr (EDGES) fetch_edges(rawe, zs);
#pragma unroll
  for (int r = 0; r <= TY; ++r) keys(raw[r], ys + r < ny, A[r]);
  if constexpr (EDGES) {
    edge_keys(rawe, true, AE);
  } else {
#pragma unroll
    for (int r = 0; r <= TY; ++r) AE[r] = trash;
  }
#pragma unroll
  for (int r = 0; r <= TY; ++r) fetch(raw[r], zs + 1, r);
  if constexpr (EDGES) fetch_edges(rawe, zs + 1);
  // one plane step: keys of plane z+1 into Y, fetch of plane z+2, rows of
  // plane z (X) against plane z+1 (Y); two steps per trip swap X and Y
  auto step = [&](int (&X)[TY + 1][VEC], int (&XE)[TY + 1], int (&Y)[TY + 1][VEC], int (&YE)[TY + 1],
                  int64_t z) {
    const bool zn = z + 1 < nz;
#pragma unroll
    for (int r = 0; r <= TY; ++r) keys(raw[r], zn && ys + r < ny, Y[r]);
    if constexpr (EDGES) {
      edge_keys(rawe, zn, YE);
    } else {
#pragma unroll
      for (int r = 0; r <= TY; ++r) YE[r] = trash;
    }
    // the last step's prefetch reloads the halo plane (a cache hit) rather
    // than read a plane the tile never uses
    const int64_t zf = z + 2 < ze ? z + 2 : ze;
#pragma unroll
    for (int r = 0; r <= TY; ++r) fetch(raw[r], zf, r);
    if constexpr (EDGES) fetch_edges(rawe, zf);
    rows3d<1, VEC, C, TY, true>(X, XE, XE, Y, YE, YE, ys, ny, hist, lofs);
  };
  for (int64_t z = zs; z < ze; z += 2) {
    step(A, AE, B, BE, z);
    if (z + 1 >= ze) break;
    step(B, BE, A, AE, z + 1);
  }
}

template <int DT, int VEC, int C, int TY>
__device__ __forceinline__ void tile3d_generic(const typename Elem<DT>::T* grid, int64_t nz, int64_t ny,
                                               int64_t nx, int64_t zs, int64_t ze, int64_t ys, int64_t xb,
                                               int lofs, int* hist, bool vok, const BinCtx& bc, int lane) {
  using T = typename Elem<DT>::T;
  constexpr int64_t CHUNK = 64 * VEC;
  const int64_t plane = ny * nx;
  const int64_t x0 = xb + lane * VEC;
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
    rows3d<DT, VEC, C, TY>(A, AL, AR, B, BL, BR, ys, ny, hist, lofs);
#pragma unroll
    for (int r = 0; r <= TY; ++r) {
#pragma unroll
      for (int j = 0; j < VEC; ++j) A[r][j] = B[r][j];
      AL[r] = BL[r];
      AR[r] = BR[r];
    }
  }
}

// Float 3D tiles other than the hot one (bucket table with one threshold per
// bucket, aligned rows): unaligned rows (element loads), and the per-bucket
// scan and binary-search keys.  They walk
// the tile's rows two at a time (each pair with its own one-row halo), which
// keeps their live registers below the hot tile's, so the kernel's register
// allocation is set by the hot tile and needs no spills.  (With all six
// paths at four rows the kernel spilled 12 VGPRs and 56 SGPRs per wave, and
// the spill code ran in the hot loop.)
template <int VEC, int C, int TY>
__device__ __forceinline__ void tile3d_lut_other(const float* grid, int64_t nz, int64_t ny, int64_t nx,
                                                 int64_t zs, int64_t ze, int64_t ys, int64_t xb, int lane,
                                                 int lofs, int* hist, int nbins, const LutBin& lb,
                                                 const SearchBin& sb, int lut_mode, bool aligned) {
  const bool partial = xb + 64 * VEC > nx;
  for (int r = 0; r < TY && ys + r < ny; r += 2) {
    const int64_t y = ys + r;
    if (lut_mode == 1) {
      // (only unaligned rows come here with this table)
      auto key = [&](float v) { return lut_key(v, lb); };
      tile3d_lut<VEC, C, 2, true>(grid, nz, ny, nx, zs, ze, y, xb, lane, lofs, hist, nbins, lb, key);
    } else if (lut_mode == 2) {
      // bucket of v, then the few thresholds sharing it
      auto key = [&](float v) {
        const float2 e = lut_entry(v, lb);
        const int b0 = __float_as_int(e.y), c = __float_as_int(e.x);
        int k = b0;
        for (int i = 0; i < c; ++i) k += (int)(sb.R[b0 + i] < v);
        return sb.base + k * sb.stride;
      };
      if (aligned)
        tile3d_lut<VEC, C, 2, false>(grid, nz, ny, nx, zs, ze, y, xb, lane, lofs, hist, nbins, lb, key, partial);
      else
        tile3d_lut<VEC, C, 2, true>(grid, nz, ny, nx, zs, ze, y, xb, lane, lofs, hist, nbins, lb, key);
    } else {
      auto key = [&](float v) { return search_key(v, sb); };
      if (aligned)
        tile3d_lut<VEC, C, 2, false>(grid, nz, ny, nx, zs, ze, y, xb, lane, lofs, hist, nbins, lb, key, partial);
      else
        tile3d_lut<VEC, C, 2, true>(grid, nz, ny, nx, zs, ze, y, xb, lane, lofs, hist, nbins, lb, key);
    }
  }
}

// NT threads per workgroup; MINW waves per SIMD that the register budget must
// allow (so that two 512-thread workgroups share a CU).
template <int DT, int VEC, int C, int TY, int NT, int MINW>
__global__ __launch_bounds__(NT, MINW) void hard3d_kernel(HardArgs a, int nbins, int64_t ntx,
                                                          int64_t nty4, int64_t TZ, int64_t ntiles,
                                                          int vec_ok, int nlut) {
  extern __shared__ __align__(16) unsigned char smem[];
  using T = typename Elem<DT>::T;
  batch_slice(a);
  BinCtx bc;
  FastBin fb;
  LutBin lb;
  Lds L = setup_lds<DT, C, NT>(smem, a, nbins, nlut, bc, fb, lb);
  const int lut_mode = __builtin_amdgcn_readfirstlane(L.flag[1]);
  SearchBin sb;
  sb.R = L.R;
  sb.H = a.H;
  sb.top = 0;
  while (sb.top * 2 <= a.H) sb.top = sb.top ? sb.top * 2 : 1;
  sb.stride = 4 * C;
  sb.base = (int)(size_t)(lds_int*)L.hist + lb.lo4;

  const T* grid = reinterpret_cast<const T*>(a.grid);
  const int64_t nz = a.nz, ny = a.ny, nx = a.nx;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int lofs = lane & (C - 1);
  constexpr int64_t CHUNK = 64 * VEC;
  const bool vok = vec_ok != 0;

  for (TileRange tr = tile_range(ntiles); tr.first < tr.end; tr.first += tr.step) {
    const int64_t t = tr.first;
    const int64_t tx = t % ntx;
    const int64_t rest = t / ntx;
    const int64_t tyg = rest % nty4, tz = rest / nty4;
    const int64_t ys = (tyg * (NT / 64) + wave) * TY;
    if (ys >= ny) continue;
    const int64_t zs = tz * TZ;
    const int64_t ze = zs + TZ < nz ? zs + TZ : nz;
    const int64_t xb = tx * CHUNK;
    if constexpr (DT == 1) {
      if (lut_mode == 1 && vok) {
        auto key = [&](float v) { return lut_key(v, lb); };
        if (xb + CHUNK <= nx)
          tile3d_lut<VEC, C, TY, false>(grid, nz, ny, nx, zs, ze, ys, xb, lane, lofs, L.hist, nbins, lb, key);
        else
          tile3d_lut<VEC, C, TY, false>(grid, nz, ny, nx, zs, ze, ys, xb, lane, lofs, L.hist, nbins, lb, key, true);
      } else {
        tile3d_lut_other<VEC, C, TY>(grid, nz, ny, nx, zs, ze, ys, xb, lane, lofs, L.hist, nbins, lb, sb, lut_mode,
                                     vok);
      }
    } else {
      if (vok && xb + CHUNK <= nx)
        tile3d_fast<DT, VEC, C, TY>(grid, nz, ny, nx, zs, ze, ys, xb, lane, lofs, L.hist, nbins, fb);
      else
        tile3d_generic<DT, VEC, C, TY>(grid, nz, ny, nx, zs, ze, ys, xb, lofs, L.hist, vok, bc, lane);
    }
  }
  flush_and_finish<DT, C, NT>(a, nbins, L.hist, L.tmp, L.ch, L.flag, L.tot);
}

// ------------------------------------------------------------- launcher
size_t lds_bytes(int DT, int nbins, int C, int H, int nlut, int NT) {
  size_t a, b;
  return lds_layout(DT, nbins, C, H, nlut, NT, &a, &b);
}

// Bucket-table entries for H thresholds: two buckets per threshold keep
// evenly spaced thresholds in distinct buckets.
int lut_entries(int H) { return 2 * H + 2; }

// Workgroups of `kernel` that fit on one CU with `lds` bytes of LDS each
// (at most 4: the sweep is issue-bound and more workgroups only add flushes).
// Raise a kernel's dynamic-LDS limit to the whole CU once (the default is
// 64 KB); later calls cost a lookup.
hipError_t allow_lds(const void* kernel, size_t lds) {
  if (lds <= 64 * 1024) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  struct Entry { const void* k; int dev; };
  static std::mutex mu;
  static Entry done[64];
  static int used = 0;
  std::lock_guard<std::mutex> g(mu);
  for (int i = 0; i < used; ++i)
    if (done[i].k == kernel && done[i].dev == dev) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e == hipSuccess && used < 64) done[used++] = Entry{kernel, dev};
  return e;
}

// The answer is cached per (kernel, LDS size): the query costs more host
// time than a small launch takes on the GPU.
int resident_blocks(const void* kernel, int nt, size_t lds) {
  struct Entry { const void* k; size_t lds; int n; };
  static std::mutex mu;
  static Entry cache[64];
  static int used = 0;
  {
    std::lock_guard<std::mutex> g(mu);
    for (int i = 0; i < used; ++i)
      if (cache[i].k == kernel && cache[i].lds == lds) return cache[i].n;
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, nt, lds) != hipSuccess) n = 1;
  const int cap = 4 * 256 / nt;
  n = n < 1 ? 1 : (n > cap ? cap : n);
  std::lock_guard<std::mutex> g(mu);
  if (used < 64) cache[used++] = Entry{kernel, lds, n};
  return n;
}

// Workgroups worth launching for a grid of nvox voxels of esz bytes and nbins
// bins.  Every workgroup flushes up to nbins+1 device-scope atomics, so on
// small grids with many bins fewer, fuller workgroups finish sooner (at least
// one per CU); and every workgroup pays its setup and flush whatever it
// sweeps, so each should get at least 16 KiB of the grid (at least 32
// workgroups).  Measured on 1024^2 float32 with H = 256: 20 -> 12.5 us; on
// 2048^2 uint8: 18 -> 13 us; large grids are not capped.
int64_t useful_blocks(int64_t nvox, int64_t esz, int nbins, int cus) {
  int64_t v = nvox / (4 * (int64_t)(nbins + 1));
  if (v < cus) v = cus;
  int64_t by_bytes = nvox * esz / (16 * 1024);
  if (by_bytes < 32) by_bytes = 32;
  return v < by_bytes ? v : by_bytes;
}

// Threads per workgroup of the 3D float kernel.
constexpr int kNT3 = 512;

// Histogram copies of the 3D float kernel: as many as keep two 512-thread
// workgroups on a CU.  LDS serves a ds_add 32 lanes at a time; with 32
// copies interleaved by lane those lanes always hit distinct banks, with
// fewer copies random keys collide and the instruction takes several passes.
int copies3d_f32(int nbins, int H) {
  const size_t budget = 160 * 1024 / 2;
  for (int c = 32; c > 1; c >>= 1)
    if (lds_bytes(1, nbins, c, H, lut_entries(H), kNT3) <= budget) return c;
  return 1;
}

int copies_for(int dt, int nbins) {
  if (dt == 0) return 32;  // uint8: 257 keys, conflict-free layout fits in 33 KB
  const int c = 4500 / (nbins + 1);
  if (c >= 32) return 32;
  if (c >= 16) return 16;
  if (c >= 8) return 8;
  if (c >= 4) return 4;
  if (c >= 2) return 2;
  return 1;
}

// Workgroups per grid when `batch` grids share a launch that wants `total`.
int64_t per_grid_blocks(int64_t total, int64_t batch) {
  const int64_t g = (total + batch - 1) / batch;
  return g < 1 ? 1 : g;
}

// Launch `go(args, nb)` for consecutive runs of at most kMaxBatchPerLaunch
// grids, with the pointers moved to the run's first grid.
template <typename Go>
hipError_t launch_batches(const HardArgs& a, Go go) {
  const size_t esz = a.dtype == 0 ? 1 : 4;
  const size_t grid_bytes = (size_t)(a.nz * a.ny * a.nx) * esz;
  for (int64_t b0 = 0; b0 < a.batch; b0 += kMaxBatchPerLaunch) {
    const int64_t nb = a.batch - b0 < kMaxBatchPerLaunch ? a.batch - b0 : kMaxBatchPerLaunch;
    HardArgs c = a;
    c.grid = reinterpret_cast<const char*>(a.grid) + (size_t)b0 * grid_bytes;
    c.tau = a.tau + b0 * a.tau_stride;
    c.out = a.out + b0 * a.H;
    c.ws = reinterpret_cast<char*>(a.ws) + (size_t)b0 * a.ws_stride;
    go(c, (unsigned)nb);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int DT, int VEC, int C, int TH>
hipError_t launch2d(const HardArgs& a, int nbins, hipStream_t s, const DeviceInfo& di) {
  constexpr int64_t CHUNK = 64 * VEC;
  const int64_t ntx = (a.nx + CHUNK - 1) / CHUNK;
  // rows per wave: TH on large grids, fewer when that would leave the chip
  // short of workgroups (the per-wave row walk is serial)
  int64_t want = per_grid_blocks((int64_t)di.cus * 4, a.batch);
  {
    const int64_t u = useful_blocks(a.ny * a.nx, DT == 0 ? 1 : 4, nbins, di.cus);
    if (want > u) want = u;
  }
  int64_t th = (a.ny * ntx) / (want * kWavesPerBlock);
  if (th > TH) th = TH;
  if (th < 1) th = 1;
  const int64_t nty = (a.ny + th * kWavesPerBlock - 1) / (th * kWavesPerBlock);
  const int64_t ntiles = ntx * nty;
  if (ntiles > INT32_MAX) return hipErrorInvalidValue;  // the kernels count tiles in 32 bits
  const size_t esz = DT == 0 ? 1 : 4;
  const int vec_ok = (reinterpret_cast<uintptr_t>(a.grid) % (VEC * esz) == 0) &&
                     ((a.nx * (int64_t)esz) % (int64_t)(VEC * esz) == 0);
  const size_t lds = lds_bytes(DT, nbins, C, a.H, 0, kBlock);
  auto k = hard2d_kernel<DT, VEC, C, TH, kBlock>;
  {
    const hipError_t e = allow_lds(reinterpret_cast<const void*>(k), lds);
    if (e != hipSuccess) return e;
  }
  int64_t g = (int64_t)di.cus * resident_blocks(reinterpret_cast<const void*>(k), kBlock, lds);
  if (g > want) g = want;
  if (g > ntiles) g = ntiles;
  if (g < 1) g = 1;
  return launch_batches(a, [&](const HardArgs& c, unsigned nb) {
    hipLaunchKernelGGL(k, dim3((unsigned)g, nb), dim3(kBlock), lds, s, c, nbins, ntx, ntiles, vec_ok, (int)th);
  });
}

template <int DT, int VEC, int C, int TY, int NT, int MINW>
hipError_t launch3d(const HardArgs& a, int nbins, hipStream_t s, const DeviceInfo& di) {
  constexpr int64_t CHUNK = 64 * VEC;
  constexpr int64_t WAVES = NT / 64;
  const int64_t ntx = (a.nx + CHUNK - 1) / CHUNK;
  const int64_t nty4 = (a.ny + TY * WAVES - 1) / (TY * WAVES);
  // split z so that there are enough tiles to fill the chip
  int64_t want = per_grid_blocks((int64_t)di.cus * (4 * 256 / NT), a.batch);
  {
    const int64_t u = useful_blocks(a.nz * a.ny * a.nx, DT == 0 ? 1 : 4, nbins, di.cus);
    if (want > u) want = u;
  }
  int64_t ntz = (want + ntx * nty4 - 1) / (ntx * nty4);
  if (ntz < 1) ntz = 1;
  if (ntz > a.nz) ntz = a.nz;
  int64_t TZ = (a.nz + ntz - 1) / ntz;
  if (TZ < 2 && a.nz >= 2) TZ = 2;  // a tile of one plane would re-read as many halo planes as it owns
  ntz = (a.nz + TZ - 1) / TZ;
  const int64_t ntiles = ntx * nty4 * ntz;
  if (ntiles > INT32_MAX) return hipErrorInvalidValue;  // the kernels count tiles in 32 bits
  const size_t esz = DT == 0 ? 1 : 4;
  const int vec_ok = (reinterpret_cast<uintptr_t>(a.grid) % (VEC * esz) == 0) &&
                     ((a.nx * (int64_t)esz) % (int64_t)(VEC * esz) == 0);
  int nlut = DT == 1 ? lut_entries(a.H) : 0;
  if (nlut > 0 && lds_bytes(DT, nbins, C, a.H, nlut, NT) > 128 * 1024) nlut = 0;  // very large H
  const size_t lds = lds_bytes(DT, nbins, C, a.H, nlut, NT);
  auto k = hard3d_kernel<DT, VEC, C, TY, NT, MINW>;
  {
    const hipError_t e = allow_lds(reinterpret_cast<const void*>(k), lds);
    if (e != hipSuccess) return e;
  }
  int64_t g = (int64_t)di.cus * resident_blocks(reinterpret_cast<const void*>(k), NT, lds);
  if (g > want) g = want;
  if (g > ntiles) g = ntiles;
  if (g < 1) g = 1;
  return launch_batches(a, [&](const HardArgs& c, unsigned nb) {
    hipLaunchKernelGGL(k, dim3((unsigned)g, nb), dim3(NT), lds, s, c, nbins, ntx, nty4, TZ, ntiles,
                       vec_ok, nlut);
  });
}

template <int C>
hipError_t dispatch_f32(const HardArgs& a, int nbins, hipStream_t s, const DeviceInfo& di) {
  if (a.nz == 1) return launch2d<1, 4, C, 16>(a, nbins, s, di);
  // (a whole-row variant, 8 values per lane without chunk edges, was measured:
  // it needs more than 128 VGPRs even at two rows per tile)
  return launch3d<1, 4, C, 4, kNT3, 4>(a, nbins, s, di);
}

int copies_f32(const HardArgs& a, int nbins) {
  return a.nz == 1 ? copies_for(1, nbins) : copies3d_f32(nbins, a.H);
}

}  // namespace

hipError_t launch_hard(const HardArgs& a, hipStream_t s) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  if (a.dtype == 0) {
    // 16 histogram copies: 8 measured slower (bank conflicts), 32 spend more
    // time summing the copies at the flush
    if (a.nz == 1) return launch2d<0, 16, 16, 16>(a, 256, s, di);
    // 8 bytes per lane when every 512-byte column chunk is full, else 4: the
    // cold tile takes partial chunks, and 256-byte chunks leave fewer of them
    // (512x256x256: 79 -> 35 us, 256x512x768: 152 -> 96 us; 512^3: 92 against
    // 107 us with 4 bytes per lane)
    if (a.nx % 512 != 0) return launch3d<0, 4, 32, 4, kBlock, 1>(a, 256, s, di);
    return launch3d<0, 8, 32, 4, kBlock, 1>(a, 256, s, di);
  }
  const int nbins = a.H;
  switch (copies_f32(a, nbins)) {
    case 32: return dispatch_f32<32>(a, nbins, s, di);
    case 16: return dispatch_f32<16>(a, nbins, s, di);
    case 8: return dispatch_f32<8>(a, nbins, s, di);
    case 4: return dispatch_f32<4>(a, nbins, s, di);
    case 2: return dispatch_f32<2>(a, nbins, s, di);
    default: return dispatch_f32<1>(a, nbins, s, di);
  }
}

}  // namespace ecc
