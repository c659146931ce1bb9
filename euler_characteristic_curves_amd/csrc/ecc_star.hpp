// Signed count of the cells whose value a voxel carries, for the gradient of
// the soft curve with respect to the grid (host and device).
//
// A cell's value is the max of its corners (page "Scalable GPU-Accelerated
// Euler Characteristic Curves", "Method / Key designs"), so the derivative of
// the value goes to one corner: the one holding the max, the first in index
// order (x fastest) among equal maxima.  The cells that send their derivative
// to voxel p are the cells around p in which every other corner q is below p
// (q before p in index order) or at most p (q after p).  Their signed count
//     c(p) = sum of (-1)^dim(c) over those cells
// is computed from one bit per neighbour of the 3x3(x3) block around p:
//     bit 9 (dz+1) + 3 (dy+1) + (dx+1) = neighbour p + (dz,dy,dx) exists and
//                                        lets p win (2D: dz = 0 only).
// A cell around p is a product of one interval per axis, [-1,0], [0] or
// [0,1]; it sends to p iff all its corners' bits are set.  Three separable
// AND steps (x, then y, then z) turn the neighbour bits into one bit per cell,
// cell bit 9 iz + 3 iy + ix with i = 0, 1, 2 for [-1,0], [0], [0,1]; the
// sign is + for an even number of non-[0] intervals.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ecc {

// cells whose number of non-[0] intervals is even (3 axes / 2 axes)
__host__ __device__ constexpr uint32_t even_cells(int axes) {
  uint32_t m = 0;
  const int n = axes == 3 ? 27 : 9;
  for (int b = 0; b < n; ++b) {
    const int ix = b % 3, iy = (b / 3) % 3, iz = b / 9;
    const int odd = (ix != 1) + (iy != 1) + (axes == 3 && iz != 1);
    if ((odd & 1) == 0) m |= 1u << b;
  }
  return m;
}

// One AND step along an axis whose index has weight S in the bit layout:
// from the bits of positions -1, 0, +1 (at S * {0, 1, 2} above each group's
// base, G = the group bases) to the bits of intervals [-1,0], [0], [0,1].
template <int S>
__host__ __device__ inline uint32_t and_step(uint32_t w, uint32_t G) {
  const uint32_t c = (w >> S) & G;
  const uint32_t l = w & c;
  const uint32_t r = c & (w >> (2 * S));
  return l | (c << S) | (r << (2 * S));
}

// c(p) from the neighbour bits (27 for 3D, 9 for 2D).
template <bool D3>
__host__ __device__ inline int star_count(uint32_t w) {
  if constexpr (D3) {
    w = and_step<1>(w, 0x1249249u);  // x: group bases dx = -1, every third bit
    w = and_step<3>(w, 0x1C0E07u);   // y: dy = -1 rows of each plane
    w = and_step<9>(w, 0x1FFu);      // z: the dz = -1 plane
    constexpr uint32_t E = even_cells(3);
    return __builtin_popcount(w & E) - __builtin_popcount(w & ~E & 0x7FFFFFFu);
  } else {
    w = and_step<1>(w, 0x49u);
    w = and_step<3>(w, 0x7u);
    constexpr uint32_t E = even_cells(2);
    return __builtin_popcount(w & E) - __builtin_popcount(w & ~E & 0x1FFu);
  }
}

}  // namespace ecc
