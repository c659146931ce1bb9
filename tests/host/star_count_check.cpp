// c(p) from neighbour bits (ecc_star.hpp) against a count written out cell by
// cell, over every neighbour mask: all 2^8 masks in 2D and all 2^26 in 3D
// (the centre bit is always set).  The cells around p are the products of one
// interval per axis out of [-1,0], [0] and [0,1]; a cell sends its derivative
// to p when each of its corners other than p has its bit set, and it adds
// (-1)^dim, dim = the number of axes whose interval is not [0].
// Usage: star_count_check [stride]  (3D masks tested: every stride-th, default 1)

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "ecc_star.hpp"

namespace {

struct Cell {
  uint32_t mask;  // bits of every corner, the centre included
  int sign;
};

// corners of a cell: per axis, interval 0 = {-1, 0}, 1 = {0}, 2 = {0, 1}
int cells_of(int axes, Cell* out) {
  const int ncell = axes == 3 ? 27 : 9;
  for (int c = 0; c < ncell; ++c) {
    int iv[3] = {c % 3, (c / 3) % 3, axes == 3 ? c / 9 : 1};
    uint32_t mask = 0;
    int dim = 0;
    for (int a = 0; a < axes; ++a) dim += iv[a] != 1;
    for (int dz = -1; dz <= 1; ++dz)
      for (int dy = -1; dy <= 1; ++dy)
        for (int dx = -1; dx <= 1; ++dx) {
          const int d[3] = {dx, dy, dz};
          bool in = true;
          for (int a = 0; a < 3; ++a) {
            const int lo = iv[a] == 2 ? 0 : (iv[a] == 0 ? -1 : 0);
            const int hi = iv[a] == 0 ? 0 : (iv[a] == 2 ? 1 : 0);
            if (a >= axes) in = in && d[a] == 0;
            else in = in && d[a] >= lo && d[a] <= hi;
          }
          if (!in) continue;
          const int bit = (axes == 3 ? 9 * (dz + 1) : 0) + 3 * (dy + 1) + (dx + 1);
          mask |= 1u << bit;
        }
    out[c] = Cell{mask, (dim & 1) ? -1 : 1};
  }
  return ncell;
}

int by_hand(uint32_t w, const Cell* cells, int n) {
  int c = 0;
  for (int i = 0; i < n; ++i)
    if ((w & cells[i].mask) == cells[i].mask) c += cells[i].sign;
  return c;
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t stride = argc > 1 ? strtoull(argv[1], nullptr, 10) : 1;
  Cell c2[9], c3[27];
  cells_of(2, c2);
  cells_of(3, c3);
  long bad = 0, tested = 0;
  int lo = 99, hi = -99;
  // 2D: centre bit 4; the other 8 bits take every value
  for (uint32_t m = 0; m < 256; ++m) {
    const uint32_t w = (m & 0xF) | (1u << 4) | ((m >> 4) << 5);
    const int want = by_hand(w, c2, 9);
    if (ecc::star_count<false>(w) != want) {
      if (bad++ < 5) fprintf(stderr, "2D mask %03x: got %d want %d\n", w, ecc::star_count<false>(w), want);
    }
    ++tested;
  }
  // 3D: centre bit 13
  for (uint64_t m = 0; m < (1ull << 26); m += stride) {
    const uint32_t w = (uint32_t)(m & 0x1FFF) | (1u << 13) | ((uint32_t)(m >> 13) << 14);
    const int want = by_hand(w, c3, 27);
    lo = want < lo ? want : lo;
    hi = want > hi ? want : hi;
    if (ecc::star_count<true>(w) != want) {
      if (bad++ < 5) fprintf(stderr, "3D mask %07x: got %d want %d\n", w, ecc::star_count<true>(w), want);
    }
    ++tested;
  }
  printf("star_count: %ld masks, %ld mismatches, 3D c(p) in [%d, %d]\n", tested, bad, lo, hi);
  return bad == 0 ? 0 : 1;
}
