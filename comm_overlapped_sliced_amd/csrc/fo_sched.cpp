// Slice scheduler and tile choice of libflashovl (host side).
//
// Slice orders follow the FlashOverlap page (gist.science paper 2604.24013), technical summary
// section 2 "Methodology": Flash-AG computes the slice the rank already holds first and the ring
// deliveries after it; Flash-RS's rank-adaptive schedule leaves the chunk that stays on the rank
// for last. Where the page is silent (ring direction, order of the outgoing chunks) the reading
// is: receive from rank r-1, so slice (r - t) mod P is the t-th to arrive; send chunk r+1+i at
// step i, so all ranks target distinct peers at every step.
#include <algorithm>

#include "fo_internal.h"

namespace fo {

int slice_order(int kind, int order, int P, int rank, int32_t* out) {
  if (P < 1 || P > FO_MAX_P || rank < 0 || rank >= P || !out) return 1;
  if (order == FO_ORDER_NATURAL) {
    for (int i = 0; i < P; ++i) out[i] = i;
    return 0;
  }
  if (order != FO_ORDER_FLASH) return 1;
  if (kind == 0) {
    for (int t = 0; t < P; ++t) out[t] = ((rank - t) % P + P) % P;
    return 0;
  }
  if (kind == 1) {
    for (int i = 0; i + 1 < P; ++i) out[i] = (rank + 1 + i) % P;
    out[P - 1] = rank;
    return 0;
  }
  return 1;
}

// AUTO tile choice. 256x256 tiles need the fewest operand bytes per MFMA and win when the grid
// covers the CUs several times over. When it is at most a few rounds and the last round is only
// partly filled, 128x256 tiles (half the rounds' granularity) finish sooner. Slices shorter than
// 256 rows use 128-row tiles, and very small problems fall back to 64x64. Rows of a tile never
// cross a slice.
int choose_tile(int P, int64_t m, int64_t N, int n_cu) {
  auto tiles = [&](int bm, int bn) {
    return (double)P * (double)((m + bm - 1) / bm) * (double)((N + bn - 1) / bn);
  };
  if (m <= 64 || N <= 64) return FO_TILE_64x64;
  if (m <= 128) return N >= 256 ? FO_TILE_128x256 : FO_TILE_128x128;
  if (N < 256) return FO_TILE_256x128;
  const double r256 = tiles(256, 256) / n_cu;
  if (r256 >= 3.0) return FO_TILE_256x256;
  const double partial = (double)(int64_t)(r256 + 0.999999) - r256;
  if (partial > 0.1) return FO_TILE_128x256;
  return FO_TILE_256x256;
}

}  // namespace fo
