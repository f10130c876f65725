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

TileShape tile_shape(int tile);

// Estimated relative cost of one call: rounds of workgroups over the CUs times the work of one
// tile, divided by how efficiently that tile shape feeds the MFMAs (larger wave tiles reuse each
// LDS fragment more often). Rows of a tile never cross a slice.
int choose_tile(int P, int64_t m, int64_t N, int n_cu) {
  struct Cand {
    int tile;
    double eff;
  };
  static const Cand cands[] = {
      {FO_TILE_256x256, 1.00}, {FO_TILE_256x128, 0.85}, {FO_TILE_128x256, 0.85},
      {FO_TILE_128x128, 0.60}, {FO_TILE_64x64, 0.20}};
  int best = FO_TILE_64x64;
  double best_cost = 1e300;
  for (const Cand& c : cands) {
    const TileShape ts = tile_shape(c.tile);
    const int64_t tm = (m + ts.bm - 1) / ts.bm, tn = (N + ts.bn - 1) / ts.bn;
    const int64_t tiles = (int64_t)P * tm * tn;
    const int64_t rounds = (tiles + n_cu - 1) / n_cu;
    const double cost = (double)rounds * ts.bm * ts.bn / c.eff;
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = c.tile;
    }
  }
  return best;
}

}  // namespace fo
