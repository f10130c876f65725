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

// AUTO tile choice. Every tile of a launch runs its whole K loop, so a launch takes about
// ceil(tiles / CUs) rounds of one tile's time, and a 256x256 round costs what two 128x256 rounds
// cost (128x256 tiles move 50% more operand bytes per flop and run ~3.5% slower per flop). The
// rules, each checked by timing the sliced calls on MI355X:
//   - slices of at most 128 rows: 128-row tiles (a 256-row tile would be half empty);
//   - fp32 output with K <= 4096: 128x256, whose shorter write-back of 128 KB per tile hides behind
//     other tiles' mainloops (Flash-RS, Llama-70B down projection: 523 vs 614 us);
//   - a weight above 128 MB: 256x256, the least operand traffic per flop once the operands
//     outgrow the last-level cache (Llama-405B gate+up: 3.3 vs 3.8 ms);
//   - otherwise the fewer rounds, counted as above, with ties to 256x256.
// Rows of a tile never cross a slice.
int choose_tile(int P, int64_t m, int64_t K, int64_t N, bool out_f32, int n_cu) {
  auto rounds = [&](int bm, int bn) {
    const double t = (double)P * (double)((m + bm - 1) / bm) * (double)((N + bn - 1) / bn);
    return (double)(int64_t)((t + n_cu - 1) / n_cu);
  };
  if (m <= 64 || N <= 64) return FO_TILE_64x64;
  if (m <= 128) return N >= 256 ? FO_TILE_128x256 : FO_TILE_128x128;
  if (N < 256) return FO_TILE_256x128;
  if (out_f32 && K <= 4096) return FO_TILE_128x256;
  if ((double)K * (double)N * 2.0 > 128.0 * 1024 * 1024) return FO_TILE_256x256;
  const double c256 = rounds(256, 256), c128 = rounds(128, 256) * 0.5 / 0.965;
  return c128 < c256 ? FO_TILE_128x256 : FO_TILE_256x256;
}

}  // namespace fo
