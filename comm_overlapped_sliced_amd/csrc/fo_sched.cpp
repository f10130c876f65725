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

// AUTO tile choice. 256x256 tiles move the fewest operand bytes per flop and keep the LDS
// below its bandwidth (128x256 tiles spend ~1.5x the LDS traffic per MFMA); the other shapes
// serve where a 256x256 tile would be half empty or where finer work pays. The rules, each
// checked by timing the sliced calls with arrivals on MI355X:
//   - slices of at most 128 rows: 128-row tiles (Llama-70B gate+up at 1K tokens: 176 vs 237 us);
//   - fewer than 256 columns: 256x128;
//   - a sliced call with fp32 output and K <= 4096 (Flash-RS at Llama-70B down-projection
//     shapes): 128x256. Such a call waits on its transfers more than on its GEMM, and the
//     smaller tiles finish the first outgoing row groups sooner (450 vs 493 us);
//   - fewer 256x256 tiles than CUs while the 128x256 tiles still fit in as many rounds over the
//     CUs: 128x256, which fills the CUs the larger tiles leave idle (the monolithic GEMM of the
//     Llama-70B gate+up at 1K tokens: 112 tiles of 256x256 on 256 CUs took 142-147 us, the
//     same product in 224 tiles of 128x256 111 us);
//   - otherwise 256x256 (Llama-70B gate+up, 2K-16K tokens, and both Llama-405B calls).
// Rows of a tile never cross a slice.
int choose_tile(int P, int64_t m, int64_t K, int64_t N, bool out_f32, int n_cu) {
  if (m <= 64 || N <= 64) return FO_TILE_64x64;
  if (m <= 128) return N >= 256 ? FO_TILE_128x256 : FO_TILE_128x128;
  if (N < 256) return FO_TILE_256x128;
  if (P > 1 && out_f32 && K <= 4096) return FO_TILE_128x256;
  if (n_cu > 0) {
    const int64_t tn = (N + 255) / 256;
    const int64_t t256 = (int64_t)P * ((m + 255) / 256) * tn;
    const int64_t t128 = (int64_t)P * ((m + 127) / 128) * tn;
    if (t256 < n_cu && (t128 + n_cu - 1) / n_cu <= (t256 + n_cu - 1) / n_cu)
      return FO_TILE_128x256;
  }
  return FO_TILE_256x256;
}

}  // namespace fo
