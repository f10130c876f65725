// Dispatch order of the sliced GEMM's tiles: the same code runs in the kernels (which tile a
// workgroup computes) and on the host (fo_tile_order, and the checks of the order).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fo {

// The tile grid of one launch: npos positions of tiles_m x tiles_n tiles; each position's tile
// rows cut into `groups` row groups of `group_rows` tile rows (the last may be shorter); the
// first `lead` and the last `trail` positions dispatched whole, the middle ones group-major.
struct TileGrid {
  int32_t npos, tiles_m, tiles_n;
  int32_t groups, group_rows;
  int32_t lead, trail;
};

// Tile rows in row group g of a position.
__host__ __device__ inline int group_rows_of(const TileGrid& t, int g) {
  const int r = t.tiles_m - g * t.group_rows;
  return r < t.group_rows ? r : t.group_rows;
}

// Tile order inside one block of T tiles (tiles_m rows x tiles_n columns). Workgroup b runs on
// XCD b % 8 (round-robin dispatch). When T is a multiple of 8, XCD x is given the x-th
// contiguous run of tile ids, and ids walk the tile grid in groups of up to 8 tile rows, column
// by column inside a group: the ~32 tiles an XCD runs at once then form an 8 x 4 block that
// shares its A row blocks and W column blocks in that XCD's L2.
__host__ __device__ inline void tile_coords(int u, int T, int tiles_m, int tiles_n, int& tm,
                                            int& tn) {
  const int id = (T % 8) ? u : (u % 8) * (T / 8) + u / 8;
  const int gm = tiles_m < 8 ? tiles_m : 8;
  const int gsize = gm * tiles_n;
  const int g = id / gsize, r = id % gsize;
  const int rows = tiles_m - g * gm < gm ? tiles_m - g * gm : gm;
  tm = g * gm + r % rows;
  tn = r / rows;
}

// Where dispatch index u (0 <= u < npos * tiles_m * tiles_n) lands: its position, row group and
// tile coordinates.
__host__ __device__ inline void locate(const TileGrid& t, int u, int& pos, int& grp, int& tm,
                                       int& tn) {
  const int T = t.tiles_m * t.tiles_n;
  const int lead_end = t.lead * T;
  const int mid = t.npos - t.lead - t.trail;
  const int mid_end = lead_end + mid * T;
  if (u < lead_end || u >= mid_end) {
    pos = u / T;
    tile_coords(u - pos * T, T, t.tiles_m, t.tiles_n, tm, tn);
    grp = tm / t.group_rows;
    return;
  }
  const int v = u - lead_end;
  const int full = mid * t.tiles_n * t.group_rows;  // tiles of one full group over the middle
  int g = v / full;
  if (g > t.groups - 1) g = t.groups - 1;
  const int r = v - g * full;
  const int rows = group_rows_of(t, g);
  const int Tg = rows * t.tiles_n;
  const int k = r / Tg;
  int tmg;
  tile_coords(r - k * Tg, Tg, rows, t.tiles_n, tmg, tn);
  pos = t.lead + k;
  grp = g;
  tm = g * t.group_rows + tmg;
}

}  // namespace fo
