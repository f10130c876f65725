// Internal interfaces of libflashovl: the launch plan the kernels consume, the tile catalogue
// and the host-side scheduler. Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flashovl.h"

namespace fo {

// One launch of the sliced GEMM. A "position" is one step of the slice schedule: the kernel's
// workgroups are laid out position-major, so lower positions are dispatched first.
struct Plan {
  const void* a_pos[FO_MAX_P];  // A rows of position p: [m, K], row stride K
  void* c_pos[FO_MAX_P];        // output rows of position p: [m, N], row stride N
  const float* recv[FO_MAX_P];  // partials added in the accumulate epilogue, in arrival order
  uint32_t* rel[FO_MAX_P];      // release flag raised when position p is complete (or null)
  int32_t gate[FO_MAX_P];       // arrival flag the mainloop of position p waits on (-1: none)
  int32_t recv_flag[FO_MAX_P];  // arrival flag of recv[i] (-1: resident, no wait)
  const void* b;                // W [K, N], row stride N
  const uint32_t* arr;          // arrival flags: flag of slice s at arr[s * kFlagStride]
  uint32_t* done;               // per-position completed-tile counters (zero between calls)
  uint32_t* err;                // set to nonzero when a wait runs past spin_limit
  uint64_t spin_limit;          // bound of each wait, in wall-clock ticks
  int64_t m, K, N;              // slice rows, reduction length, output columns
  int32_t npos;                 // positions in this launch
  int32_t n_recv;               // partials added at accum_pos
  int32_t accum_pos;            // position whose epilogue adds recv[] (-1: none)
  int32_t out_f32;              // 1: fp32 output, 0: bf16 (round to nearest even)
  int32_t tiles_m, tiles_n;     // tiles per position
  uint32_t epoch;               // value the flags carry for this call
};

// Each arrival flag is the first word of its own 64 KiB block. The block is what the copy engine
// writes to raise the flag: the HIP runtime runs device-to-device copies smaller than this as
// copy kernels (and its stream write/wait operations as kernels too), and an arrival must never
// need a compute unit, all of which the waiting GEMM may hold.
constexpr int kFlagBytes = 65536;
constexpr int kFlagStride = kFlagBytes / 4;  // in 32-bit words

struct TileShape {
  int bm, bn;
};

// Tile catalogue of the bf16 kernel (indexed by fo_tile, AUTO excluded).
TileShape tile_shape(int tile);
// AUTO selection for P slices of m rows; returns a fo_tile value.
int choose_tile(int P, int64_t m, int64_t N, int n_cu);

// Launches the sliced GEMM for `plan` (bf16 MFMA kernel with the given tile, or the fp32
// kernel when in_dt is FO_DT_F32). max_grid > 0 caps the number of workgroups: they then walk
// the tiles persistently, and the CUs beyond the cap stay free for other kernels.
hipError_t launch_gemm(const Plan& plan, int in_dt, int tile, int max_grid, hipStream_t stream);

// Fills the kFlagBytes block at `block` with `value` (one workgroup; stream-ordered).
hipError_t launch_stamp(uint32_t* block, uint32_t value, hipStream_t stream);

// Slice schedule: kind 0 = AG, 1 = RS; order = fo_order. Writes P ids.
int slice_order(int kind, int order, int P, int rank, int32_t* out);

}  // namespace fo
