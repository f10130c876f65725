// Internal interfaces of libflashovl: the launch plan the kernels consume, the tile catalogue,
// the host-side scheduler and the DMA transfer layer. Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "flashovl.h"
#include "fo_tiles.h"

namespace fo {

// Largest number of row groups a slice is cut into for its transfer and gating.
constexpr int kMaxGroups = FO_MAX_GROUPS;

// One launch of the sliced GEMM. A "position" is one step of the slice schedule; each position's
// rows are cut into `groups` row groups of `group_rows` tile rows (the last may be shorter), and
// a group is the unit of transfer, of gating and of release. Workgroups are laid out in dispatch
// order: the first `lead` positions whole, then the middle positions group-major (group 0 of
// every middle position in position order, then group 1, ...), then the last `trail` positions
// whole. With one group this is plain position order.
//
// Arrival and release flags are the 64-bit values of HSA signals, reached through tables of
// value addresses indexed [slice or position][group] (kMaxGroups entries per row). A copy engine
// decrements the value of a group's completion signal from 1 to 0 when the group has landed (a
// negative value reports a failed copy); the kernel stores 0 into a (position, group) release
// signal when that group of the position is complete, and a copy engine waiting on it then
// starts the matching transfer.
struct Plan {
  const void* a_pos[FO_MAX_P];       // A rows of position p: [m, K], row stride K
  void* c_pos[FO_MAX_P];             // output rows of position p: [m, N], row stride N
  const float* recv[FO_MAX_P];       // partials added in the accumulate epilogue, in arrival order
  int32_t gate_slice[FO_MAX_P];      // slice whose arrival gates position p's mainloop (-1: none)
  int32_t recv_slice[FO_MAX_P];      // slice id of recv[i], whose arrival is awaited (-1: resident)
  const int64_t* const* comp_tab;    // completion-signal values [slice][group]
  int64_t* const* rel_tab;           // release-signal values [position][group] (null: no release)
  const void* b;                     // W [K, N], row stride N
  uint32_t* done;                    // completed-tile counters [position][group] (zero between calls)
  uint32_t* err;                     // wait record, two words: [0] what failed (1: a wait ran past
                                     // spin_limit, 2: a copy reported failure), [1] the number
                                     // of the last call that failed
  uint32_t* lead;                    // [slice][group]: the last call whose poller is elected
  uint32_t* ready;                   // [slice][group]: the last call whose group has landed
  uint32_t gen;                      // this call's number (> 0, grows by one per call)
  int32_t act;                       // 1: SwiGLU epilogue (Flash-AG of the MLP block's gate+up)
  int64_t* start;                    // the call's start signal value, stored 0 at kernel start
                                     // (null: no copies wait for this kernel)
  uint64_t spin_limit;               // bound of each wait, in wall-clock ticks
  int64_t m, K, N;                   // slice rows, reduction length, output columns
  int32_t n_recv;                    // partials added at accum_pos
  int32_t accum_pos;                 // position whose epilogue adds recv[] (-1: none)
  int32_t out_f32;                   // 1: fp32 output, 0: bf16 (round to nearest even)
  TileGrid grid;                      // tiles per position, row groups, dispatch layout
  // K chunks of every A slice (1: row-major [m, K]; c > 1: c blocks [m, K/c] one after another).
  // A gated tile waits for arrival unit grp * chunks + j before it reads block j. chunk_magic =
  // ceil(2^32 / (K / c / 32)) gives a K step's block as umulhi(step, chunk_magic); 0 when c = 1.
  int32_t chunks;
  uint32_t chunk_magic;
  // Flash-RS tail (tail_units > 0): the accum_pos tiles store their plain fp32 sums, and
  // tail_units workgroups appended to the grid (tail_per_group per row group of tail_bm-row
  // tiles) add the partials onto them once the group's tiles are stored (own_done[group] = gen)
  // and its partials have landed, in the same order as the fused epilogue.
  int32_t tail_units, tail_per_group, tail_bm;
  uint32_t* own_done;
  // 1: acquire (invalidate the caches) after each arrival wait, because a transfer may share a
  // cache line with data read before it landed; 0: every transfer is cache-line aligned.
  int32_t acq;
};

// A plan with nothing to wait for: no gates, no awaited partials, no tables, no release.
inline Plan empty_plan() {
  Plan p{};
  for (int i = 0; i < FO_MAX_P; ++i) {
    p.gate_slice[i] = -1;
    p.recv_slice[i] = -1;
  }
  p.accum_pos = -1;
  p.start = nullptr;
  p.act = 0;
  p.chunks = 1;
  p.chunk_magic = 0;
  p.tail_units = 0;
  p.tail_per_group = 0;
  p.tail_bm = 0;
  p.own_done = nullptr;
  p.acq = 1;
  return p;
}

struct TileShape {
  int bm, bn;
};

// Tile catalogue of the bf16 kernel (indexed by fo_tile, AUTO excluded).
TileShape tile_shape(int tile);
// AUTO selection for P slices of m rows, reduction length K, N columns; returns a fo_tile value.
int choose_tile(int P, int64_t m, int64_t K, int64_t N, bool out_f32, int n_cu);

// Launches the sliced GEMM for `plan` (bf16 MFMA kernel with the given tile, or the fp32
// kernel when in_dt is FO_DT_F32). A plan whose waits or releases point at no signal table, or
// whose grid and row groups do not fit together, is refused (hipErrorInvalidValue) before
// anything is launched.
// e0 / e1 (optional): events given the kernel's own start and end times
hipError_t launch_gemm(const Plan& plan, int in_dt, int tile, hipStream_t stream,
                       hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

// Zeroes `words` 32-bit words at p from a small kernel on `stream` (no hipMemsetAsync, so the
// work can be captured in a HIP graph).
hipError_t launch_zero(uint32_t* p, int words, hipStream_t stream);

// Stores 0 into the signal value `v` from a one-thread kernel (stream-ordered), after a
// system-scope release: every copy that depends on the signal starts after the work enqueued
// before it on `stream`.
hipError_t launch_release(int64_t* v, hipStream_t stream);

// One-workgroup kernel that waits (bounded by spin_limit ticks) until the completion signals of
// groups 0..groups-1 of each listed slice have dropped to zero (comp_tab as in Plan), recording a
// timeout or a failed copy of call `gen` in the wait record err like the GEMM's waits.
hipError_t launch_wait(const int64_t* const* comp_tab, const int32_t* slices, int n, int groups,
                       uint64_t spin_limit, uint32_t* err, uint32_t gen, hipStream_t stream);

// The received partials added onto `out` after the GEMM (Flash-RS in the data-slicing order,
// where the own chunk is not the last one computed): out[i] += recv[0][i] + recv[1][i] + ... in
// that order, for i < count, once every row group of every awaited slice has landed.
struct ReduceArgs {
  float* out;
  const float* recv[FO_MAX_P];   // in arrival order
  int32_t recv_slice[FO_MAX_P];  // slice id whose arrival is awaited (-1: resident)
  int32_t n_recv;
  const int64_t* const* comp_tab;  // completion-signal values [slice][group] (null: no waits)
  int32_t groups;
  int32_t vec4;                    // every pointer 16-byte aligned and count % 4 == 0
  int64_t count;
  uint64_t spin_limit;
  uint32_t* err;                   // the wait record (two words, as in Plan)
  uint32_t gen;                    // the call's number
  int32_t max_blocks;              // persistent grid size
  uint32_t* go;                    // device word (uncached) block 0 sets to go_value once every
  uint32_t go_value;               // partial has landed; the other blocks wait on it
};
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream);

// silu(g) * u = g * u / (1 + e^-g) in fp32: the SwiGLU of the MLP block (fo_swiglu and the
// GEMM's SwiGLU epilogue compute it the same way). e^-g = 2^(-g log2 e) by the hardware exp2 and
// the quotient by the hardware reciprocal (each about 1 ulp of fp32, far below the bf16 rounding
// that follows) instead of an IEEE division, whose fix-up sequence costs the epilogue several
// times more VALU work. Large |g|: 2^(+big) = inf gives a reciprocal of 0 and h = 0; 2^(-big) =
// 0 gives h = g * u.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
  return g * u * __builtin_amdgcn_rcpf(1.0f + e);
}

// h[rows, inter] = silu(y[:, :inter]) * y[:, inter:] in bf16 (fp32 arithmetic, one rounding to
// nearest even); y is [rows, 2*inter] bf16. inter % 8 == 0, both 16-byte aligned.
hipError_t launch_swiglu(const void* y, void* h, int64_t rows, int64_t inter, hipStream_t stream);

// Query-split attention of one rank after a Flash All-to-All (fo_attn): slice s holds the query,
// key and value rows of sequence positions s*m .. s*m+m-1 for this rank's heads, one row per
// token laid out as [hq query heads | hkv key heads | hkv value heads] x 128 bf16. Workgroups
// take (slice, 128-query tile, head) in `order` (position -> slice id) and walk the key slices
// in the same order. A slice whose `gated` entry is set arrives in `groups` row groups of
// `group_rows` rows (a multiple of 128; the last may be shorter): a query tile waits for the
// group holding its rows and a key tile for the group holding its keys.
struct AttnPlan {
  const void* slice[FO_MAX_P];       // by slice id: its rows [m, (hq + 2 hkv) * 128]
  void* out;                         // [P*m, hq * 128] bf16, query position-major
  int32_t order[FO_MAX_P];           // arrival order: position -> slice id
  int32_t gated[FO_MAX_P];           // by slice id: 1 = wait for its arrival
  const int64_t* const* comp_tab;    // completion-signal values [slice][group]
  uint32_t* lead;                    // elected-poller words, as in Plan
  uint32_t* ready;
  uint32_t gen;
  uint32_t* err;
  uint64_t spin_limit;
  int64_t* start;                    // the call's start signal (null: no copies)
  int64_t m;                         // tokens per slice
  int64_t group_rows;                // rows per arrival group (multiple of 128)
  int32_t groups;                    // arrival groups per slice (1..kMaxGroups)
  int32_t P, hq, hkv, causal;
  // > 0: the workgroups are dispatched as two halves of pair_half, the first taking the query
  // tiles with the most keys first and the second the fewest first, so that the pair of
  // workgroups that shares a CU has a balanced amount of work (causal, one workgroup per slot)
  int32_t pair_half;
  float scale_log2;                  // log2(e) / sqrt(128)
  int32_t acq;                       // 1: acquire after each arrival wait (see Plan::acq)
  // Dispatch order of the query slices (position -> slice id) when pair_half is 0; the key walk
  // follows `order`. With the return exchange the own slice is dispatched last.
  int32_t dispatch[FO_MAX_P];
  // The return exchange (the second All-to-All of Ulysses parallelism): when every work item of
  // (slice s, row group g) with send[s] set has stored its output rows, the last one to finish
  // stores 0 into the release signal rel_tab[s][g]; the copy engine that sends those rows to
  // rank s waits for it. rel_tab null: no return exchange.
  int64_t* const* rel_tab;
  uint32_t* done;                    // finished work items [slice][group] (zero between calls)
  int32_t send[FO_MAX_P];            // by slice id: 1 = its output rows are sent back
  // the outgoing groups: rows of a slice released and sent together (a multiple of the 128-row
  // query tile, independent of the arriving groups above)
  int64_t out_group_rows;
  int32_t out_groups;
  // Work table (null: one item per (slice, query tile, head) in the order above). Entry u is the
  // workgroup's item: {slice, query tile, head, w}; w < 0 covers every key of the item, else the
  // item's key walk is cut in two at ceil(tiles / 2) and entry w covers part w & 1 of pair w >> 1.
  // The two parts of a pair each store their unnormalized output, running max and sum in
  // part_buf; the second to finish (pair_cnt counts them, zero between calls) combines them and
  // stores the item's output.
  // Workgroup b takes entries bins[b] .. bins[b + 1] - 1 of the table, one after the other
  // (n_bins workgroups, all resident at once: two per CU).
  const int4* table;
  const int32_t* bins;
  int32_t n_items, n_bins;
  float* part_buf;                   // [pair][part][kAttnPartFloats] (null: no pair)
  uint32_t* pair_cnt;                // [pair]
};
// floats of one part's partial output: 4 waves x (64 output values + running max + sum) x 64 lanes
constexpr int kAttnPartFloats = 4 * 66 * 64;
bool attn_plan_ok(const AttnPlan& p);
hipError_t launch_attn(const AttnPlan& p, hipStream_t stream, hipEvent_t e0 = nullptr,
                       hipEvent_t e1 = nullptr);

// Slice schedule: kind 0 = AG, 1 = RS; order = fo_order. Writes P ids.
int slice_order(int kind, int order, int P, int rank, int32_t* out);

// ------------------------------------------------------------------ DMA transfer layer -------
//
// Emulated point-to-point transfers run on the GPU's SDMA engines through the HSA runtime that
// HIP itself uses: each transfer is an asynchronous copy on one engine (one engine stands for
// one link), gated by dependency signals that the engine itself polls, so no part of a transfer
// or of its gating needs a compute unit (the GEMM may hold all of them).
namespace dma {

constexpr int kSlots = 4;  // calls in flight per device before the host waits for the oldest

// The signals of one call: the start signal's value, and the device tables of completion and
// release signal values ([slice or position][group], kMaxGroups per row) the kernels read.
struct Call {
  int slot;
  int64_t* start;
  const int64_t* const* comp_tab;
  int64_t* const* rel_tab;
  // a link is an engine pair whose two engines take the link's copies in turn (else one engine);
  // with split each copy is cut in two halves, one on each engine of the pair
  bool pairs = false;
  bool split = false;
};

// Per-device setup (called once, under the device lock, with the device current): finds the
// runtime and the device's agent, chooses the engines, creates the signal slots and runs one
// small copy on every engine (an engine's first copy sets up its queue, which takes
// milliseconds). `scratch` is device memory of at least 2 * 65536 bytes.
bool init(int dev, void* scratch, std::string* err);
int n_engines(int dev);

// Starts a call: takes the device's next slot (first waiting, on the host, until the call that
// used it last is complete: its event done and its copies landed), re-arms the start signal and
// the release and completion signals of P slices x `groups` groups to 1, and returns them.
bool begin(int dev, int P, int groups, Call* call, std::string* err);
// Copy `bytes` from src to dst on link `link` (engine link mod n_engines; with call.pairs the
// next engine in turn of pair link mod n_pairs, or with call.split both engines of the pair, a
// half each), starting once the call's start signal and, when rel_pos >= 0, the release signal
// of (rel_pos, group) are zero.
// The completion signal of (slice, group) is decremented when the copy has landed.
bool copy(int dev, const Call& call, int link, int slice, int group, int rel_pos, void* dst,
          const void* src, size_t bytes, std::string* err);
// Records, on `stream`, the point after which the call's kernels no longer read its signals
// (after the call's last kernel); *ev receives the recorded event.
bool end(int dev, const Call& call, hipStream_t stream, std::string* err, hipEvent_t* ev = nullptr);
// Waits (host, bounded) until every copy issued on the device has landed. On failure
// *timed_out tells a copy still in flight at the bound from one the engine reported as failed.
bool drain(int dev, uint32_t timeout_ms, std::string* err, bool* timed_out);

}  // namespace dma
}  // namespace fo
