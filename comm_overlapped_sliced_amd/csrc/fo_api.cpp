// C ABI of libflashovl: argument checks, per-device state, emulated arrivals and the launch.
//
// Flash-AG / Flash-RS as described on the FlashOverlap page (gist.science paper 2604.24013),
// technical summary section 2: collectives split into point-to-point transfers, slices computed
// in an order that hides them (local slice first for AG, own chunk last for RS), with per-slice
// synchronisation instead of step barriers (section 3). On one GPU a transfer is emulated by an
// SDMA copy from a "peer" buffer into the receive buffer (fo_dma.cpp); the GEMM kernel's tiles
// of a slice wait for that copy's completion signal. Every call enqueues, on the compute stream:
// a one-thread kernel that releases the call's copies, then the GEMM; the copies are issued to
// the DMA engines after that, gated on the release (and, for Flash-RS in lockstep, on the GEMM's
// step releases).
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <queue>
#include <string>
#include <vector>

#include "fo_internal.h"

namespace {

thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

fo_status invalid(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return FO_ERR_INVALID_ARG;
}

fo_status unsupported(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return FO_ERR_UNSUPPORTED;
}

#define FO_HIP(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      set_error("%s failed: %s", #call, hipGetErrorString(e_));                   \
      return FO_ERR_HIP;                                                          \
    }                                                                             \
  } while (0)

// a DMA-layer call that reports failure through a message
#define FO_DMA(call)                                                              \
  do {                                                                            \
    std::string e_;                                                               \
    if (!(call)) {                                                                \
      set_error("%s", e_.c_str());                                                \
      return FO_ERR_HIP;                                                          \
    }                                                                             \
  } while (0)

constexpr int kMaxDevices = 64;
constexpr uint32_t kDefaultTimeoutUs = 2000000u;
constexpr size_t kScratchBytes = 2 * 65536;

// Library-owned objects of one device, allocated once and kept for the life of the process.
struct DevState {
  std::mutex mu;
  bool ready = false;
  int dev = 0;
  int n_cu = 0;
  int wall_khz = 100000;     // wall-clock counter rate read by the kernels' bounded waits
  uint32_t* err = nullptr;   // wait record, two words: what failed (1 timeout, 2 failed copy)
                             // and the number of the last call that failed (uncached memory)
  uint32_t* go = nullptr;    // the tail reduce's start word (same uncached block)
  uint32_t* own_done = nullptr;  // Flash-RS tail: own-chunk row groups stored [group] (same block)
  uint32_t go_value = 0;
  uint32_t* done = nullptr;  // completed-tile counters [position][group]
  uint32_t* arr_lead = nullptr;   // arrival-poller election and landed words [slice][group]
  uint32_t* arr_ready = nullptr;  // (uncached)
  uint32_t gen = 0;          // number of the last call (the kernels' election round)
  void* scratch = nullptr;   // source and destination of the DMA engines' first copies
  hipEvent_t ev_last = nullptr;     // recorded after a call that has no copy slot
  hipEvent_t last_ev = nullptr;     // the event recorded after the device's last call
  hipStream_t last_stream = nullptr;
  bool have_last = false;
  // the attention's work tables, by shape (built once per shape, kept until the process ends),
  // and the partial outputs and counters of its split items (grown to the largest call)
  struct AttnTable {
    int32_t P, hq, causal;
    int64_t m;
    int4* table;
    int32_t* bins;
    int32_t n_items, n_bins, n_pairs;
  };
  std::vector<AttnTable> attn_tables;
  float* attn_part = nullptr;
  uint32_t* attn_cnt = nullptr;
  int64_t attn_pairs_cap = 0;
};

DevState g_dev[kMaxDevices];

fo_status ensure_ready(int dev, DevState& st) {
  if (st.ready) return FO_OK;
  st.dev = dev;
  FO_HIP(hipDeviceGetAttribute(&st.n_cu, hipDeviceAttributeMultiprocessorCount, dev));
  int khz = 0;
  FO_HIP(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev));
  if (khz > 0) st.wall_khz = khz;
  void* p = nullptr;
  FO_HIP(hipExtMallocWithFlags(&p, 4096, hipDeviceMallocUncached));
  st.err = (uint32_t*)p;
  st.go = (uint32_t*)((uint8_t*)p + 256);
  st.own_done = (uint32_t*)((uint8_t*)p + 512);
  FO_HIP(hipMemset(p, 0, 4096));
  const size_t words = (size_t)FO_MAX_P * fo::kMaxGroups * sizeof(uint32_t);
  FO_HIP(hipExtMallocWithFlags(&p, 2 * words, hipDeviceMallocUncached));
  st.arr_lead = (uint32_t*)p;
  st.arr_ready = (uint32_t*)((uint8_t*)p + words);
  FO_HIP(hipMemset(p, 0, 2 * words));
  const size_t counters = (size_t)FO_MAX_P * fo::kMaxGroups * sizeof(uint32_t);
  FO_HIP(hipMalloc(&p, counters));
  st.done = (uint32_t*)p;
  FO_HIP(hipMemset(st.done, 0, counters));
  FO_HIP(hipMalloc(&st.scratch, kScratchBytes));
  FO_HIP(hipMemset(st.scratch, 0, kScratchBytes));
  FO_HIP(hipEventCreateWithFlags(&st.ev_last, hipEventDisableTiming));
  FO_HIP(hipDeviceSynchronize());
  FO_DMA(fo::dma::init(dev, st.scratch, &e_));
  st.ready = true;
  return FO_OK;
}

// The state of the current device, initialized on first use, with its lock held by `lk`.
fo_status current_state(DevState** out, std::unique_lock<std::mutex>* lk) {
  int dev = 0;
  FO_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("device %d beyond the library's limit of %d", dev, kMaxDevices);
    return FO_ERR_UNSUPPORTED;
  }
  DevState& st = g_dev[dev];
  *lk = std::unique_lock<std::mutex>(st.mu);
  const fo_status s = ensure_ready(dev, st);
  if (s != FO_OK) return s;
  *out = &st;
  return FO_OK;
}

size_t dt_size(int dt) { return dt == FO_DT_BF16 ? 2 : 4; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range rng(const void* p, size_t bytes) { return {(uintptr_t)p, (uintptr_t)p + bytes}; }

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo < a.hi && b.lo < b.hi; }

fo_status check_opts(const fo_opts* o, fo_opts* out) {
  fo_opts_init(out);
  if (!o) return FO_OK;
  if (o->order != FO_ORDER_FLASH && o->order != FO_ORDER_NATURAL)
    return invalid("opts.order %d is not a fo_order", o->order);
  if (o->arrival < FO_ARR_DEFAULT || o->arrival > FO_ARR_LOCKSTEP)
    return invalid("opts.arrival %d is not a fo_arrival", o->arrival);
  if (o->tile < FO_TILE_AUTO || o->tile > FO_TILE_64x64)
    return invalid("opts.tile %d is not a fo_tile", o->tile);
  if (o->links < 0 || o->links > FO_MAX_P)
    return invalid("opts.links %d outside [0, %d]", o->links, FO_MAX_P);
  if (o->row_groups < 0 || o->row_groups > fo::kMaxGroups)
    return invalid("opts.row_groups %d outside [0, %d]", o->row_groups, fo::kMaxGroups);
  if (o->epilogue != FO_EPI_NONE && o->epilogue != FO_EPI_SWIGLU)
    return invalid("opts.epilogue %d is not a fo_epilogue", o->epilogue);
  if (o->k_chunks < 0 || o->k_chunks > fo::kMaxGroups)
    return invalid("opts.k_chunks %d outside [0, %d]", o->k_chunks, fo::kMaxGroups);
  if (o->engines_per_link < 0 || o->engines_per_link > 3)
    return invalid("opts.engines_per_link %d outside [0, 3]", o->engines_per_link);
  if (o->reserved != 0) return invalid("opts.reserved must be 0");
  *out = *o;
  if (out->spin_timeout_us == 0) out->spin_timeout_us = kDefaultTimeoutUs;
  return FO_OK;
}

fo_status check_common(int P, int rank, int64_t m, int64_t K, int64_t N, int in_dt) {
  if (P < 1 || P > FO_MAX_P) return invalid("P = %d outside [1, %d]", P, FO_MAX_P);
  if (rank < 0 || rank >= P) return invalid("rank = %d outside [0, P = %d)", rank, P);
  if (m < 0 || K < 0 || N < 0) return invalid("negative size (m %lld, K %lld, N %lld)",
                                              (long long)m, (long long)K, (long long)N);
  if (in_dt != FO_DT_BF16 && in_dt != FO_DT_F32) return invalid("in_dt %d is not a fo_dtype", in_dt);
  const int64_t lim = (int64_t)1 << 40;
  if (m > lim || K > lim || N > lim || (double)P * m * std::max<int64_t>(K, N) > 4.0e15)
    return invalid("sizes too large");
  if (in_dt == FO_DT_BF16 && (K % 8 || N % 8))
    return invalid("bf16 operands need K and N to be multiples of 8 (K %lld, N %lld)",
                   (long long)K, (long long)N);
  // the bf16 kernel addresses a tile's rows of A and of the output with 31-bit byte offsets
  if (in_dt == FO_DT_BF16 && (K > ((int64_t)1 << 21) || N > ((int64_t)1 << 20)))
    return invalid("bf16 operands need K <= 2^21 and N <= 2^20 (K %lld, N %lld)",
                   (long long)K, (long long)N);
  return FO_OK;
}

int resolve_tile(const fo_opts& o, int in_dt, int out_dt, int P, int64_t m, int64_t K, int64_t N,
                 int n_cu) {
  if (in_dt == FO_DT_F32) return 0;
  if (o.tile != FO_TILE_AUTO) return o.tile;
  return fo::choose_tile(P, m, K, N, out_dt == FO_DT_F32, n_cu);
}

fo_status tiles_for(int in_dt, int tile, int64_t m, int64_t N, int P, fo::Plan& p,
                    int* bm_out = nullptr) {
  int bm = 64, bn = 64;
  if (in_dt == FO_DT_BF16) {
    const fo::TileShape ts = fo::tile_shape(tile);
    bm = ts.bm;
    bn = ts.bn;
  }
  const int64_t tm = (m + bm - 1) / bm, tn = (N + bn - 1) / bn;
  if (tm * tn * P > 0x7fffffffLL) return invalid("too many tiles");
  p.grid.tiles_m = (int32_t)tm;
  p.grid.tiles_n = (int32_t)tn;
  if (bm_out) *bm_out = bm;
  return FO_OK;
}

// Row groups: `req` groups (0 = one per tile row), at most kMaxGroups and at most one per tile
// row, each a whole number of tile rows.
void set_groups(int req, fo::Plan& p) {
  int G = req == 0 ? p.grid.tiles_m : req;
  G = std::max(1, std::min({G, fo::kMaxGroups, (int)p.grid.tiles_m}));
  p.grid.group_rows = (p.grid.tiles_m + G - 1) / G;
  p.grid.groups = (p.grid.tiles_m + p.grid.group_rows - 1) / p.grid.group_rows;
}

// Dispatch layout of a call of `kind` (0 AG, 1 RS): Flash-AG puts the local slice first, whole,
// and computes the received slices group by group; Flash-RS computes the chunks for the other
// ranks group by group and its own chunk last, whole. NATURAL: every slice group by group in
// index order.
void set_layout(int kind, const fo_opts& o, fo::Plan& p) {
  set_groups(o.row_groups, p);
  // Flash-AG with K-chunk-major slices: groups x chunks arrival units per slice
  const int c = kind == 0 ? std::max(1, o.k_chunks) : 1;
  if (c > 1 && p.grid.groups * c > fo::kMaxGroups) set_groups(fo::kMaxGroups / c, p);
  p.grid.lead = (kind == 0 && o.order == FO_ORDER_FLASH) ? 1 : 0;
  p.grid.trail = (kind == 1 && o.order == FO_ORDER_FLASH) ? 1 : 0;
}

// Element rows [*r0, *r1) of row group g of a slice of m rows with tile height bm.
void group_span(const fo::Plan& p, int bm, int64_t m, int g, int64_t* r0, int64_t* r1) {
  *r0 = std::min<int64_t>(m, (int64_t)g * p.grid.group_rows * bm);
  *r1 = std::min<int64_t>(m, (int64_t)(g + 1) * p.grid.group_rows * bm);
}

uint64_t spin_ticks(const DevState& st, uint32_t us) { return (uint64_t)us * st.wall_khz / 1000u; }

// Links (DMA engines) one call's transfers are spread over: transfer t goes over link t mod L.
// Default: one link per peer.
int links_for(const fo_opts& o, int P) {
  const int L = o.links == 0 ? P - 1 : o.links;
  return std::max(1, std::min(L, P - 1));
}

// Arrival order of the slices a rank receives: for FLASH (and for RS always) rank-1, rank-2, ...
// (mod P), the order in which a ring from rank-1 delivers them; for the NATURAL AG order the
// slices are needed, and so sent, in index order.
int arrival_sequence(int kind, int order, int P, int rank, int* seq) {
  int n = 0;
  if (kind == 0 && order == FO_ORDER_NATURAL) {
    for (int s = 0; s < P; ++s)
      if (s != rank) seq[n++] = s;
  } else {
    for (int i = 1; i < P; ++i) seq[n++] = ((rank - i) % P + P) % P;
  }
  return n;
}

// The engines of one link (opts.engines_per_link): 1 one engine; 2 an engine pair taking the
// link's copies in turn; 3 the pair, every copy split in two halves, one on each engine.
void set_engines(const fo_opts& o, int dflt, fo::dma::Call* call) {
  const int e = o.engines_per_link ? o.engines_per_link : dflt;
  call->pairs = e >= 2;
  call->split = e == 3;
}

// Default engines per link: the pair with every transfer split across it. A released Flash-RS
// group then leaves at the pair's rate, not one engine's (70B call: one engine 416 us, pairs
// taking copies in turn 352 us, split 323 us), and the first row group of a Flash-AG slice lands
// sooner (row-major 70B call 456 -> 438 us).
constexpr int kEnginesAG = 3, kEnginesRS = 3, kEnginesAttn = 3;

// Every call on a device is ordered after the previous one (they share the device's signals,
// counters and words): a call on another stream first waits for the previous call's event; on
// the same stream the order is already given.
fo_status order_after_last(DevState* st, hipStream_t cs) {
  if (st->have_last && cs != st->last_stream) FO_HIP(hipStreamWaitEvent(cs, st->last_ev, 0));
  return FO_OK;
}

// Marks the end of a call on `cs`: the copy slot's event when the call has one (already
// recorded), else the device's own event.
fo_status mark_last(DevState* st, hipStream_t cs, hipEvent_t slot_ev) {
  if (slot_ev) {
    st->last_ev = slot_ev;
  } else {
    FO_HIP(hipEventRecord(st->ev_last, cs));
    st->last_ev = st->ev_last;
  }
  st->last_stream = cs;
  st->have_last = true;
  return FO_OK;
}

fo_status launch_with_events(const fo::Plan& p, int in_dt, int tile, hipStream_t cs,
                             const fo_opts& o) {
  FO_HIP(fo::launch_gemm(p, in_dt, tile, cs, (hipEvent_t)o.kernel_events[0],
                         (hipEvent_t)o.kernel_events[1]));
  return FO_OK;
}

// What a Flash-RS call takes from its device: the words its kernels count, wait and record in,
// the call's number, and the device's CU count and wait bound. fo_gemm_rs takes them from the
// library-allocated state, fo_gemm_rs_noalloc from the static scratch array.
struct Words {
  uint32_t* done = nullptr;
  uint32_t* own_done = nullptr;
  uint32_t* err = nullptr;
  uint32_t* lead = nullptr;
  uint32_t* ready = nullptr;
  uint32_t* go = nullptr;
  uint32_t gen = 0, go_value = 0;
  int n_cu = 0;
  uint64_t spin_limit = 0;
};

// Argument checks of fo_gemm_rs (and of fo_gemm_rs_noalloc, with no peer partials); *o
// receives the options with defaults filled in. Nothing is enqueued.
fo_status rs_check(const void* x_shard, const void* w, const float* send_buf, const float* out,
                   const float* const* peer_partial, const float* recv_buf, int P, int rank,
                   int64_t m, int64_t K, int64_t N, int in_dt, const fo_opts* opts, fo_opts* o) {
  fo_status s = check_opts(opts, o);
  if (s != FO_OK) return s;
  s = check_common(P, rank, m, K, N, in_dt);
  if (s != FO_OK) return s;
  if (o->epilogue != FO_EPI_NONE) return invalid("opts.epilogue applies to fo_ag_gemm only");
  if (o->k_chunks > 1) return invalid("opts.k_chunks applies to fo_ag_gemm only");
  const int arrival = o->arrival == FO_ARR_DEFAULT ? FO_ARR_LOCKSTEP : o->arrival;
  const bool arrivals = peer_partial != nullptr && arrival != FO_ARR_NONE && P > 1;
  const size_t es = dt_size(in_dt);
  const size_t align = in_dt == FO_DT_BF16 ? 16 : 4;
  if (!x_shard || !w || !out || (P > 1 && (!send_buf || !recv_buf))) return invalid("NULL buffer");
  if (!aligned(x_shard, align) || !aligned(w, align) || !aligned(out, 4) ||
      (send_buf && !aligned(send_buf, 4)) || (recv_buf && !aligned(recv_buf, 4)))
    return invalid("misaligned buffer (inputs need %zu-byte alignment)", align);
  const size_t chunk_b = (size_t)m * N * 4;
  const Range r_x = rng(x_shard, (size_t)P * m * K * es), r_w = rng(w, (size_t)K * N * es);
  const Range r_out = rng(out, chunk_b);
  const Range r_send = rng(send_buf, send_buf ? (size_t)P * chunk_b : 0);
  const Range r_recv = rng(recv_buf, recv_buf ? (size_t)P * chunk_b : 0);
  for (Range o1 : {r_out, r_send}) {
    if (overlap(o1, r_x) || overlap(o1, r_w) || overlap(o1, r_recv))
      return invalid("an output overlaps an input");
  }
  if (overlap(r_out, r_send)) return invalid("out overlaps send_buf");
  if (arrivals) {
    for (int q = 0; q < P; ++q) {
      if (q == rank) continue;
      if (!peer_partial[q]) return invalid("peer_partial[%d] is NULL", q);
      if (!aligned(peer_partial[q], 4)) return invalid("peer_partial[%d] misaligned", q);
      const Range rp = rng(peer_partial[q], chunk_b);
      if (overlap(rp, r_recv) || overlap(rp, r_out) || overlap(rp, r_send))
        return invalid("peer_partial[%d] overlaps recv_buf or an output", q);
    }
  }
  return FO_OK;
}

// The launch plan of a Flash-RS call (no transfer tables: the caller adds them). `arrivals`
// only decides the acquire after arrival waits. *bm, *tile and *own_pos receive the tile height,
// the tile shape and the position of the own chunk.
fo_status rs_plan(const void* x_shard, const void* w, float* send_buf, float* out, float* recv_buf,
                  int P, int rank, int64_t m, int64_t K, int64_t N, int in_dt, const fo_opts& o,
                  const Words& wd, bool arrivals, fo::Plan* pp, int* bm, int* tile,
                  int* own_pos) {
  fo::Plan& p = *pp;
  const size_t es = dt_size(in_dt), chunk_b = (size_t)m * N * 4;
  *tile = resolve_tile(o, in_dt, FO_DT_F32, P, m, K, N, wd.n_cu);
  const fo_status s = tiles_for(in_dt, *tile, m, N, P, p, bm);
  if (s != FO_OK) return s;
  set_layout(1, o, p);
  // NATURAL (data slicing): chunks in index order, the own chunk written plainly where it falls,
  // and the partials added after the GEMM by a separate kernel
  const bool natural = o.order == FO_ORDER_NATURAL;
  int32_t order[FO_MAX_P];
  fo::slice_order(1, o.order, P, rank, order);
  for (int pos = 0; pos < P; ++pos) {
    const int d = order[pos];
    p.a_pos[pos] = (const uint8_t*)x_shard + (size_t)d * m * K * es;
    p.c_pos[pos] = d == rank ? (void*)out : (void*)((uint8_t*)send_buf + (size_t)d * chunk_b);
    p.gate_slice[pos] = -1;
    if (d == rank) *own_pos = pos;
  }
  if (!natural) p.accum_pos = *own_pos;
  // partials arrive from rank-1, rank-2, ... (mod P) and are added in that order
  for (int i = 1; i < P; ++i) {
    const int q = ((rank - i) % P + P) % P;
    p.recv[i - 1] = (const float*)((const uint8_t*)recv_buf + (size_t)q * chunk_b);
    p.recv_slice[i - 1] = -1;
  }
  p.n_recv = P - 1;
  p.b = w;
  p.done = wd.done;
  p.lead = wd.lead;
  p.ready = wd.ready;
  p.gen = wd.gen;
  p.err = wd.err;
  p.spin_limit = wd.spin_limit;
  p.m = m;
  p.K = K;
  p.N = N;
  p.grid.npos = P;
  p.out_f32 = 1;
  // partials' transfers on cache-line (128-byte) boundaries: no acquire after the arrival waits
  p.acq = (!arrivals || (aligned(recv_buf, 128) && ((size_t)N * 4) % 128 == 0)) ? 0 : 1;
  // Flash-RS tail: the own chunk's tiles store their sums and workgroups appended to the grid add
  // the partials (same order, same bits), spread over the CUs the other chunks have freed. Needs
  // 16-byte aligned out and partials (else the own tiles add them in their epilogue).
  if (!natural && P > 1 && in_dt == FO_DT_BF16 && aligned(out, 16) &&
      (double)m * N * 4 < (double)(1u << 31)) {
    bool al = true;
    for (int i = 0; i < P - 1; ++i) al = al && aligned(p.recv[i], 16);
    if (al) {
      const int64_t rows_g = (int64_t)p.grid.group_rows * *bm;
      const int64_t pieces = rows_g * N / 4;  // 16-byte pieces of a full group
      p.tail_per_group = (int32_t)std::max<int64_t>(1, std::min<int64_t>(128, pieces / 2048));
      p.tail_units = p.grid.groups * p.tail_per_group;
      p.tail_bm = *bm;
      p.own_done = wd.own_done;
    }
  }
  return FO_OK;
}

// The separate pass of Flash-RS in the data-slicing order: out += the partials in arrival order
// once they have landed (comp_tab null: resident).
fo_status launch_rs_reduce(const fo::Plan& p, float* out, int64_t m, int64_t N, const Words& wd,
                           const int64_t* const* comp_tab, hipStream_t cs) {
  fo::ReduceArgs ra{};
  ra.out = out;
  ra.n_recv = p.n_recv;
  bool al = aligned(out, 16) && ((size_t)m * N) % 4 == 0;
  for (int i = 0; i < p.n_recv; ++i) {
    ra.recv[i] = p.recv[i];
    ra.recv_slice[i] = p.recv_slice[i];
    al = al && aligned(p.recv[i], 16);
  }
  ra.comp_tab = comp_tab;
  ra.groups = p.grid.groups;
  ra.vec4 = al ? 1 : 0;
  ra.count = m * N;
  ra.spin_limit = p.spin_limit;
  ra.err = wd.err;
  ra.gen = wd.gen;
  ra.max_blocks = 2 * wd.n_cu;
  ra.go = wd.go;
  ra.go_value = wd.go_value;
  FO_HIP(fo::launch_reduce(ra, cs));
  return FO_OK;
}

// ---- the scratch of fo_gemm_rs_noalloc -------------------------------------------------------
// A static device array instead of library-allocated memory, 32-bit words: [0, kNaOwn) the tile
// counters [position][row group], [kNaOwn, kNaErr) the own chunk's row-group words, [kNaErr,
// kNaErr + 2) the wait record, kNaGo the start word of the data-slicing reduce. Each device holds
// its own copy of the array until the process ends; host code reaches it only through the
// address hipGetSymbolAddress returns on that device (the array's name is a host-side stand-in).
constexpr int kNaCounters = 0;
constexpr int kNaOwn = FO_MAX_P * fo::kMaxGroups;
constexpr int kNaErr = kNaOwn + fo::kMaxGroups;
constexpr int kNaGo = kNaErr + 8;
static_assert((kNaGo + 1) * 4 <= FO_NOALLOC_SCRATCH_BYTES, "scratch layout");
__device__ __align__(256) static uint32_t scratch[FO_NOALLOC_SCRATCH_BYTES / 4];

struct NoAllocDev {
  std::mutex mu;
  uint32_t* ptr = nullptr;  // device address of `scratch` on this device
  int n_cu = 0;
  int wall_khz = 100000;
  uint32_t gen = 0;         // number of the device's last fo_gemm_rs_noalloc call
};
NoAllocDev g_na[kMaxDevices];

// The current device's scratch, set up on its first call (the symbol's address and two device
// attributes; nothing is allocated), with its lock held by `lk`.
fo_status noalloc_state(NoAllocDev** out, std::unique_lock<std::mutex>* lk) {
  int dev = 0;
  FO_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("device %d beyond the library's limit of %d", dev, kMaxDevices);
    return FO_ERR_UNSUPPORTED;
  }
  NoAllocDev& na = g_na[dev];
  *lk = std::unique_lock<std::mutex>(na.mu);
  if (na.ptr == nullptr) {
    void* ptr = nullptr;
    FO_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (ptr == nullptr || !aligned(ptr, 256)) {
      set_error("hipGetSymbolAddress returned no usable address for the scratch array");
      return FO_ERR_HIP;
    }
    int n_cu = 0, khz = 0;
    FO_HIP(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
    FO_HIP(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev));
    na.n_cu = n_cu;
    if (khz > 0) na.wall_khz = khz;
    na.ptr = (uint32_t*)ptr;
  }
  *out = &na;
  return FO_OK;
}

constexpr int kAttnItemCost = 4;        // per item, in key tiles
constexpr size_t kAttnTablesMax = 64;   // attention shapes whose tables a device keeps
constexpr double kAttnFirstShare = 0.6;

// The lists of one causal attention shape for n_cu CUs (host only): entries {slice, query tile,
// head, w} list by list, bins[b] .. bins[b + 1] - 1 the entries of workgroup b; returns the
// number of split pairs. False when the shape is too large for a table.
bool attn_lists(int32_t P, int64_t m, int32_t hq, int64_t n_cu, std::vector<int4>* entries,
                std::vector<int32_t>* bins_out, int32_t* n_pairs) {
  const int64_t qtiles = (m + 127) / 128;
  const int64_t base = (int64_t)P * qtiles * hq;
  const int64_t slots = 2 * n_cu;
  if (base < 1 || base > ((int64_t)1 << 22) || n_cu < 1) return false;
  const int64_t mt = (m + 63) / 64;
  struct Item {
    int64_t cost;
    int4 e;
  };
  std::vector<Item> items;
  int64_t sum = 0;
  for (int s = 0; s < P; ++s)
    for (int64_t qt = 0; qt < qtiles; ++qt) {
      const int64_t q1 = std::min<int64_t>(m, (qt + 1) * 128);
      sum += hq * (s * mt + (q1 + 63) / 64 + kAttnItemCost);
    }
  const int64_t share = (sum + slots - 1) / slots;
  int32_t pairs = 0;
  for (int s = 0; s < P; ++s)
    for (int64_t qt = 0; qt < qtiles; ++qt) {
      const int64_t q1 = std::min<int64_t>(m, (qt + 1) * 128);
      const int32_t w = (int32_t)(s * mt + (q1 + 63) / 64);
      for (int h = 0; h < hq; ++h) {
        if (w >= 2 && w + kAttnItemCost > share) {
          const int32_t cut = (w + 1) / 2;
          items.push_back({cut + kAttnItemCost, make_int4(s, (int)qt, h, 2 * pairs)});
          items.push_back({w - cut + kAttnItemCost, make_int4(s, (int)qt, h, 2 * pairs + 1)});
          ++pairs;
        } else {
          items.push_back({w + kAttnItemCost, make_int4(s, (int)qt, h, -1)});
        }
      }
    }
  // longest first (equal costs keep their table order: the schedule is a function of the shape)
  std::stable_sort(items.begin(), items.end(),
                   [](const Item& a, const Item& b) { return a.cost > b.cost; });
  const int64_t E = (int64_t)items.size();
  std::vector<std::vector<int4>> lists;
  if (E <= n_cu) {
    // one item per workgroup, each on a CU of its own
    for (const Item& it : items) lists.push_back({it.e});
  } else {
    using Load = std::pair<int64_t, int>;
    std::priority_queue<Load, std::vector<Load>, std::greater<Load>> heap;
    for (int c = 0; c < n_cu; ++c) heap.push({0, c});
    std::vector<std::vector<const Item*>> cu(n_cu);
    for (const Item& it : items) {
      Load l = heap.top();
      heap.pop();
      cu[l.second].push_back(&it);
      l.first += it.cost;
      heap.push(l);
    }
    lists.assign(slots, {});
    for (int c = 0; c < n_cu; ++c) {
      // the first workgroup's items: the subset whose cost is closest to its share (every
      // subset while there are few items, else longest first up to the share)
      const auto& v = cu[c];
      int64_t tot = 0;
      for (const Item* it : v) tot += it->cost;
      const double want = kAttnFirstShare * (double)tot;
      std::vector<char> first(v.size(), 0);
      if (v.size() <= 10) {
        double best = 1e300;
        uint32_t pick = 0;
        for (uint32_t mask = 0; mask < (1u << v.size()); ++mask) {
          int64_t a = 0;
          for (size_t i = 0; i < v.size(); ++i)
            if (mask >> i & 1) a += v[i]->cost;
          const double d = std::fabs((double)a - want);
          if (d < best) {
            best = d;
            pick = mask;
          }
        }
        for (size_t i = 0; i < v.size(); ++i) first[i] = (char)(pick >> i & 1);
      } else {
        int64_t a = 0;
        for (size_t i = 0; i < v.size(); ++i)
          if ((double)(a + v[i]->cost) <= want) {
            a += v[i]->cost;
            first[i] = 1;
          }
      }
      for (size_t i = 0; i < v.size(); ++i) lists[first[i] ? c : n_cu + c].push_back(v[i]->e);
    }
  }
  const int nb = (int)lists.size();
  entries->clear();
  bins_out->assign(nb + 1, 0);
  for (int b = 0; b < nb; ++b) {
    (*bins_out)[b] = (int32_t)entries->size();
    entries->insert(entries->end(), lists[b].begin(), lists[b].end());
  }
  (*bins_out)[nb] = (int32_t)entries->size();
  *n_pairs = pairs;
  return true;
}

}  // namespace

extern "C" {

void fo_opts_init(fo_opts* o) {
  if (!o) return;
  memset(o, 0, sizeof *o);
  o->order = FO_ORDER_FLASH;
  o->arrival = FO_ARR_DEFAULT;
  o->tile = FO_TILE_AUTO;
  o->spin_timeout_us = kDefaultTimeoutUs;
}

const char* fo_status_str(fo_status s) {
  switch (s) {
    case FO_OK: return "FO_OK";
    case FO_ERR_INVALID_ARG: return "FO_ERR_INVALID_ARG";
    case FO_ERR_UNSUPPORTED: return "FO_ERR_UNSUPPORTED";
    case FO_ERR_HIP: return "FO_ERR_HIP";
    case FO_ERR_TIMEOUT: return "FO_ERR_TIMEOUT";
  }
  return "FO_ERR_UNKNOWN";
}

const char* fo_last_error(void) { return g_last_error.c_str(); }

int32_t fo_version(void) { return FO_VERSION; }

fo_status fo_slice_order(int32_t kind, int32_t order, int32_t P, int32_t rank, int32_t* out) {
  if (kind != 0 && kind != 1) return invalid("kind %d is neither 0 (AG) nor 1 (RS)", kind);
  if (!out) return invalid("out is NULL");
  if (order != FO_ORDER_FLASH && order != FO_ORDER_NATURAL) return invalid("bad order %d", order);
  if (P < 1 || P > FO_MAX_P || rank < 0 || rank >= P) return invalid("bad P %d / rank %d", P, rank);
  fo::slice_order(kind, order, P, rank, out);
  return FO_OK;
}

fo_status fo_tile_info(int32_t P, int64_t m, int64_t K, int64_t N, int32_t in_dt, int32_t out_dt,
                       int32_t tile, int32_t* bm, int32_t* bn, int64_t* workgroups) {
  fo_status s = check_common(P, 0, m, K, N, in_dt);
  if (s != FO_OK) return s;
  if (out_dt != FO_DT_BF16 && out_dt != FO_DT_F32) return invalid("out_dt %d is not a fo_dtype", out_dt);
  if (tile < FO_TILE_AUTO || tile > FO_TILE_64x64) return invalid("bad tile %d", tile);
  // the CU count only matters for AUTO; use the device's when one is present
  int n_cu = 256, dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
      n_cu = c;
  }
  fo_opts o;
  fo_opts_init(&o);
  o.tile = tile;
  const int t = resolve_tile(o, in_dt, out_dt, P, m, K, N, n_cu);
  fo::Plan p = fo::empty_plan();
  s = tiles_for(in_dt, t, m, N, P, p);
  if (s != FO_OK) return s;
  int vbm = 64, vbn = 64;
  if (in_dt == FO_DT_BF16) {
    vbm = fo::tile_shape(t).bm;
    vbn = fo::tile_shape(t).bn;
  }
  if (bm) *bm = vbm;
  if (bn) *bn = vbn;
  if (workgroups) *workgroups = (int64_t)P * p.grid.tiles_m * p.grid.tiles_n;
  return FO_OK;
}

fo_status fo_tile_order(int32_t kind, int32_t P, int64_t m, int64_t K, int64_t N, int32_t in_dt,
                        int32_t out_dt, const fo_opts* opts, int32_t* out, int64_t capacity,
                        int64_t* count) {
  fo_opts o;
  fo_status s = check_opts(opts, &o);
  if (s != FO_OK) return s;
  if (kind != 0 && kind != 1) return invalid("kind %d is neither 0 (AG) nor 1 (RS)", kind);
  s = check_common(P, 0, m, K, N, in_dt);
  if (s != FO_OK) return s;
  if (out_dt != FO_DT_BF16 && out_dt != FO_DT_F32) return invalid("out_dt %d is not a fo_dtype", out_dt);
  if (capacity < 0 || (capacity > 0 && !out)) return invalid("bad output buffer");
  int n_cu = 256, dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
      n_cu = c;
  }
  if (m == 0 || N == 0) {
    if (count) *count = 0;
    return FO_OK;
  }
  const int tile = resolve_tile(o, in_dt, kind == 1 ? FO_DT_F32 : out_dt, P, m, K, N, n_cu);
  fo::Plan p = fo::empty_plan();
  s = tiles_for(in_dt, tile, m, N, P, p);
  if (s != FO_OK) return s;
  p.grid.npos = P;
  set_layout(kind, o, p);
  const int64_t total = (int64_t)P * p.grid.tiles_m * p.grid.tiles_n;
  if (count) *count = total;
  for (int64_t u = 0; u < std::min(total, capacity); ++u) {
    int pos, grp, tm, tn;
    fo::locate(p.grid, (int)u, pos, grp, tm, tn);
    out[4 * u] = pos;
    out[4 * u + 1] = grp;
    out[4 * u + 2] = tm;
    out[4 * u + 3] = tn;
  }
  return FO_OK;
}

fo_status fo_attn_schedule(int32_t P, int64_t m, int32_t hq, int32_t n_cu, int32_t* out,
                           int64_t capacity, int64_t* count, int32_t* workgroups) {
  if (P < 1 || P > FO_MAX_P || m < 1 || hq < 1 || n_cu < 1) return invalid("bad shape");
  if (count == nullptr || workgroups == nullptr || (capacity > 0 && out == nullptr))
    return invalid("NULL output");
  std::vector<int4> entries;
  std::vector<int32_t> bins;
  int32_t pairs = 0;
  if (!attn_lists(P, m, hq, n_cu, &entries, &bins, &pairs)) {
    *count = 0;
    *workgroups = 0;
    return FO_OK;
  }
  *count = (int64_t)entries.size();
  *workgroups = (int32_t)bins.size() - 1;
  int64_t k = 0;
  for (int b = 0; b + 1 < (int)bins.size(); ++b)
    for (int u = bins[b]; u < bins[b + 1] && k < capacity; ++u, ++k) {
      out[5 * k + 0] = b;
      out[5 * k + 1] = entries[u].x;
      out[5 * k + 2] = entries[u].y;
      out[5 * k + 3] = entries[u].z;
      out[5 * k + 4] = entries[u].w;
    }
  return FO_OK;
}

fo_status fo_ag_gemm(const void* x_local, const void* const* x_peer, void* x_recv, const void* w,
                     void* y, int32_t P, int32_t rank, int64_t m, int64_t K, int64_t N,
                     int32_t in_dt, int32_t out_dt, void* compute_stream, const fo_opts* opts) {
  fo_opts o;
  fo_status s = check_opts(opts, &o);
  if (s != FO_OK) return s;
  s = check_common(P, rank, m, K, N, in_dt);
  if (s != FO_OK) return s;
  if (out_dt != FO_DT_BF16 && out_dt != FO_DT_F32) return invalid("out_dt %d is not a fo_dtype", out_dt);
  if (o.arrival == FO_ARR_LOCKSTEP) return invalid("LOCKSTEP arrivals apply to fo_gemm_rs only");
  const bool act = o.epilogue == FO_EPI_SWIGLU;
  if (act && (in_dt != FO_DT_BF16 || out_dt != FO_DT_BF16 || N % 16))
    return invalid("the SwiGLU epilogue needs bf16 operands and output and N %% 16 == 0 (N %lld)",
                   (long long)N);
  const int64_t n_out = act ? N / 2 : N;  // columns of y
  const int chunks = std::max(1, o.k_chunks);
  if (chunks > 1 && (in_dt != FO_DT_BF16 || K % (256 * chunks) ||
                     (double)m * K * 2 > (double)(1 << 30)))
    return unsupported("opts.k_chunks %d needs bf16 operands, K a multiple of 256 * k_chunks and "
                       "m * K * 2 <= 2^30 bytes (K %lld, m %lld)", chunks, (long long)K,
                       (long long)m);
  const bool arrivals = x_peer != nullptr && o.arrival != FO_ARR_NONE && P > 1;
  const size_t es = dt_size(in_dt), os = dt_size(out_dt);
  const size_t align = in_dt == FO_DT_BF16 ? 16 : 4;
  if (!x_local || !w || !y || (P > 1 && !x_recv)) return invalid("NULL buffer");
  if (!aligned(x_local, align) || !aligned(w, align) || (x_recv && !aligned(x_recv, align)) ||
      !aligned(y, os))
    return invalid("misaligned buffer (inputs need %zu-byte alignment)", align);
  const size_t slice_b = (size_t)m * K * es;
  const Range r_y = rng(y, (size_t)P * m * n_out * os);
  const Range r_recv = rng(x_recv, x_recv ? (size_t)P * slice_b : 0);
  if (overlap(r_y, rng(x_local, slice_b)) || overlap(r_y, rng(w, (size_t)K * N * es)) ||
      overlap(r_y, r_recv))
    return invalid("y overlaps an input");
  if (arrivals) {
    for (int q = 0; q < P; ++q) {
      if (q == rank) continue;
      if (!x_peer[q]) return invalid("x_peer[%d] is NULL", q);
      if (!aligned(x_peer[q], align)) return invalid("x_peer[%d] misaligned", q);
      const Range rp = rng(x_peer[q], slice_b);
      if (overlap(rp, r_recv) || overlap(rp, r_y)) return invalid("x_peer[%d] overlaps x_recv or y", q);
    }
  }
  if (m == 0 || N == 0) return FO_OK;

  DevState* st = nullptr;
  std::unique_lock<std::mutex> lk;
  s = current_state(&st, &lk);
  if (s != FO_OK) return s;

  const int tile = resolve_tile(o, in_dt, out_dt, P, m, K, N, st->n_cu);
  fo::Plan p = fo::empty_plan();
  int bm = 0;
  s = tiles_for(in_dt, tile, m, N, P, p, &bm);
  if (s != FO_OK) return s;
  set_layout(0, o, p);
  p.chunks = chunks;
  // transfers on cache-line (128-byte) boundaries: no acquire needed after the arrival waits
  p.acq = (aligned(x_recv, 128) && ((size_t)(K / chunks) * es) % 128 == 0) ? 0 : 1;
  // ceil(2^32 / steps per chunk): umulhi(step, magic) = step / steps per chunk (steps < 2^16)
  p.chunk_magic = chunks > 1 ? (uint32_t)((((uint64_t)1 << 32) + K / chunks / 32 - 1) /
                                          (uint64_t)(K / chunks / 32)) : 0u;
  fo::dma::Call call{};
  if (arrivals) FO_DMA(fo::dma::begin(st->dev, P, p.grid.groups * chunks, &call, &e_));
  set_engines(o, kEnginesAG, &call);
  int32_t order[FO_MAX_P];
  fo::slice_order(0, o.order, P, rank, order);
  for (int pos = 0; pos < P; ++pos) {
    const int sl = order[pos];
    p.a_pos[pos] = sl == rank ? x_local : (const uint8_t*)x_recv + (size_t)sl * slice_b;
    p.c_pos[pos] = (uint8_t*)y + (size_t)sl * m * n_out * os;
    p.gate_slice[pos] = (arrivals && sl != rank) ? sl : -1;
  }
  p.comp_tab = call.comp_tab;
  p.b = w;
  p.done = st->done;
  p.lead = st->arr_lead;
  p.ready = st->arr_ready;
  p.gen = ++st->gen;
  p.err = st->err;
  p.spin_limit = spin_ticks(*st, o.spin_timeout_us);
  p.m = m;
  p.K = K;
  p.N = N;
  p.grid.npos = P;
  p.n_recv = 0;
  p.accum_pos = -1;
  p.out_f32 = out_dt == FO_DT_F32;
  p.act = act ? 1 : 0;

  hipStream_t cs = (hipStream_t)compute_stream;
  if (arrivals) p.start = call.start;
  s = order_after_last(st, cs);
  if (s != FO_OK) return s;
  s = launch_with_events(p, in_dt, tile, cs, o);
  if (s != FO_OK) return s;
  hipEvent_t slot_ev = nullptr;
  if (arrivals) FO_DMA(fo::dma::end(st->dev, call, cs, &e_, &slot_ev));
  s = mark_last(st, cs, slot_ev);
  if (s != FO_OK) return s;
  if (arrivals) {
    // group-major, in arrival order inside a group: the order the kernel consumes them in
    int seq[FO_MAX_P];
    const int n = arrival_sequence(0, o.order, P, rank, seq);
    const int L = links_for(o, P);
    // a K-chunk-major slice sends each row group block by block (unit g * chunks + j): rows
    // r0 .. r1 of block j are contiguous, at (j * m + r0) rows of K / chunks values
    const size_t row_b = (size_t)(K / chunks) * es;
    for (int g = 0; g < p.grid.groups; ++g) {
      int64_t r0, r1;
      group_span(p, bm, m, g, &r0, &r1);
      for (int t = 0; t < n; ++t) {
        const int sl = seq[t];
        for (int j = 0; j < chunks; ++j) {
          const size_t in_slice = ((size_t)j * m + (size_t)r0) * row_b;
          FO_DMA(fo::dma::copy(st->dev, call, t % L, sl, g * chunks + j, -1,
                               (uint8_t*)x_recv + (size_t)sl * slice_b + in_slice,
                               (const uint8_t*)x_peer[sl] + in_slice, (size_t)(r1 - r0) * row_b,
                               &e_));
        }
      }
    }
  }
  return FO_OK;
}

fo_status fo_gemm_rs(const void* x_shard, const void* w, float* send_buf, float* out,
                     const float* const* peer_partial, float* recv_buf, int32_t P, int32_t rank,
                     int64_t m, int64_t K, int64_t N, int32_t in_dt, void* compute_stream,
                     const fo_opts* opts) {
  fo_opts o;
  fo_status s = rs_check(x_shard, w, send_buf, out, peer_partial, recv_buf, P, rank, m, K, N,
                         in_dt, opts, &o);
  if (s != FO_OK || m == 0 || N == 0) return s;
  const int arrival = o.arrival == FO_ARR_DEFAULT ? FO_ARR_LOCKSTEP : o.arrival;
  const bool arrivals = peer_partial != nullptr && arrival != FO_ARR_NONE && P > 1;

  DevState* st = nullptr;
  std::unique_lock<std::mutex> lk;
  s = current_state(&st, &lk);
  if (s != FO_OK) return s;

  Words wd{};
  wd.done = st->done;
  wd.own_done = st->own_done;
  wd.err = st->err;
  wd.lead = st->arr_lead;
  wd.ready = st->arr_ready;
  wd.go = st->go;
  wd.gen = ++st->gen;
  if (++st->go_value == 0) ++st->go_value;
  wd.go_value = st->go_value;
  wd.n_cu = st->n_cu;
  wd.spin_limit = spin_ticks(*st, o.spin_timeout_us);
  fo::Plan p = fo::empty_plan();
  int bm = 0, tile = 0, own_pos = 0;
  s = rs_plan(x_shard, w, send_buf, out, recv_buf, P, rank, m, K, N, in_dt, o, wd, arrivals, &p,
              &bm, &tile, &own_pos);
  if (s != FO_OK) return s;
  const bool lockstep = arrivals && arrival == FO_ARR_LOCKSTEP;
  const bool natural = o.order == FO_ORDER_NATURAL;
  fo::dma::Call call{};
  if (arrivals) FO_DMA(fo::dma::begin(st->dev, P, p.grid.groups, &call, &e_));
  set_engines(o, kEnginesRS, &call);
  p.comp_tab = call.comp_tab;
  p.rel_tab = lockstep ? call.rel_tab : nullptr;
  if (arrivals) p.start = call.start;
  for (int i = 0; i < P - 1; ++i) {
    const int q = ((rank - 1 - i) % P + P) % P;
    p.recv_slice[i] = arrivals ? q : -1;
  }

  hipStream_t cs = (hipStream_t)compute_stream;
  s = order_after_last(st, cs);
  if (s != FO_OK) return s;
  s = launch_with_events(p, in_dt, tile, cs, o);
  if (s != FO_OK) return s;
  if (natural && P > 1) {
    s = launch_rs_reduce(p, out, m, N, wd, call.comp_tab, cs);
    if (s != FO_OK) return s;
  }
  hipEvent_t slot_ev = nullptr;
  if (arrivals) FO_DMA(fo::dma::end(st->dev, call, cs, &e_, &slot_ev));
  s = mark_last(st, cs, slot_ev);
  if (s != FO_OK) return s;
  if (arrivals) {
    // transfer t brings the partial of peer rank-1-t. In lockstep that peer sends its group g at
    // its own unit (t, g), which (peers progressing together) ends when this rank ends its unit
    // (t, g): the copy waits for that release.
    // In the NATURAL order every rank computes chunk d at step d, so all partials for this rank
    // are sent when its own position is complete.
    int seq[FO_MAX_P];
    const int n = arrival_sequence(1, FO_ORDER_FLASH, P, rank, seq);
    const int L = links_for(o, P);
    const size_t row_b = (size_t)N * 4, chunk_b = (size_t)m * N * 4;
    for (int g = 0; g < p.grid.groups; ++g) {
      int64_t r0, r1;
      group_span(p, bm, m, g, &r0, &r1);
      for (int t = 0; t < n; ++t) {
        const int q = seq[t];
        const size_t off = (size_t)q * chunk_b + (size_t)r0 * row_b;
        const int rel_pos = !lockstep ? -1 : (natural ? own_pos : t);
        FO_DMA(fo::dma::copy(st->dev, call, t % L, q, g, rel_pos,
                             (uint8_t*)recv_buf + off,
                             (const uint8_t*)peer_partial[q] + (size_t)r0 * row_b,
                             (size_t)(r1 - r0) * row_b, &e_));
      }
    }
  }
  return FO_OK;
}

fo_status fo_gemm_rs_noalloc(const void* x_shard, const void* w, float* send_buf, float* out,
                             float* recv_buf, int32_t P, int32_t rank, int64_t m, int64_t K,
                             int64_t N, int32_t in_dt, void* compute_stream, const fo_opts* opts) {
  fo_opts o;
  fo_status s = rs_check(x_shard, w, send_buf, out, nullptr, recv_buf, P, rank, m, K, N, in_dt,
                         opts, &o);
  if (s != FO_OK) return s;
  if (o.arrival != FO_ARR_DEFAULT && o.arrival != FO_ARR_NONE)
    return invalid("fo_gemm_rs_noalloc takes resident partials: opts.arrival must be DEFAULT or "
                   "NONE");
  // what the call keeps in the static array: the tile counters of P positions, the own chunk's
  // row-group words, the wait record and the start word of the tail reduce
  const int need = kNaGo + 1;
  if (P > FO_MAX_P || need * 4 > FO_NOALLOC_SCRATCH_BYTES)
    return unsupported("fo_gemm_rs_noalloc: P = %d needs more than the %d-byte scratch array", P,
                       FO_NOALLOC_SCRATCH_BYTES);
  if (m == 0 || N == 0) return FO_OK;
  NoAllocDev* na = nullptr;
  std::unique_lock<std::mutex> lk;
  s = noalloc_state(&na, &lk);
  if (s != FO_OK) return s;

  Words wd{};
  wd.done = na->ptr + kNaCounters;
  wd.own_done = na->ptr + kNaOwn;
  wd.err = na->ptr + kNaErr;
  wd.go = na->ptr + kNaGo;
  if (++na->gen == 0) ++na->gen;
  wd.gen = na->gen;
  wd.go_value = na->gen;
  wd.n_cu = na->n_cu;
  wd.spin_limit = (uint64_t)o.spin_timeout_us * na->wall_khz / 1000u;
  fo::Plan p = fo::empty_plan();
  int bm = 0, tile = 0, own_pos = 0;
  s = rs_plan(x_shard, w, send_buf, out, recv_buf, P, rank, m, K, N, in_dt, o, wd, false, &p, &bm,
              &tile, &own_pos);
  if (s != FO_OK) return s;
  hipStream_t cs = (hipStream_t)compute_stream;
  // the counters and the own chunk's words start at zero in every call (a kernel, so that the
  // call can be captured in a HIP graph)
  FO_HIP(fo::launch_zero(na->ptr + kNaCounters, kNaErr - kNaCounters, cs));
  s = launch_with_events(p, in_dt, tile, cs, o);
  if (s != FO_OK) return s;
  if (o.order == FO_ORDER_NATURAL && P > 1) return launch_rs_reduce(p, out, m, N, wd, nullptr, cs);
  return FO_OK;
}

fo_status fo_gemm_ref(const void* a, const void* b, void* c, int64_t M, int64_t K, int64_t N,
                      int32_t in_dt, int32_t out_dt, int32_t tile, void* stream) {
  fo_status s = check_common(1, 0, M, K, N, in_dt);
  if (s != FO_OK) return s;
  if (out_dt != FO_DT_BF16 && out_dt != FO_DT_F32) return invalid("out_dt %d is not a fo_dtype", out_dt);
  if (tile < FO_TILE_AUTO || tile > FO_TILE_64x64) return invalid("tile %d is not a fo_tile", tile);
  const size_t es = dt_size(in_dt), os = dt_size(out_dt);
  const size_t align = in_dt == FO_DT_BF16 ? 16 : 4;
  if (!a || !b || !c) return invalid("NULL buffer");
  if (!aligned(a, align) || !aligned(b, align) || !aligned(c, os)) return invalid("misaligned buffer");
  const Range rc = rng(c, (size_t)M * N * os);
  if (overlap(rc, rng(a, (size_t)M * K * es)) || overlap(rc, rng(b, (size_t)K * N * es)))
    return invalid("c overlaps an input");
  if (M == 0 || N == 0) return FO_OK;

  DevState* st = nullptr;
  std::unique_lock<std::mutex> lk;
  s = current_state(&st, &lk);
  if (s != FO_OK) return s;
  fo_opts o;
  fo_opts_init(&o);
  o.tile = tile;
  const int t = resolve_tile(o, in_dt, out_dt, 1, M, K, N, st->n_cu);
  fo::Plan p = fo::empty_plan();
  s = tiles_for(in_dt, t, M, N, 1, p);
  if (s != FO_OK) return s;
  p.a_pos[0] = a;
  p.c_pos[0] = c;
  p.b = b;
  p.done = st->done;
  p.lead = st->arr_lead;
  p.ready = st->arr_ready;
  p.gen = ++st->gen;
  p.err = st->err;
  p.spin_limit = spin_ticks(*st, kDefaultTimeoutUs);
  p.m = M;
  p.K = K;
  p.N = N;
  p.grid.npos = 1;
  p.accum_pos = -1;
  p.out_f32 = out_dt == FO_DT_F32;
  set_groups(1, p);
  p.grid.lead = 1;
  FO_HIP(fo::launch_gemm(p, in_dt, t, (hipStream_t)stream));
  return FO_OK;
}

fo_status fo_swiglu(const void* y, void* h, int64_t rows, int64_t inter, void* stream) {
  if (rows < 0 || inter < 0) return invalid("negative size (rows %lld, inter %lld)", (long long)rows,
                                            (long long)inter);
  if (inter % 8) return invalid("inter %lld is not a multiple of 8", (long long)inter);
  if (rows > ((int64_t)1 << 40) || inter > ((int64_t)1 << 30)) return invalid("sizes too large");
  if (rows == 0 || inter == 0) return FO_OK;
  if (!y || !h) return invalid("NULL buffer");
  if (!aligned(y, 16) || !aligned(h, 16)) return invalid("misaligned buffer (16-byte alignment)");
  if (overlap(rng(y, (size_t)rows * 2 * inter * 2), rng(h, (size_t)rows * inter * 2)))
    return invalid("h overlaps y");
  FO_HIP(fo::launch_swiglu(y, h, rows, inter, (hipStream_t)stream));
  return FO_OK;
}

// Shapes of the attention calls: head_dim 128 only, whole query heads per key head (GQA), and
// 32-bit byte offsets inside one slice of rows.
static fo_status check_attn(int32_t P, int32_t rank, int64_t m, int32_t hq, int32_t hkv,
                            int32_t head_dim, int32_t causal) {
  if (P < 1 || P > FO_MAX_P || rank < 0 || rank >= P) return invalid("bad P %d / rank %d", P, rank);
  if (m < 0) return invalid("negative m %lld", (long long)m);
  if (hq < 1 || hkv < 1 || hq % hkv) return invalid("hq %d must be a positive multiple of hkv %d", hq, hkv);
  if (causal != 0 && causal != 1) return invalid("causal must be 0 or 1");
  if (head_dim != 128) return unsupported("head_dim %d (the attention kernel is built for 128)", head_dim);
  const int64_t W = (int64_t)(hq + 2 * hkv) * 256;
  if ((m + 128) * W >= ((int64_t)1 << 31)) return invalid("a slice of rows is too large");
  return FO_OK;
}

// Causal attention whose workgroups all fit at once (two per CU) and fill the second slot of
// every CU: pair long and short query tiles (AttnPlan::pair_half).
static int32_t attn_pair_half(int32_t P, int64_t m, int32_t hq, int32_t causal, int n_cu) {
  const int64_t total = (int64_t)P * ((m + 127) / 128) * hq;
  return (causal && total % 2 == 0 && total > n_cu && total <= 2 * (int64_t)n_cu) ? (int32_t)(total / 2) : 0;
}

// The attention's work table for causal calls. Under causal masking the items' key walks run
// from 1 to P * m / 64 tiles, and with one workgroup per item the longest ones set the kernel's
// time (70B share, 8K tokens: a CU running a 128-tile item next to a 2-tile one ended at 183 us,
// CUs with two 65-tile items at 128 us). Instead each CU's two workgroups (b and b + CUs, all
// resident at once) take lists of items that give every CU the same work:
//   - items longer than a workgroup slot's share are cut in two along their key walk;
//   - the items go longest first to the least loaded CU, each counted with a fixed cost for its
//     query load, pipeline fill and epilogue;
//   - a CU's items are divided between its two workgroups so that the first one dispatched takes
//     about 60% of the cost: of two workgroups sharing a CU the older one ran a key tile in ~1.7
//     us and the younger in ~2.5 (16K tokens), so both then end together.
// Measured and not kept: assigning each item to the list that would end it first (the same for
// resident calls, slower behind the transfers: 8K, both exchanges, 260 against 246 us), taking
// the slices one after another in arrival order (under causal masking the slice that arrives
// first may need every other slice's keys: 194 -> 231 us inbound), and the own slice's items
// last with the return exchange (246 -> 259 us).
static fo_status attn_schedule(DevState* st, fo::AttnPlan& p) {
  p.table = nullptr;
  p.bins = nullptr;
  if (!p.causal) return FO_OK;
  const DevState::AttnTable* t = nullptr;
  for (const auto& e : st->attn_tables)
    if (e.P == p.P && e.m == p.m && e.hq == p.hq && e.causal == p.causal) t = &e;
  if (t == nullptr) {
    std::vector<int4> host;
    std::vector<int32_t> bins;
    int32_t pairs = 0;
    if (!attn_lists(p.P, p.m, p.hq, st->n_cu, &host, &bins, &pairs)) return FO_OK;
    if (st->attn_tables.size() >= kAttnTablesMax) {
      // a bounded cache: past this many shapes the tables are dropped (after every earlier
      // launch that may read one has ended) and built again as shapes come back
      FO_HIP(hipDeviceSynchronize());
      for (const auto& e : st->attn_tables) FO_HIP(hipFree(e.table));
      st->attn_tables.clear();
    }
    const int nb = (int)bins.size() - 1;
    const size_t tb = host.size() * sizeof(int4), bb = bins.size() * sizeof(int32_t);
    void* d = nullptr;
    FO_HIP(hipMalloc(&d, tb + bb));
    FO_HIP(hipMemcpy(d, host.data(), tb, hipMemcpyHostToDevice));
    FO_HIP(hipMemcpy((uint8_t*)d + tb, bins.data(), bb, hipMemcpyHostToDevice));
    st->attn_tables.push_back({p.P, p.hq, p.causal, p.m, (int4*)d,
                               (int32_t*)((uint8_t*)d + tb), (int32_t)host.size(), nb, pairs});
    t = &st->attn_tables.back();
  }
  if (t->n_pairs > st->attn_pairs_cap) {
    // grown to the largest call so far; the previous buffers may still be in use by an earlier
    // call's kernel
    FO_HIP(hipDeviceSynchronize());
    if (st->attn_part) FO_HIP(hipFree(st->attn_part));
    if (st->attn_cnt) FO_HIP(hipFree(st->attn_cnt));
    st->attn_part = nullptr;
    st->attn_cnt = nullptr;
    st->attn_pairs_cap = 0;
    const size_t n = (size_t)t->n_pairs;
    FO_HIP(hipMalloc((void**)&st->attn_part, n * 2 * fo::kAttnPartFloats * sizeof(float)));
    FO_HIP(hipMalloc((void**)&st->attn_cnt, n * sizeof(uint32_t)));
    FO_HIP(hipMemset(st->attn_cnt, 0, n * sizeof(uint32_t)));
    st->attn_pairs_cap = t->n_pairs;
  }
  p.table = t->table;
  p.bins = t->bins;
  p.n_items = t->n_items;
  p.n_bins = t->n_bins;
  p.part_buf = st->attn_part;
  p.pair_cnt = st->attn_cnt;
  if (t->n_pairs > 0 && (p.part_buf == nullptr || p.pair_cnt == nullptr)) return FO_ERR_HIP;
  return FO_OK;
}

static fo_status launch_attn_events(const fo::AttnPlan& p, hipStream_t cs, const fo_opts& o) {
  FO_HIP(fo::launch_attn(p, cs, (hipEvent_t)o.kernel_events[0], (hipEvent_t)o.kernel_events[1]));
  return FO_OK;
}

fo_status fo_attn(const void* qkv_local, const void* const* qkv_peer, void* qkv_recv, void* out,
                  void* const* out_peer, int32_t P, int32_t rank, int64_t m, int32_t hq,
                  int32_t hkv, int32_t head_dim, int32_t causal, void* compute_stream,
                  const fo_opts* opts) {
  fo_opts o;
  fo_status s = check_opts(opts, &o);
  if (s != FO_OK) return s;
  s = check_attn(P, rank, m, hq, hkv, head_dim, causal);
  if (s != FO_OK) return s;
  if (o.arrival == FO_ARR_LOCKSTEP) return invalid("LOCKSTEP arrivals apply to fo_gemm_rs only");
  if (o.tile != FO_TILE_AUTO) return invalid("opts.tile applies to the GEMM calls only");
  if (o.epilogue != FO_EPI_NONE) return invalid("opts.epilogue applies to fo_ag_gemm only");
  if (o.k_chunks > 1) return invalid("opts.k_chunks applies to fo_ag_gemm only");
  const bool arrivals = qkv_peer != nullptr && o.arrival != FO_ARR_NONE && P > 1;
  const bool sends = out_peer != nullptr && P > 1;
  if (sends && 2 * P > FO_MAX_P)
    return unsupported("the return exchange needs P <= %d (P = %d)", FO_MAX_P / 2, P);
  const size_t W = (size_t)(hq + 2 * hkv) * 256, slice_b = (size_t)m * W;
  const size_t ow = (size_t)hq * 256, oslice_b = (size_t)m * ow;
  if (!qkv_local || !out || (P > 1 && !qkv_recv)) return invalid("NULL buffer");
  if (!aligned(qkv_local, 16) || !aligned(out, 16) || (qkv_recv && !aligned(qkv_recv, 16)))
    return invalid("misaligned buffer (16-byte alignment)");
  const Range r_out = rng(out, (size_t)P * oslice_b);
  const Range r_recv = rng(qkv_recv, qkv_recv ? (size_t)P * slice_b : 0);
  const Range r_local = rng(qkv_local, slice_b);
  if (overlap(r_out, r_local) || overlap(r_out, r_recv)) return invalid("out overlaps an input");
  if (arrivals) {
    for (int q = 0; q < P; ++q) {
      if (q == rank) continue;
      if (!qkv_peer[q]) return invalid("qkv_peer[%d] is NULL", q);
      if (!aligned(qkv_peer[q], 16)) return invalid("qkv_peer[%d] misaligned", q);
      const Range rp = rng(qkv_peer[q], slice_b);
      if (overlap(rp, r_recv) || overlap(rp, r_out)) return invalid("qkv_peer[%d] overlaps qkv_recv or out", q);
    }
  }
  if (sends) {
    for (int q = 0; q < P; ++q) {
      if (q == rank) continue;
      if (!out_peer[q]) return invalid("out_peer[%d] is NULL", q);
      if (!aligned(out_peer[q], 16)) return invalid("out_peer[%d] misaligned", q);
      const Range rp = rng(out_peer[q], oslice_b);
      if (overlap(rp, r_out) || overlap(rp, r_recv) || overlap(rp, r_local))
        return invalid("out_peer[%d] overlaps out or an input", q);
      for (int q2 = 0; q2 < q; ++q2)
        if (q2 != rank && overlap(rp, rng(out_peer[q2], oslice_b)))
          return invalid("out_peer[%d] overlaps out_peer[%d]", q, q2);
    }
  }
  if (m == 0) return FO_OK;

  DevState* st = nullptr;
  std::unique_lock<std::mutex> lk;
  s = current_state(&st, &lk);
  if (s != FO_OK) return s;
  fo::AttnPlan p{};
  // row groups: opts.row_groups (0: whole slices), each a multiple of the 128-row query tile.
  // Whole slices by default: every further copy costs the engine ~9 us of its own, more than a
  // group's earlier start saves here.
  const int req = o.row_groups ? o.row_groups : 1;
  const int64_t gr = ((m + req - 1) / req + 127) / 128 * 128;
  p.group_rows = gr;
  p.groups = (int32_t)((m + gr - 1) / gr);
  // outgoing groups: the arriving groups (whole slices by default). Sending each 128-row query
  // tile as soon as it is done measured far slower (70B share, S = 8192: 273 -> 398 us): 56
  // small transfers per call each pay the engines' per-copy cost.
  const int64_t ogr = gr;
  p.out_group_rows = ogr;
  p.out_groups = (int32_t)((m + ogr - 1) / ogr);
  fo::dma::Call call{};
  if (arrivals || sends)
    FO_DMA(fo::dma::begin(st->dev, sends ? 2 * P : P, std::max(p.groups, p.out_groups), &call,
                          &e_));
  set_engines(o, kEnginesAttn, &call);
  int32_t order[FO_MAX_P];
  fo::slice_order(0, o.order, P, rank, order);
  for (int i = 0; i < P; ++i) {
    p.order[i] = order[i];
    p.slice[i] = i == rank ? qkv_local : (const uint8_t*)qkv_recv + (size_t)i * slice_b;
    p.gated[i] = (arrivals && i != rank) ? 1 : 0;
    p.send[i] = (sends && i != rank) ? 1 : 0;
  }
  // dispatch: the arrival order; with the return exchange in the FLASH order the own slice goes
  // last (its rows stay on the rank, so the slice computed last has nothing left to send), the
  // Flash-RS order of the page's rank-adaptive schedule applied to the outgoing exchange; the
  // data-slicing (NATURAL) order keeps index order
  const bool own_last = sends && o.order == FO_ORDER_FLASH;
  int n_disp = 0;
  for (int i = 0; i < P; ++i)
    if (!(own_last && order[i] == rank)) p.dispatch[n_disp++] = order[i];
  if (own_last) p.dispatch[n_disp++] = rank;
  p.out = out;
  p.comp_tab = call.comp_tab;
  p.rel_tab = sends ? call.rel_tab : nullptr;
  p.done = st->done;
  p.lead = st->arr_lead;
  p.ready = st->arr_ready;
  p.gen = ++st->gen;
  p.err = st->err;
  p.spin_limit = spin_ticks(*st, o.spin_timeout_us);
  p.m = m;
  p.P = P;
  p.hq = hq;
  p.hkv = hkv;
  p.causal = causal;
  p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
  p.pair_half = attn_pair_half(P, m, hq, causal, st->n_cu);
  s = attn_schedule(st, p);
  if (s != FO_OK) return s;
  // transfers on cache-line (128-byte) boundaries: no acquire needed after the arrival waits
  const size_t row_bytes = (size_t)(hq + 2 * hkv) * head_dim * 2;
  p.acq = (aligned(qkv_recv, 128) && row_bytes % 128 == 0) ? 0 : 1;

  hipStream_t cs = (hipStream_t)compute_stream;
  if (arrivals || sends) p.start = call.start;
  s = order_after_last(st, cs);
  if (s != FO_OK) return s;
  s = launch_attn_events(p, cs, o);
  if (s != FO_OK) return s;
  int seq[FO_MAX_P];
  const int n = arrival_sequence(0, o.order, P, rank, seq);
  if (sends) {
    // the call ends when its outgoing rows have landed: a one-workgroup kernel after the
    // attention waits for the completion of every send
    int out_ids[FO_MAX_P];
    for (int t = 0; t < n; ++t) out_ids[t] = P + seq[t];
    FO_HIP(fo::launch_wait(call.comp_tab, out_ids, n, p.out_groups, p.spin_limit, st->err, p.gen,
                           cs));
  }
  hipEvent_t slot_ev = nullptr;
  if (arrivals || sends) FO_DMA(fo::dma::end(st->dev, call, cs, &e_, &slot_ev));
  s = mark_last(st, cs, slot_ev);
  if (s != FO_OK) return s;
  const int L = links_for(o, P);
  if (arrivals) {
    for (int g = 0; g < p.groups; ++g) {
      const int64_t r0 = g * gr, r1 = std::min<int64_t>(m, r0 + gr);
      for (int t = 0; t < n; ++t) {
        const int sl = seq[t];
        FO_DMA(fo::dma::copy(st->dev, call, t % L, sl, g, -1,
                             (uint8_t*)qkv_recv + (size_t)sl * slice_b + (size_t)r0 * W,
                             (const uint8_t*)qkv_peer[sl] + (size_t)r0 * W, (size_t)(r1 - r0) * W, &e_));
      }
    }
  }
  if (sends) {
    // slice s's output rows to rank s, group by group once released, over the link its slice
    // arrived on, in the other direction (with one engine per link: the partner engine of that
    // link's pair, so that the two directions are separate queues)
    const int half = std::max(1, fo::dma::n_engines(st->dev) / 2);
    for (int g = 0; g < p.out_groups; ++g) {
      const int64_t r0 = g * ogr, r1 = std::min<int64_t>(m, r0 + ogr);
      for (int t = 0; t < n; ++t) {
        const int sl = seq[t];
        FO_DMA(fo::dma::copy(st->dev, call, (t % L) + half, P + sl, g, sl,
                             (uint8_t*)out_peer[sl] + (size_t)r0 * ow,
                             (const uint8_t*)out + ((size_t)sl * m + (size_t)r0) * ow,
                             (size_t)(r1 - r0) * ow, &e_));
      }
    }
  }
  return FO_OK;
}

fo_status fo_attn_ref(const void* qkv, void* out, int64_t S, int32_t hq, int32_t hkv,
                      int32_t head_dim, int32_t causal, void* stream) {
  fo_status s = check_attn(1, 0, S, hq, hkv, head_dim, causal);
  if (s != FO_OK) return s;
  if (!qkv || !out) return invalid("NULL buffer");
  if (!aligned(qkv, 16) || !aligned(out, 16)) return invalid("misaligned buffer (16-byte alignment)");
  if (overlap(rng(out, (size_t)S * hq * 256), rng(qkv, (size_t)S * (hq + 2 * hkv) * 256)))
    return invalid("out overlaps qkv");
  if (S == 0) return FO_OK;
  DevState* st = nullptr;
  std::unique_lock<std::mutex> lk;
  s = current_state(&st, &lk);
  if (s != FO_OK) return s;
  fo::AttnPlan p{};
  p.group_rows = (S + 127) / 128 * 128;
  p.groups = 1;
  p.order[0] = 0;
  p.dispatch[0] = 0;
  p.slice[0] = qkv;
  p.gated[0] = 0;
  p.out = out;
  p.err = st->err;
  p.spin_limit = spin_ticks(*st, kDefaultTimeoutUs);
  p.m = S;
  p.P = 1;
  p.hq = hq;
  p.hkv = hkv;
  p.causal = causal;
  p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
  p.pair_half = attn_pair_half(1, S, hq, causal, st->n_cu);
  s = attn_schedule(st, p);
  if (s != FO_OK) return s;
  hipStream_t cs = (hipStream_t)stream;
  if (p.table != nullptr) {
    // split items share the device's partial buffers: ordered after the device's last call
    s = order_after_last(st, cs);
    if (s != FO_OK) return s;
  }
  FO_HIP(fo::launch_attn(p, cs));
  if (p.table != nullptr) return mark_last(st, cs, nullptr);
  return FO_OK;
}

fo_status fo_transfer_ref(int32_t kind, const void* const* src, void* dst, int32_t P,
                          int32_t rank, int64_t slice_bytes, void* stream, const fo_opts* opts) {
  fo_opts o;
  fo_status s = check_opts(opts, &o);
  if (s != FO_OK) return s;
  if (o.epilogue != FO_EPI_NONE) return invalid("opts.epilogue applies to fo_ag_gemm only");
  if (o.k_chunks > 1) return invalid("opts.k_chunks applies to fo_ag_gemm only");
  if (kind != 0 && kind != 1) return invalid("kind %d is neither 0 (AG) nor 1 (RS)", kind);
  if (P < 1 || P > FO_MAX_P || rank < 0 || rank >= P) return invalid("bad P %d / rank %d", P, rank);
  if (slice_bytes < 0 || slice_bytes % 4) return invalid("slice_bytes must be a multiple of 4");
  if (!src || !dst) return invalid("NULL buffer");
  const Range rd = rng(dst, (size_t)P * slice_bytes);
  for (int q = 0; q < P; ++q) {
    if (q == rank) continue;
    if (!src[q]) return invalid("src[%d] is NULL", q);
    if (overlap(rng(src[q], slice_bytes), rd)) return invalid("src[%d] overlaps dst", q);
  }
  if (P == 1 || slice_bytes == 0) return FO_OK;
  DevState* st = nullptr;
  std::unique_lock<std::mutex> lk;
  s = current_state(&st, &lk);
  if (s != FO_OK) return s;
  // the slices cut into opts.row_groups equal pieces (0: whole), issued group-major like the calls
  const int G = std::max(1, o.row_groups);
  fo::dma::Call call{};
  FO_DMA(fo::dma::begin(st->dev, P, G, &call, &e_));
  set_engines(o, kind == 1 ? kEnginesRS : kEnginesAG, &call);
  int seq[FO_MAX_P];
  const int n = arrival_sequence(kind, o.order, P, rank, seq);
  hipStream_t ks = (hipStream_t)stream;
  s = order_after_last(st, ks);
  if (s != FO_OK) return s;
  FO_HIP(fo::launch_release(call.start, ks));
  FO_HIP(fo::launch_wait(call.comp_tab, seq, n, G, spin_ticks(*st, o.spin_timeout_us), st->err,
                         ++st->gen, ks));
  hipEvent_t slot_ev = nullptr;
  FO_DMA(fo::dma::end(st->dev, call, ks, &e_, &slot_ev));
  s = mark_last(st, ks, slot_ev);
  if (s != FO_OK) return s;
  const int L = links_for(o, P);
  const size_t piece = ((size_t)slice_bytes / G + 255) / 256 * 256;
  for (int g = 0; g < G; ++g) {
    const size_t b0 = std::min((size_t)slice_bytes, (size_t)g * piece);
    const size_t b1 = std::min((size_t)slice_bytes, (size_t)(g + 1) * piece);
    for (int t = 0; t < n; ++t) {
      const int sl = seq[t];
      FO_DMA(fo::dma::copy(st->dev, call, t % L, sl, g, -1,
                           (uint8_t*)dst + (size_t)sl * slice_bytes + b0,
                           (const uint8_t*)src[sl] + b0, b1 - b0, &e_));
    }
  }
  return FO_OK;
}

fo_status fo_check(void* stream) {
  FO_HIP(hipStreamSynchronize((hipStream_t)stream));
  int dev = 0;
  FO_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return FO_OK;
  // the wait records: the library's (fo_ag_gemm, fo_gemm_rs, fo_attn, fo_transfer_ref) and the
  // scratch array's (fo_gemm_rs_noalloc); each is read, then its "what failed" word cleared
  uint32_t kinds = 0;
  {
    DevState& st = g_dev[dev];
    std::lock_guard<std::mutex> lk(st.mu);
    if (st.ready) {
      std::string e;
      bool timed_out = false;
      if (!fo::dma::drain(dev, 30000, &e, &timed_out)) {
        set_error("%s", e.c_str());
        return timed_out ? FO_ERR_TIMEOUT : FO_ERR_HIP;
      }
      uint32_t w = 0;
      FO_HIP(hipMemcpy(&w, st.err, sizeof w, hipMemcpyDeviceToHost));
      if (w) {
        const uint32_t zero = 0;
        FO_HIP(hipMemcpy(st.err, &zero, sizeof zero, hipMemcpyHostToDevice));
      }
      kinds |= w;
    }
  }
  {
    NoAllocDev& na = g_na[dev];
    std::lock_guard<std::mutex> lk(na.mu);
    if (na.ptr != nullptr) {
      uint32_t w = 0;
      FO_HIP(hipMemcpy(&w, na.ptr + kNaErr, sizeof w, hipMemcpyDeviceToHost));
      if (w) {
        const uint32_t zero = 0;
        FO_HIP(hipMemcpy(na.ptr + kNaErr, &zero, sizeof zero, hipMemcpyHostToDevice));
      }
      kinds |= w;
    }
  }
  if (kinds & 2u) {
    set_error("a DMA transfer reported failure");
    return FO_ERR_HIP;
  }
  if (kinds) {
    set_error("an in-kernel arrival wait ran past its bound");
    return FO_ERR_TIMEOUT;
  }
  return FO_OK;
}

}  // extern "C"
