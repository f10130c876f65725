// Query-split attention behind a Flash All-to-All: one rank's share of Ulysses (sequence)
// parallelism on MI355X (gfx950).
//
// The FlashOverlap page (gist.science paper 2604.24013), technical summary §2 "Methodology",
// extends the sliced overlap in two ways: attention computed by query slices, for overlap at a
// finer grain, and the All-to-All of Ulysses parallelism decomposed like the All-Gather. After
// the All-to-All a rank holds, for its own heads, the query, key and value rows of every peer's
// sequence chunk (slice s = sequence positions s*m .. s*m+m-1). Here the slices arrive in row
// groups (emulated copies, group by group as for Flash-AG; whole slices by default) and the
// attention runs by query slices: a workgroup takes 128 queries of one head of slice s as soon as
// their row group has landed, and walks the key slices in arrival order, waiting before each for
// the row groups that hold the keys it reads (with causal masking only the slices j <= s). The
// online softmax makes the order of the keys irrelevant up to rounding.
//
// Kernel design (CDNA4):
// - One work item per (slice, 128-query tile, head): 4 waves of 32 queries; key tiles of 64.
//   Causal calls run from a table built on the host: each workgroup (two per CU, all resident)
//   walks its own list of items, and an item longer than a workgroup's share of the key tiles
//   is cut in two along its key walk, each half storing its unnormalized output, running max
//   and sum, the second to finish combining them in a fixed order (attn_tile's end).
// - Scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16, K from LDS as the A
//   operand, Q in registers as the B operand), so that each lane owns one query: the softmax
//   row state (running max and sum) is per lane, and a row reduction needs one cross-lane swap.
// - The output is accumulated transposed too, O^T += V^T P^T: the probabilities go from the
//   score accumulators straight into the B operand (bf16) without moving between lanes, because
//   the keys of a 16-key MFMA step are numbered in the order the accumulator holds them; V^T's A
//   operand is read with the same numbering by transpose reads (ds_read_b64_tr_b16).
// - K and V tiles are filled straight from HBM into a 2-stage LDS ring by LDS-writing buffer
//   loads (16 bytes per lane); rows past a slice read zeros through the buffer range check and
//   are masked. K rows are XOR-swizzled by key (the A-operand reads of 32 keys at one offset
//   spread over the banks), V rows by key mod 4 (the transpose reads: chunk XOR (0, 6, 12,
//   10)[key & 3], which gives the 4 key rows x 4 chunks a 32-lane read covers distinct bank
//   groups whether the LDS serves 128 or 256 bytes per cycle).
// - Two workgroups per CU (64 KB of LDS each), two waves per SIMD, so that a wave's softmax can
//   run while the other wave of its SIMD issues MFMAs (they fill each other's gaps only in
//   part: the kernel stays latency-bound).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fo_internal.h"
#include "fo_wait.h"

namespace fo {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int kThreads = 256;
constexpr int kAQ = 128;                   // queries per workgroup (4 waves x 32)
constexpr int kAK = 64;                    // keys per tile
constexpr int kAD = 128;                   // head dim
constexpr int kRowB = kAD * 2;             // one head's row of K or V: 256 bytes
constexpr int kTileB = kAK * kRowB;        // one K or V tile in LDS: 16 KB
constexpr int kStage = 2 * kTileB;         // K tile, then V tile
constexpr int kStages = 2;
constexpr int kPieces = kTileB / 1024;     // 1 KB loads per tile (16), 4 per wave
constexpr int kLoads = 2 * kPieces / 4;    // loads per wave per key tile (K and V): 8
constexpr int kOutStride = kRowB + 16;     // output staging row (bytes): 16-byte aligned, padded
constexpr float kNegBig = -1.0e30f;        // "minus infinity" that keeps exp2 finite
constexpr float kLazyLog2 = 8.0f;          // growth of a row max (log2 units) that moves it
constexpr int kRsrcWord3 = 0x00020000;     // raw buffer, 32-bit data format
static_assert(4 * 32 * kOutStride <= kStages * kStage, "output staging fits in the ring");

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const void* uni_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = (uint32_t)uni((int)(uint32_t)v), hi = (uint32_t)uni((int)(uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}
// raw buffer descriptor (wave-uniform: SGPRs), as the int vector the LDS-load asm takes
__device__ __forceinline__ i32x4 rsrc_i(const void* base, uint32_t bytes) {
  const uint64_t v = (uint64_t)uni_ptr(base);
  i32x4 r;
  r.x = uni((int)(uint32_t)v);
  r.y = uni((int)(uint32_t)(v >> 32));
  r.z = uni((int)bytes);
  r.w = kRsrcWord3;
  return r;
}
// the same descriptor in the type of the buffer load/store builtins
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_b(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uni_ptr(base)), (short)0,
                                           (int)uni((int)bytes), kRsrcWord3);
}

// 16 bytes per lane from the buffer at byte offset voff into LDS at m0v + 16 * lane (an offset
// past num_records reads zeros). Issued as inline assembly so that the compiler neither waits
// for it at barriers nor orders LDS reads behind it; completion is counted with wait_vmcnt.
__device__ __forceinline__ void load_lds16(i32x4 rsrc, uint32_t m0v, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(m0v), "v"(voff), "s"(rsrc)
      : "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// workgroup barrier after this wave's LDS accesses, without a memory fence
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// chunk swizzle of a V row (256 bytes, 16 chunks) by its key: (0, 6, 12, 10)[key & 3]
__device__ __forceinline__ int vswz(int key) { return (0xAC60 >> ((key & 3) * 4)) & 15; }

__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Thread 0 waits until row groups g0..g1 of slice j have landed; the barrier holds the other
// waves until then. With p.acq thread 0 also acquires at system scope (invalidating this CU's L1
// and its XCD's L2) before the barrier; without it (every transfer on 128-byte cache-line
// boundaries) no cache can hold a stale line of the rows: the launch invalidated what earlier
// kernels cached, and nothing reads a row before its transfer has landed.
__device__ __forceinline__ void wait_groups(const AttnPlan& p, int j, int g0, int g1) {
  if (threadIdx.x == 0 && p.comp_tab != nullptr) {
    for (int g = g0; g <= g1; ++g)
      wait_group(p.comp_tab, p.lead, p.ready, p.gen, p.spin_limit, p.err, j, g);
    if (p.acq) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
  }
  __syncthreads();
}

__device__ __forceinline__ void attn_tile(const AttnPlan& p, const int u, uint8_t* const lds,
                                          uint32_t* const bcast) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int lh = lane >> 5, l32 = lane & 31, g16 = lane >> 4, i16 = lane & 15;
  const int m = (int)p.m;
  const int hq = p.hq;
  const int qtiles = (m + kAQ - 1) / kAQ;
  int s, qt, h, wpart = -1;
  if (p.table != nullptr) {
    const int4 e = p.table[u];
    s = uni(e.x);
    qt = uni(e.y);
    h = uni(e.z);
    wpart = uni(e.w);
  } else if (p.pair_half > 0) {
    // items by global query tile, most keys first; the second half of the grid in reverse, so
    // that workgroup b and workgroup b + pair_half (which share a CU) sum to about the same work
    const int total = p.P * qtiles * hq;
    const int v = u < p.pair_half ? u : total - 1 - (u - p.pair_half);
    const int g = p.P * qtiles - 1 - v / hq;
    s = uni(g / qtiles);
    qt = uni(g % qtiles);
    h = uni(v % hq);
  } else {
    const int per_pos = qtiles * hq;
    const int pos = uni(u / per_pos);
    const int rr = u - pos * per_pos;
    // inside a slice, the query tiles with the most keys (the last ones, under causal masking)
    // are dispatched first
    qt = uni(qtiles - 1 - rr / hq);
    h = uni(rr % hq);
    s = uni(p.dispatch[pos]);
  }
  const int kvh = h / (hq / p.hkv);
  const int W = (hq + 2 * p.hkv) * kRowB;  // bytes of one token's Q, K and V rows
  const int q0 = qt * kAQ;
  const int qrows = m - q0 < kAQ ? m - q0 : kAQ;
  const int64_t qpos = (int64_t)s * m + q0 + 32 * wave + l32;  // this lane's query position
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;

  const int gr = (int)p.group_rows;
  // the query rows' group (group_rows is a multiple of the 128-row query tile)
  if (p.gated[s]) wait_groups(p, s, 0, q0 / gr);

  // Q of this lane's query as the B operand of S^T = K Q^T: K step kd holds the head-dim values
  // 16 kd + 8 lh .. 16 kd + 8 lh + 7 (rows past the slice read zeros and are never stored)
  bf16x8 qf[kAD / 16];
  {
    const __amdgpu_buffer_rsrc_t qres = rsrc_b(p.slice[s], (uint32_t)m * (uint32_t)W);
    const uint32_t qoff = (uint32_t)(q0 + 32 * wave + l32) * (uint32_t)W + h * kRowB + lh * 16;
#pragma unroll
    for (int kd = 0; kd < kAD / 16; ++kd)
      qf[kd] = __builtin_bit_cast(bf16x8,
                                  __builtin_amdgcn_raw_buffer_load_b128(qres, qoff + kd * 32, 0, 0));
  }
  wait_vmcnt<0>();

  f32x16 oacc[kAD / 32];
#pragma unroll
  for (int i = 0; i < kAD / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[i][v] = 0.f;
  float mrow = kNegBig, lrow = 0.f;

  // per-lane LDS offsets of the loads: a 1 KB piece covers 4 key rows, lane -> (row, chunk)
  const int prow = lane >> 4, pch = lane & 15;

  // the key tiles of the item's walk (every slice, or under causal masking the slices j < s and
  // the diagonal slice up to the tile's last query), numbered in walk order; a part of a split
  // item visits walk tiles [w_lo, w_hi) only
  const int mt = (m + kAK - 1) / kAK;
  const int wtot = p.causal ? s * mt + (q0 + qrows + kAK - 1) / kAK : p.P * mt;
  int w_lo = 0, w_hi = wtot;
  if (wpart >= 0) {
    const int cut = (wtot + 1) / 2;
    if (wpart & 1)
      w_lo = cut;
    else
      w_hi = cut;
  }
  int wt = 0;  // walk tiles before slice j

  for (int jp = 0; jp < p.P; ++jp) {
    const int j = uni(p.order[jp]);
    if (p.causal && j > s) continue;
    // keys of slice j to visit: all of them, or (the diagonal slice, causal) up to the tile's
    // last query
    const int nk = (p.causal && j == s) ? (q0 + qrows) : m;
    const int nt = (nk + kAK - 1) / kAK;
    // this item's tiles of slice j: [lo, hi)
    const int lo = w_lo - wt > 0 ? w_lo - wt : 0;
    const int hi = w_hi - wt < nt ? w_hi - wt : nt;
    wt += nt;
    if (lo >= hi) continue;
    // the row groups holding those keys, all before the walk (a wait inside the tile loop slows
    // its code down more than an earlier start of a slice's first groups gains)
    if (p.gated[j]) wait_groups(p, j, lo * kAK / gr, ((hi * kAK < nk ? hi * kAK : nk) - 1) / gr);
    const int64_t kpos0 = (int64_t)j * m;
    const i32x4 kvres = rsrc_i(p.slice[j], (uint32_t)m * (uint32_t)W);
    const uint32_t kcol = (uint32_t)(hq + kvh) * kRowB, vcol = (uint32_t)(hq + p.hkv + kvh) * kRowB;
    // key tile t into stage st: K rows with chunk c at position c ^ (key & 15), V rows with
    // chunk c at c ^ vswz(key)
    auto issue = [&](int t, int st) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const bool isv = i >= kLoads / 2;
        const int piece = wave * (kLoads / 2) + (i % (kLoads / 2));
        const int row = 4 * piece + prow;
        const int gch = isv ? (pch ^ vswz(row)) : (pch ^ (row & 15));
        const uint32_t voff =
            (uint32_t)(t * kAK + row) * (uint32_t)W + (isv ? vcol : kcol) + gch * 16;
        load_lds16(kvres, (uint32_t)uni((int)(lds0 + st * kStage + (isv ? kTileB : 0) + piece * 1024)),
                   voff);
      }
    };
    issue(lo, 0);
    for (int t = lo; t < hi; ++t) {
      const int st = (t - lo) & 1;
      wait_vmcnt<0>();  // tile t has landed (this wave's loads)
      lds_barrier();    // every wave's loads of tile t landed; tile t-1's stage is free
      if (t + 1 < hi) issue(t + 1, st ^ 1);
      const uint8_t* kt = lds + st * kStage;
      const uint8_t* vt = kt + kTileB;

      // S^T = K Q^T for 64 keys (two fragments of 32) x this wave's 32 queries; the two
      // fragments' products alternate, so that consecutive MFMAs never wait on each other
      f32x16 sacc[2];
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[f][v] = 0.f;
      // K fragments one head-dim step ahead of their MFMAs
      auto kfrag = [&](int kd, int f) {
        const int key = 32 * f + l32;
        const int ch = (2 * kd + lh) ^ (key & 15);
        return __builtin_bit_cast(bf16x8, *(const uint4*)(kt + key * kRowB + ch * 16));
      };
      bf16x8 a[2][2];
      a[0][0] = kfrag(0, 0);
      a[0][1] = kfrag(0, 1);
#pragma unroll
      for (int kd = 0; kd < kAD / 16; ++kd) {
        if (kd + 1 < kAD / 16) {
          a[(kd + 1) & 1][0] = kfrag(kd + 1, 0);
          a[(kd + 1) & 1][1] = kfrag(kd + 1, 1);
        }
#pragma unroll
        for (int f = 0; f < 2; ++f)
          sacc[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kd & 1][f], qf[kd], sacc[f], 0, 0, 0);
      }
      // keep that order: the first two steps' reads, then per step its two MFMAs and the next
      // step's two reads (the scheduler would otherwise wait for each step's reads in turn)
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int kd = 0; kd + 1 < kAD / 16; ++kd) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);

      // online softmax in base 2 on the raw scores (the reference max mrow in raw units, the
      // scale folded into the exponent's fma); value v of fragment f is key 32 f + 8 (v / 4) +
      // 4 lh + v % 4. Only a tile that runs past the slice's keys or, under causal masking, past
      // this wave's first query (the diagonal of the own slice) needs the mask (wave-uniform
      // test); masked scores are overwritten in place.
      const int kb = t * kAK;
      const bool full = uni((kb + kAK <= m) &&
                            (!p.causal || j < s || kb + kAK - 1 <= q0 + 32 * wave) ? 1 : 0) != 0;
      if (!full) {
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kj = kb + 32 * f + 8 * (v >> 2) + 4 * lh + (v & 3);
            const bool ok = kj < m && (!p.causal || kpos0 + kj <= qpos);
            if (!ok) sacc[f][v] = kNegBig;
          }
      }
      float mx = kNegBig;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[f][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // A lane moves its reference max only when the tile's max exceeds it by more than
      // kLazyLog2 in the exponent: below that its probabilities are at most 2^kLazyLog2, which
      // fp32 and bf16 hold with their usual relative rounding, and softmax does not depend on
      // the reference (the sum lrow uses the same one). The output rows then need rescaling
      // only when some lane of the wave moved it, which after a query's first keys is rare.
      const float sc = p.scale_log2;
      const bool grow = (mx - mrow) * sc > kLazyLog2;
      const float mnew = grow ? mx : mrow;
      const float alpha = grow ? __builtin_amdgcn_exp2f((mrow - mnew) * sc) : 1.f;
      const float mns = -mnew * sc;
      float psum = 0.f;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          // a masked score (kNegBig) gives exp2 of about -1e29: exactly 0
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[f][v], sc, mns));
          sacc[f][v] = e;
          psum += e;
        }
      lrow = lrow * alpha + psum;
      if (__ballot(grow) != 0) {
#pragma unroll
        for (int i = 0; i < kAD / 32; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) oacc[i][v] *= alpha;
      }
      mrow = mnew;
      // P^T as B operands: 16-key step kk takes values 8 (kk % 2) .. 8 (kk % 2) + 7 of fragment
      // kk / 2, i.e. keys 16 kk + 8 (e / 4) + 4 lh + e % 4 for e = 0..7
      bf16x8 pb[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int f = kk >> 1, b = 8 * (kk & 1);
        uint4 w;
        w.x = cvt_bf16x2(sacc[f][b + 0], sacc[f][b + 1]);
        w.y = cvt_bf16x2(sacc[f][b + 2], sacc[f][b + 3]);
        w.z = cvt_bf16x2(sacc[f][b + 4], sacc[f][b + 5]);
        w.w = cvt_bf16x2(sacc[f][b + 6], sacc[f][b + 7]);
        pb[kk] = __builtin_bit_cast(bf16x8, w);
      }
      // O^T += V^T P^T: A operand row d = 32 i + l32 with the keys of step kk in the same order,
      // from two transpose reads (keys 16 kk + 4 lh + 0..3, then 8 further); per key step the
      // four row blocks' reads are issued together and their MFMAs, on four accumulators, follow
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int kr = 16 * kk + 4 * (g16 >> 1) + (i16 >> 2);
        bf16x8 a[kAD / 32];
#pragma unroll
        for (int i = 0; i < kAD / 32; ++i) {
          const int d = 32 * i + 16 * (g16 & 1) + 4 * (i16 & 3);
          const int off = kr * kRowB + (((d >> 3) ^ vswz(kr)) * 16) + ((d >> 2) & 1) * 8;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + off));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + off + 8 * kRowB));
          const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
          a[i] = __builtin_bit_cast(bf16x8, make_uint4(l2.x, l2.y, h2.x, h2.y));
        }
#pragma unroll
        for (int i = 0; i < kAD / 32; ++i)
          oacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], pb[kk], oacc[i], 0, 0, 0);
      }
    }
    lds_barrier();  // every wave is done with the stages before the next slice refills them
  }

  if (wpart >= 0) {
    // ---- a part of a split item: store this part's output, max and sum; the second part to
    // finish combines the two. The partials are written through to memory and read back with
    // system-coherent loads (sc0 sc1), so neither side needs a cache invalidate.
    constexpr int kSys = 1 | 16;  // cache policy sc0 | sc1
    const int pair = wpart >> 1, part = wpart & 1;
    const uint32_t wbase = (uint32_t)(wave * 66 * 64 + lane) * 4u;
    const __amdgpu_buffer_rsrc_t mine =
        rsrc_b(p.part_buf + ((size_t)pair * 2 + part) * kAttnPartFloats, kAttnPartFloats * 4);
#pragma unroll
    for (int i = 0; i < kAD / 32; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        // through a scalar: a bit cast of the vector element itself reads element 0
        const float x = oacc[i][v];
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, x), mine,
                                              wbase + (uint32_t)((i * 16 + v) * 64 * 4), 0, kSys);
      }
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, mrow), mine, wbase + 64 * 64 * 4, 0,
                                          kSys);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, lrow), mine, wbase + 65 * 64 * 4, 0,
                                          kSys);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();  // every wave's partial is stored
    if (tid == 0)
      *bcast = __hip_atomic_fetch_add(p.pair_cnt + pair, 1u, __ATOMIC_RELEASE,
                                      __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*bcast == 0) return;  // the other part combines (every wave leaves here together)
    if (tid == 0) __hip_atomic_store(p.pair_cnt + pair, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const __amdgpu_buffer_rsrc_t other =
        rsrc_b(p.part_buf + ((size_t)pair * 2 + (part ^ 1)) * kAttnPartFloats, kAttnPartFloats * 4);
    const float om = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(other, wbase + 64 * 64 * 4, 0, kSys));
    const float ol = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(other, wbase + 65 * 64 * 4, 0, kSys));
    // both parts relative to the larger reference max; the sums are formed in part order (part
    // 0's term through the fma), so the result does not depend on which part finished last
    const float mm = fmaxf(mrow, om);
    const float f_own = __builtin_amdgcn_exp2f((mrow - mm) * p.scale_log2);
    const float f_oth = __builtin_amdgcn_exp2f((om - mm) * p.scale_log2);
    lrow = part == 0 ? __builtin_fmaf(lrow, f_own, ol * f_oth) : __builtin_fmaf(ol, f_oth, lrow * f_own);
#pragma unroll
    for (int i = 0; i < kAD / 32; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float ov = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(other, wbase + (uint32_t)((i * 16 + v) * 64 * 4),
                                                        0, kSys));
        oacc[i][v] = part == 0 ? __builtin_fmaf(oacc[i][v], f_own, ov * f_oth)
                               : __builtin_fmaf(ov, f_oth, oacc[i][v] * f_own);
      }
  }

  // ---- epilogue: O = O^T / l, staged per wave as [query][d] bf16, stored row-contiguous -----
  const float ltot = lrow + __shfl_xor(lrow, 32);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  uint8_t* const ost = lds + wave * 32 * kOutStride;
#pragma unroll
  for (int i = 0; i < kAD / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const int d = 32 * i + 8 * (v >> 2) + 4 * lh + (v & 3);
      *(uint32_t*)(ost + l32 * kOutStride + d * 2) = cvt_bf16x2(oacc[i][v] * inv, oacc[i][v + 1] * inv);
    }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging writes are done
  const int ow = hq * kRowB;
  const __amdgpu_buffer_rsrc_t ores =
      rsrc_b((const uint8_t*)p.out + (int64_t)s * m * ow, (uint32_t)m * (uint32_t)ow);
#pragma unroll
  for (int k = 0; k < 32 * kRowB / 16 / 64; ++k) {
    const int c = lane + 64 * k;
    const int row = c >> 4, ch = c & 15;
    const uint4 x = *(const uint4*)(ost + row * kOutStride + ch * 16);
    const uint32_t off = (uint32_t)(q0 + 32 * wave + row) * (uint32_t)ow + h * kRowB + ch * 16;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x), ores, off, 0, 0);
  }
  if (p.rel_tab != nullptr && p.send[s]) {
    // the return exchange: every wave's stores of this item are complete before the barrier;
    // the last item of (slice, row group) then releases the copy of its rows to rank s
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (tid == 0) {
      const int og = (int)p.out_group_rows;
      const int g = q0 / og;
      const int r1 = (g + 1) * og < m ? (g + 1) * og : m;
      const uint32_t items = (uint32_t)(((r1 - g * og + kAQ - 1) / kAQ) * hq);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
      uint32_t* cnt = p.done + s * kMaxGroups + g;
      const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      if (old + 1 == items) {
        __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.rel_tab[s * kMaxGroups + g], (int64_t)0, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
  }
  lds_barrier();  // the next tile's loads overwrite the staging rows
}

__global__ __launch_bounds__(kThreads, 2) void attn_kernel(AttnPlan p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * kStage];
  __shared__ uint32_t bcast;
  release_start(p.start);
  const int qtiles = (int)((p.m + kAQ - 1) / kAQ);
  if (p.table != nullptr) {
    const int u1 = p.bins[blockIdx.x + 1];
    for (int u = p.bins[blockIdx.x]; u < u1; ++u) attn_tile(p, u, lds, &bcast);
    return;
  }
  const int total = p.P * qtiles * p.hq;
  for (int u = blockIdx.x; u < total; u += gridDim.x) attn_tile(p, u, lds, &bcast);
}

}  // namespace

bool attn_plan_ok(const AttnPlan& p) {
  if (p.P < 1 || p.P > FO_MAX_P || p.m < 1 || p.hq < 1 || p.hkv < 1 || p.hq % p.hkv != 0)
    return false;
  if (p.err == nullptr) return false;
  if (p.groups < 1 || p.groups > kMaxGroups || p.group_rows < 1 || p.group_rows % kAQ != 0 ||
      p.group_rows * p.groups < p.m)
    return false;
  const int64_t W = (int64_t)(p.hq + 2 * p.hkv) * kRowB;
  if ((p.m + kAQ) * W >= ((int64_t)1 << 31) || (p.m + kAQ) * p.hq * kRowB >= ((int64_t)1 << 31))
    return false;
  if (p.rel_tab != nullptr &&
      (p.done == nullptr || p.out_groups < 1 || p.out_groups > kMaxGroups ||
       p.out_group_rows < 1 || p.out_group_rows % kAQ != 0 || p.out_group_rows * p.out_groups < p.m))
    return false;
  if (p.table != nullptr && (p.bins == nullptr || p.n_items < 1 || p.n_bins < 1)) return false;
  bool seen[FO_MAX_P] = {};
  for (int i = 0; i < p.P; ++i) {
    if (p.dispatch[i] < 0 || p.dispatch[i] >= p.P || seen[p.dispatch[i]]) return false;
    seen[p.dispatch[i]] = true;
  }
  for (int i = 0; i < p.P; ++i) {
    if (p.order[i] < 0 || p.order[i] >= p.P || p.slice[i] == nullptr) return false;
    if (p.gated[i] && (p.comp_tab == nullptr || p.lead == nullptr || p.ready == nullptr || p.gen == 0))
      return false;
  }
  return true;
}

hipError_t launch_attn(const AttnPlan& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (!attn_plan_ok(p)) return hipErrorInvalidValue;
  const int64_t total =
      p.table != nullptr ? p.n_bins : (int64_t)p.P * ((p.m + kAQ - 1) / kAQ) * p.hq;
  hipExtLaunchKernelGGL(attn_kernel, dim3((unsigned)total), dim3(kThreads), 0, s, e0, e1, 0, p);
  return hipGetLastError();
}

}  // namespace fo
