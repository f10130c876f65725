// Sliced GEMM kernels of libflashovl for gfx950 (MI355X).
//
// One launch computes every slice of a Flash-AG or Flash-RS call (FlashOverlap page, technical
// summary section 2): workgroups are laid out in schedule order, a tile of a slice that is still
// in flight waits on that slice's arrival signal before reading it, and the chunk that stays on
// the rank (Flash-RS) adds the partials received from the peers in its write-back.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 with fp32 accumulation. Each workgroup is 4 waves (2 x 2);
// each wave owns a (BM/2) x (BN/2) block of 32x32 fragments. K advances in steps of 32 through a
// ring of 4 LDS stages that buffer loads fill straight from HBM (the bf16 section below has the
// layout); the accumulators leave through LDS so that output stores and partial loads are
// row-contiguous 16-byte accesses.
//
// fp32 path: a plain LDS-tiled fp32 FMA kernel (exact fp32 products, fp32 sums in k order).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "fo_internal.h"
#include "fo_wait.h"

namespace fo {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kThreads = 256;
constexpr int kBK = 32;  // K step

// ---------------------------------------------------------------- waits and flags -----------

// Wait for group `grp` of `slice` to have landed (the elected poller of fo_wait.h).
__device__ __forceinline__ void wait_group(const Plan& p, int slice, int grp) {
  fo::wait_group(p.comp_tab, p.lead, p.ready, p.gen, p.spin_limit, p.err, slice, grp);
}

// Thread 0 waits for group `grp` of each listed slice (negative ids are skipped); the barrier
// holds the other waves until then, so every load of the group's rows is issued after the copy
// engine's data has landed in memory.
// With p.acq = 0 no cache invalidation follows, because the caches can hold no stale line of
// these rows: the kernel's launch invalidates the L1s and L2s of what earlier kernels (earlier
// calls on the same buffers) cached, inside the launch no workgroup reads a row before its
// transfer has landed, and the host sets p.acq = 0 only when every transfer starts and ends on
// a 128-byte cache-line boundary (so no line holds data of two transfers, or of a transfer and
// another buffer). Otherwise thread 0 acquires at system scope before the barrier. An acquire
// per waiting workgroup invalidates the XCD's L2 under the other tiles: 15-23 us per Flash-AG
// call.
__device__ __forceinline__ void wait_groups_wg(const Plan& p, const int32_t* slices, int n,
                                               int grp) {
  if (threadIdx.x == 0 && p.comp_tab != nullptr) {
    for (int i = 0; i < n; ++i)
      if (slices[i] >= 0) wait_group(p, slices[i], grp);
    if (p.acq) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
  }
  __syncthreads();
}

// After a tile of (position, group) is stored: count it; the last tile of that group stores 0
// into its release signal (polled by the copy engine that carries the matching transfer) and
// re-arms the counter. Every wave first waits for its own stores of the tile (the workgroup
// barrier does not), so that the release below covers the whole tile.
// With the Flash-RS tail, the last tile of a row group of the own chunk also raises
// own_done[group] to the call's number, which the tail workgroups of that group wait for.
__device__ __forceinline__ void release_tile(const Plan& p, int pos, int grp) {
  const bool own = p.tail_units > 0 && pos == p.accum_pos;
  if (p.rel_tab == nullptr && !own) return;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
    uint32_t* cnt = p.done + pos * kMaxGroups + grp;
    const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == (uint32_t)(group_rows_of(p.grid, grp) * p.grid.tiles_n)) {
      __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (p.rel_tab != nullptr)
        __hip_atomic_store(p.rel_tab[pos * kMaxGroups + grp], (int64_t)0, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_SYSTEM);
      if (own)
        __hip_atomic_store(p.own_done + grp, p.gen, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Two fp32 -> bf16 (a in the low half), round to nearest even: one v_cvt_pk_bf16_f32 (CDNA4),
// in the kernel's default float mode (round to nearest even, denormals kept). Five integer
// operations per value instead made the bf16 write-back of a 256x256 tile VALU-bound.
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// fp32 -> bf16, round to nearest, ties to even (quiet NaN kept); branch-free (a select).
__device__ __forceinline__ uint32_t to_bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet = (u >> 16) | 0x40u;
  return (u & 0x7fffffffu) > 0x7f800000u ? quiet : rounded;
}

// ---------------------------------------------------------------- bf16 MFMA kernel ----------
//
// A ring of C::STAGES LDS stages; stage s holds the A tile [BM rows][kBK k] (64-byte rows) and the
// W tile [kBK rows][BN cols] (2*BN-byte rows). Both are filled straight from HBM by buffer loads
// that write LDS (16 bytes per lane, no VGPR staging); a load outside the matrix reads zero
// through the buffer's range check, so ragged edges need no branches. The 16-byte chunks of a
// row are XOR-swizzled by the row index so that the MFMA operand reads spread over the banks.
// A fragments are read with ds_read_b128 (K-contiguous); W fragments with two
// ds_read_b64_tr_b16 transpose reads, which turn 4 rows x 16 columns of the row-major W tile
// into 4 K-values per lane.

constexpr int kLdsBytes = 160 * 1024;  // LDS of one CU
constexpr uint32_t kOOB = 0x80000000u;          // offset past every range: the load reads 0
constexpr int kRsrcWord3 = 0x00020000;          // raw buffer, 32-bit data format

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int BM, int BN>
struct Cfg {
  static constexpr int WTM = BM / 2, WTN = BN / 2;   // wave tile (2 x 2 waves)
  static constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 fragments per wave
  static constexpr int A_BYTES = BM * kBK * 2;        // 64-byte rows
  static constexpr int B_ROW = BN * 2;
  static constexpr int B_BYTES = kBK * B_ROW;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_LOADS = A_BYTES / 1024 / 4;  // 1 KB loads per wave per stage
  static constexpr int B_LOADS = B_BYTES / 1024 / 4;
  static constexpr int LOADS = A_LOADS + B_LOADS;
  // A step's loads go out in two groups, half a step apart (see the pipeline below).
  static constexpr int L0 = LOADS / 2, L1 = LOADS - L0;
  // Four stages: three K steps in flight while one is consumed. Deeper rings (5 for 256x256, 6
  // for 128x256, as many as the LDS holds) measured no faster on MI355X, and 256x256 slower.
  static constexpr int STAGES = 4;
  static constexpr int RING = STAGES * STAGE;
  // Epilogue staging: fp32 rows padded by 8 floats (rows 4 apart land 32 banks apart), in
  // blocks of ER rows; the LDS allocation grows past the ring (up to the CU's LDS) so that the
  // block holds the whole tile, or half of it.
  static constexpr int EW = BN + 8;
  static constexpr int ER = (BM * EW * 4 <= (RING > kLdsBytes ? RING : kLdsBytes)) ? BM
                            : (BM / 2 * EW * 4 <= kLdsBytes)                        ? BM / 2
                                                                                    : BM / 4;
  static constexpr int LDS = RING > ER * EW * 4 ? RING : ER * EW * 4;
  static_assert(LDS <= kLdsBytes, "LDS");
  static_assert(A_LOADS >= 1 && B_LOADS >= 1 && FM >= 1 && FN >= 1 && L0 >= 1, "tile");
  static_assert(STAGES >= 3 && (STAGES - 1) * LOADS < 64, "stages");
  static_assert(ER % 32 == 0 && BM % ER == 0, "epilogue block");
};

// Swizzles of the 16-byte chunks of an LDS row, conflict-free whether the LDS serves 128 bytes
// (32 banks) or 256 bytes (64 banks) per cycle.
// A (64-byte rows, ds_read_b128: 8 or 16 rows at one chunk offset per cycle): the chunk XOR
// ((row >> 1) ^ (row >> 3)) & 3 puts those rows on distinct 16-byte bank groups.
// W (rows of B_ROW bytes, ds_read_b64_tr_b16 of 8 bytes per lane: per cycle 16 lanes = 4 k rows
// x 2 chunks, or 32 lanes = 4 k rows x 4 chunks): a row of 256 or more bytes starts on bank 0,
// so the chunks of row k are XORed with (0, 6, 12, 10)[k & 3], which gives the 4 rows distinct
// bank groups under both widths. The earlier XOR with 2 (k & 3) left rows k and k + 1 on the
// same 32-lane groups: rocprofv3 counted bank-conflict stalls in half of the LDS's busy cycles
// of the 70B gate+up GEMM. 128-byte rows alternate bank halves by themselves and take 2 (k & 3).
__device__ __forceinline__ int swz_a(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }
template <int B_ROW>
__device__ __forceinline__ int swz_b(int krow) {
  return B_ROW >= 256 ? ((0xAC60 >> ((krow & 3) * 4)) & 15) : (krow & 3) << 1;
}

// Values the compiler cannot prove wave-uniform (they come out of VALU integer division) are
// moved to scalar registers explicitly: buffer descriptors must live in SGPRs.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const void* uni_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = (uint32_t)uni((int)(uint32_t)v), hi = (uint32_t)uni((int)(uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;

// Raw buffer descriptor (base, stride 0, num_records bytes, 32-bit data format); every field is
// wave-uniform so it lives in SGPRs.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t v = (uint64_t)uni_ptr(base);
  i32x4 r;
  r.x = uni((int)(uint32_t)v);
  r.y = uni((int)(uint32_t)(v >> 32));  // stride 0
  r.z = uni((int)bytes);
  r.w = kRsrcWord3;
  return r;
}
// The same descriptor in the type the buffer load/store builtins take.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_res(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uni_ptr(base)), (short)0,
                                           (int)uni((int)bytes), kRsrcWord3);
}

// 16 bytes per lane from the buffer at byte offset voff into LDS at base + imm + 16 * lane (an
// offset past num_records reads zeros); imm folds to a constant once the loops are unrolled, so
// a wave keeps one LDS base per operand instead of one per load. Issued as inline assembly so
// that the compiler neither orders later LDS reads behind it nor drains it at barriers:
// completion is tracked by hand with wait_vmcnt, which counts these loads.
__device__ __forceinline__ void load_lds16(i32x4 rsrc, uint32_t base, int imm, uint32_t voff,
                                           uint32_t soff) {
  asm volatile(
      "s_add_u32 m0, %0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds"
      :
      : "s"(base), "i"(imm), "v"(voff), "s"(rsrc), "s"(soff)
      : "m0", "scc");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// The workgroup barrier proper: this wave's LDS accesses are done, no memory fence (vector
// loads and stores in flight stay in flight); the "memory" clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// position of the q-th of n memory instructions among nx issue slots (evenly spread)
__host__ __device__ constexpr int spread_slot(int q, int n, int nx) { return (2 * q + 1) * nx / (2 * n); }

template <int BM, int BN, bool ACT>
__device__ __forceinline__ void bf16_tile(const Plan& p, const int tile, uint8_t* const lds_ring) {
  using C = Cfg<BM, BN>;
  constexpr int S = C::STAGES;
  auto st = [&](int i) -> uint8_t* { return lds_ring + i * C::STAGE; };
  auto lds_addr = [](const uint8_t* q) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)q;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform (scalar) so that the LDS destination of the LDS-writing loads is uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  int pos_, grp_, tm_, tn_;
  locate(p.grid, tile, pos_, grp_, tm_, tn_);
  const int pos = uni(pos_), grp = uni(grp_), tm = uni(tm_), tn = uni(tn_);

  const int64_t K = p.K, N = p.N;
  // With the SwiGLU epilogue (act) the tile's first BN/2 columns are gate columns and its last
  // BN/2 the up columns of the same hidden units (W columns inter + ...); it writes BN/2
  // columns of h = silu(gate) * up. col0 is the tile's first output column.
  constexpr bool act = ACT;
  const int64_t inter = N / 2;
  const int64_t row0 = (int64_t)tm * BM;
  const int64_t col0 = (int64_t)tn * (act ? BN / 2 : BN);
  const int64_t rows_valid = p.m - row0;  // >= 1
  const int a_rows = uni((int)(rows_valid < BM ? rows_valid : BM));
  // A slice is row-major [m, K] (chunks = 1) or K-chunk-major: `chunks` blocks [m, Kc] one
  // after another. A points at the tile's first row in block 0; element (row, k) of the tile is
  // at A + row * Kc + (k - j * Kc) + j * m * Kc for block j = k / Kc.
  const int chunks = uni(p.chunks);
  const int64_t Kc = chunks > 1 ? K / chunks : K;
  const int64_t chunk_extra = (p.m - 1) * Kc;  // block j starts j * chunk_extra past k = j * Kc
  const uint32_t chunk_magic = (uint32_t)uni((int)p.chunk_magic);
  const uint16_t* A = (const uint16_t*)uni_ptr((const uint16_t*)p.a_pos[pos] + row0 * Kc);
  const uint16_t* W = (const uint16_t*)uni_ptr(p.b);

  // Flash-AG: rows of a received slice are read only after their group (its first K block when
  // the slice travels in K blocks) has landed.
  const int gslice = uni(p.gate_slice[pos]);
  if (gslice >= 0) wait_groups_wg(p, p.gate_slice + pos, 1, grp * chunks);

  // ---- loads. Per-lane offsets are fixed for the whole K loop: the K step enters A's loads as
  // the scalar offset and W's through a descriptor re-based on the step's first row (whose
  // num_records also cuts off rows past K). Lanes outside the tile carry kOOB and read zeros.
  const i32x4 rsrc_a = buffer_rsrc(A, (uint32_t)(((chunks - 1) * p.m * Kc + a_rows * Kc) * 2));
  const uint32_t lds0 = lds_addr(lds_ring);
  const uint32_t a_base = (uint32_t)uni((int)(lds0 + wave * C::A_LOADS * 1024));
  const uint32_t b_base = (uint32_t)uni((int)(lds0 + C::A_BYTES + wave * C::B_LOADS * 1024));
  uint32_t a_voff[C::A_LOADS];
  int a_kel[C::A_LOADS];
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const int row = (wave * C::A_LOADS + j) * 16 + (lane >> 2);
    a_kel[j] = ((lane & 3) ^ swz_a(row)) * 8;
    a_voff[j] = row < a_rows ? (uint32_t)(((int64_t)row * Kc + a_kel[j]) * 2) : kOOB;
  }
  uint32_t b_voff[C::B_LOADS];
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j) {
    const int P = (wave * C::B_LOADS + j) * 1024 + lane * 16;
    const int kr = P / C::B_ROW;
    const int n = ((((P % C::B_ROW) >> 4) ^ swz_b<C::B_ROW>(kr))) * 8;
    int64_t wc;  // W column of tile column n
    bool ok;
    if constexpr (act) {
      const int half = n >= BN / 2 ? 1 : 0;
      const int64_t c = col0 + n - half * (BN / 2);
      ok = c < inter;
      wc = c + half * inter;
    } else {
      wc = col0 + n;
      ok = wc < N;
    }
    b_voff[j] = ok ? (uint32_t)(((int64_t)kr * N + wc) * 2) : kOOB;
  }

  // load number l (A loads first, then W loads) of K step kt into stage si (0..S-1); rb is W's
  // descriptor for that step (from w_rsrc). TAIL: the step runs past K, so A columns beyond K
  // are redirected to kOOB (W rows beyond K fall outside rb's range by themselves).
  auto w_rsrc = [&](int kt) {
    const int64_t k0 = (int64_t)kt * kBK;
    const int64_t rows = K - k0 < kBK ? K - k0 : kBK;
    return buffer_rsrc(W + k0 * N, (uint32_t)(rows * N * 2));
  };
  auto issue_one = [&](auto tail, int kt, int si, const i32x4& rb, int l) {
    const int64_t k0 = (int64_t)kt * kBK;
    if (l < C::A_LOADS) {
      uint32_t v = a_voff[l];
      if constexpr (decltype(tail)::value) {
        if (k0 + a_kel[l] >= K) v = kOOB;
      }
      // K block of this step (0 when row-major: chunk_magic = 0)
      const uint32_t blk =
          (uint32_t)__builtin_amdgcn_readfirstlane((int)__umulhi((uint32_t)kt, chunk_magic));
      load_lds16(rsrc_a, a_base, si * C::STAGE + l * 1024, v,
                 (uint32_t)((k0 + (int64_t)blk * chunk_extra) * 2));
    } else {
      const int j = l - C::A_LOADS;
      load_lds16(rb, b_base, si * C::STAGE + j * 1024, b_voff[j], 0u);
    }
  };
  // loads [l0, l1) of step kt into stage si
  auto issue_range = [&](int kt, int si, int l0, int l1) {
    const i32x4 rb = w_rsrc(kt);
    if ((int64_t)(kt + 1) * kBK > K) {
#pragma unroll
      for (int l = 0; l < C::LOADS; ++l)
        if (l >= l0 && l < l1) issue_one(std::true_type{}, kt, si, rb, l);
    } else {
#pragma unroll
      for (int l = 0; l < C::LOADS; ++l)
        if (l >= l0 && l < l1) issue_one(std::false_type{}, kt, si, rb, l);
    }
  };

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int lr = lane & 31, lh = lane >> 5;
  const int g16 = lane >> 4, i16 = lane & 15;

  struct Frags {
    bf16x8 a[C::FM], b[C::FN];
  };
  // fragment i of A / j of W for K-substep kk (16 values of k) of a stage
  auto rd_a = [&](const uint8_t* stage, int kk, int i) {
    const int r = wm * C::WTM + i * 32 + lr;
    const int c = 2 * kk + lh;
    return __builtin_bit_cast(bf16x8, *(const uint4*)(stage + r * 64 + ((c ^ swz_a(r)) << 4)));
  };
  auto rd_b = [&](const uint8_t* stage, int kk, int j) {
    const uint8_t* sb = stage + C::A_BYTES;
    const int kr = 16 * kk + 8 * (g16 >> 1) + (i16 >> 2);
    const int n = wn * C::WTN + j * 32 + 16 * (g16 & 1) + 4 * (i16 & 3);
    const int off = ((n >> 3) ^ swz_b<C::B_ROW>(kr)) * 16 + ((n >> 2) & 1) * 8;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sb + kr * C::B_ROW + off));
    const s16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sb + (kr + 4) * C::B_ROW + off));
    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(bf16x8, make_uint4(l2.x, l2.y, h2.x, h2.y));
  };
  // fragment read number q of a Frags set (A fragments first)
  auto rd_frag = [&](const uint8_t* stage, int kk, Frags& f, int q) {
    if (q < C::FM)
      f.a[q] = rd_a(stage, kk, q);
    else
      f.b[q - C::FM] = rd_b(stage, kk, q - C::FM);
  };
  auto mfma = [&](const Frags& f, int idx) {
    const int i = idx / C::FN, j = idx % C::FN;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };
  // this wave's loads of the oldest pending stage have landed when at most n later stages'
  // loads are still in flight
  auto wait_stages = [&](int n) {
    switch (n) {
      case 7: wait_vmcnt<(7 < S ? 7 : 0) * C::LOADS>(); break;
      case 6: wait_vmcnt<(6 < S ? 6 : 0) * C::LOADS>(); break;
      case 5: wait_vmcnt<(5 < S ? 5 : 0) * C::LOADS>(); break;
      case 4: wait_vmcnt<(4 < S ? 4 : 0) * C::LOADS>(); break;
      case 3: wait_vmcnt<(3 < S ? 3 : 0) * C::LOADS>(); break;
      case 2: wait_vmcnt<2 * C::LOADS>(); break;
      case 1: wait_vmcnt<C::LOADS>(); break;
      default: wait_vmcnt<0>(); break;
    }
  };

  constexpr int NMFMA = C::FM * C::FN, NREAD = C::FM + C::FN;
  // Software pipeline over K steps of kBK; stage kt % S holds step kt. A step runs its MFMAs in
  // two halves (K-substeps 0 and 1). The first half's fragments are already in registers; while
  // its MFMAs issue, the second half's fragments are read. Then, once every wave holds the next
  // stage and nobody reads this one any more (barrier), the second half's MFMAs issue
  // interleaved with the reads of the next step's first-half fragments.
  // The stage freed at a barrier is refilled with the step S ahead in two groups of loads: the
  // first group during the second half that follows the barrier, the second during the next
  // step's first half. Spreading them over the whole step keeps the address unit busy evenly
  // instead of in one burst after each barrier (a burst stalls the issuing waves). The count of
  // loads issued after any given step is unchanged, so the waits are the same as with one group.
  // The order inside each half is pinned with scheduling barriers so that memory instructions
  // issue under running MFMAs.
  const int KT = uni((int)((K + kBK - 1) / kBK));
  const int KFULL = uni((int)(K / kBK));  // steps that lie entirely inside K
  Frags f0, f1;
  if (KT > 0) {
#pragma unroll
    for (int i = 0; i < S - 1; ++i)
      if (i < KT) issue_range(i, i, 0, C::LOADS);
    if (S - 1 < KT) issue_range(S - 1, S - 1, 0, C::L0);
    // step 0 landed: at most the later steps' loads still in flight (rounded down to whole steps)
    wait_stages(KT - 1 < S - 2 ? KT - 1 : S - 2);
    lds_barrier();
#pragma unroll
    for (int q = 0; q < NREAD; ++q) rd_frag(st(0), 0, f0, q);
  }
  constexpr int NX1 = NMFMA > NREAD ? NMFMA : NREAD;
  constexpr int NX1L = NMFMA > C::L1 ? NMFMA : C::L1;
  constexpr int NX2L = NMFMA > C::L0 ? NMFMA : C::L0;
  constexpr int NXA = NX1 > NX1L ? NX1 : NX1L;
  constexpr int NXB = NX1 > NX2L ? NX1 : NX2L;
  // load l of step kt into stage si, with the K-tail check when `tail` (branches around single
  // load instructions only, so that the MFMA sequence is not duplicated)
  auto issue_if = [&](bool issue, bool tail, int kt, int si, const i32x4& rb, int l) {
    if (issue) {
      if (tail)
        issue_one(std::true_type{}, kt, si, rb, l);
      else
        issue_one(std::false_type{}, kt, si, rb, l);
    }
  };
  // first half of step kt (stage si): MFMAs of f0 with the reads of f1 and, when `issue`, the
  // second load group of step `late` into the stage freed at the previous barrier
  // (The descriptor of a load group is computed under the first MFMA of its half, not ahead of
  // it, so that its scalar arithmetic does not hold back the MFMA that follows a barrier.)
  auto first_half = [&](int si, int late, bool issue, bool tail) {
    i32x4 rb{};
    const int ls = (si + S - 1) % S;
#pragma unroll
    for (int x = 0; x < NXA; ++x) {
      if (x < NMFMA) mfma(f0, x);
      if (x == 0 && issue) rb = w_rsrc(late);
      if (x < NREAD) rd_frag(st(si), 1, f1, x);
#pragma unroll
      for (int q = 0; q < C::L1; ++q)
        if (x == spread_slot(q, C::L1, NX1L)) issue_if(issue, tail, late, ls, rb, C::L0 + q);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // second half of step kt: MFMAs of f1, the first load group of step kt + S into stage si when
  // `issue`, and the reads of the next step's f0 when `more`
  auto second_half = [&](int kt, int si, bool issue, bool tail, bool more) {
    i32x4 rb{};
#pragma unroll
    for (int x = 0; x < NXB; ++x) {
      if (x < NMFMA) mfma(f1, x);
      if (x == 0 && issue) rb = w_rsrc(kt + S);
#pragma unroll
      for (int q = 0; q < C::L0; ++q)
        if (x == spread_slot(q, C::L0, NX2L)) issue_if(issue, tail, kt + S, si, rb, q);
      if (x < NREAD && more) rd_frag(st((si + 1) % S), 0, f0, x);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // A received slice that travels in K blocks: the first loads of block j (step j * spc) are
  // issued after the barrier of step j * spc - S, so before that barrier thread 0 waits for
  // block j of the tile's row group to have landed (acquiring only with p.acq, as at the wait
  // at the start); the barrier holds the other waves until then. gate_kt = -1: nothing left.
  const int spc = (int)(Kc / kBK);
  int gate_kt = (gslice >= 0 && chunks > 1) ? spc - S : -1;
  int gate_j = 1;
  auto chunk_gate = [&](int kt) {
    if (kt == gate_kt) {
      if (tid == 0) {
        wait_group(p, gslice, grp * chunks + gate_j);
        if (p.acq) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
      }
      ++gate_j;
      gate_kt = gate_j < chunks ? gate_kt + spc : -1;
    }
  };
  // Steady-state step: every step it loads lies entirely inside K.
  auto step_main = [&](int kt, int si) {
    first_half(si, kt + S - 1, true, false);
    wait_stages(S - 2);
    chunk_gate(kt);
    lds_barrier();
    second_half(kt, si, true, false, true);
  };
  // Any step (start-up, last steps, K tail), with the conditions checked at run time.
  auto step_any = [&](int kt, int si) {
    const int late = kt + S - 1;
    first_half(si, late, late < KT, late >= KFULL);
    const int later = KT - 2 - kt;  // steps issued beyond kt + 1 (at most S - 2 at this point)
    wait_stages(later < 0 ? 0 : (later > S - 2 ? S - 2 : later));
    chunk_gate(kt);
    lds_barrier();
    second_half(kt, si, kt + S < KT, kt + S >= KFULL, kt + 1 < KT);
  };
  int kt = 0;
  for (; kt + 2 * S <= KFULL; kt += S) {
#pragma unroll
    for (int i = 0; i < S; ++i) step_main(kt + i, i);
  }
  for (; kt < KT; kt += S) {
#pragma unroll
    for (int i = 0; i < S; ++i)
      if (kt + i < KT) step_any(kt + i, i);
  }

  // ---- epilogue ---------------------------------------------------------------------------
  // The accumulators go through LDS (free now) in blocks of ER rows so that every global access
  // is a row-contiguous 16-byte (fp32) or 8-byte (bf16) vector: output stores, and for the chunk
  // that stays on the rank, the loads of the received partials, which are all issued before any
  // of them is added (the adds keep the arrival order). Stores go through a buffer descriptor
  // that covers the tile's valid rows, so rows past the slice are dropped by the range check;
  // columns past N get an offset outside every range. Nothing waits for the stores here: the
  // next tile's loads overlap them (release_tile waits for them where a copy engine reads them).
  // the own chunk adds its partials here, unless the tail workgroups do (tail_units > 0)
  const bool accum = (pos == p.accum_pos) && p.tail_units == 0;
  if (accum) wait_groups_wg(p, p.recv_slice, p.n_recv, grp);
  lds_barrier();  // LDS stages no longer read
  float* const ep = (float*)lds_ring;  // [ER rows][EW floats]
  constexpr int ER = C::ER, EW = C::EW;
  constexpr int CPR = BN / 4;                   // 4-float chunks per row
  constexpr int CPT = ER * CPR / kThreads;      // chunks per thread per block
  static_assert(CPT >= 1 && (ER * CPR) % kThreads == 0, "epilogue chunks");
  constexpr int BATCH = CPT < 4 ? CPT : 4;      // chunks whose partial loads are in flight together
  const int esz = p.out_f32 ? 4 : 2;
  const uint32_t nn = (uint32_t)N;
  const int64_t n_out = act ? inter : N;  // output row stride
  const __amdgpu_buffer_rsrc_t out_res =
      buffer_res((const uint8_t*)p.c_pos[pos] + row0 * n_out * esz, (uint32_t)(a_rows * n_out * esz));
  // Chunk b of this thread in a block is chunk b * kThreads + tid: row b * (kThreads / CPR) +
  // tid / CPR, the same 4 columns for every b. Its element offset is e0 + b * e_step (e0 for the
  // block's first row); a thread whose columns lie past N stores nowhere (kOOB).
  static_assert(kThreads % CPR == 0, "epilogue rows");
  constexpr int RPB = kThreads / CPR;  // rows covered by one chunk of every thread
  const uint32_t gcol = (uint32_t)col0 + (tid % CPR) * 4;
  const bool col_ok = gcol < nn;
  const uint32_t e_step = (uint32_t)RPB * nn;
  // Per-lane LDS offsets of the staging rows, re-derived in each block behind an empty asm:
  // otherwise the compiler precomputes one address per chunk at kernel start, spills them, and
  // the reloads in the store loop wait for every store in flight.
  int ep_rd = 0, ep_wr = 0;
  auto chunk_lds = [&](int b) -> float4 { return *(const float4*)(ep + ep_rd + b * RPB * EW); };
#pragma unroll
  for (int blk = 0; blk < BM / ER; ++blk) {
    ep_rd = (tid / CPR) * EW + (tid % CPR) * 4;
    ep_wr = 4 * lh * EW + wn * C::WTN + lr;
    asm volatile("" : "+v"(ep_rd), "+v"(ep_wr));
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const int fr = wm * C::WTM + i * 32;  // first tile row of fragment row i
      if (fr < blk * ER || fr >= (blk + 1) * ER) continue;
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = fr - blk * ER + 8 * (v >> 2) + (v & 3);
          ep[ep_wr + r * EW + j * 32] = acc[i][j][v];
        }
        // one fragment at a time: the accumulators stay in place until written (no spills)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    lds_barrier();
    if constexpr (act) {
      // h = silu(gate) * up: gate in staging columns [0, BN/2), up in [BN/2, BN); BN/2 output
      // columns of h (row stride inter), 4 per chunk
      constexpr int CPRA = BN / 8, RPBA = kThreads / CPRA, CPTA = ER * CPRA / kThreads;
      static_assert(kThreads % CPRA == 0 && CPTA >= 1 && (ER * CPRA) % kThreads == 0, "act chunks");
      const uint32_t gca = (uint32_t)col0 + (tid % CPRA) * 4;
      const bool oka = gca < (uint32_t)inter;
      // the block's byte offset, behind an empty asm like the LDS offsets (else the compiler
      // precomputes every chunk's offset at kernel start and spills them)
      uint32_t va = ((uint32_t)(blk * ER + tid / CPRA) * (uint32_t)inter + gca) * 2;
      int ep_a = (tid / CPRA) * EW + (tid % CPRA) * 4;
      asm volatile("" : "+v"(ep_a), "+v"(va));
      const uint32_t va_step = (uint32_t)RPBA * (uint32_t)inter * 2;
#pragma unroll
      for (int b = 0; b < CPTA; ++b) {
        const float4 g = *(const float4*)(ep + ep_a + b * RPBA * EW);
        const float4 u = *(const float4*)(ep + ep_a + b * RPBA * EW + BN / 2);
        const uint32_t lo = cvt_bf16x2(silu_mul(g.x, u.x), silu_mul(g.y, u.y));
        const uint32_t hi = cvt_bf16x2(silu_mul(g.z, u.z), silu_mul(g.w, u.w));
        const uint32_t off = oka ? va + (uint32_t)b * va_step : kOOB;
        __builtin_amdgcn_raw_buffer_store_b64(i32x2{(int)lo, (int)hi}, out_res, off, 0, 0);
        if (b % 4 == 3) __builtin_amdgcn_sched_barrier(0);
      }
      lds_barrier();
      continue;
    }
    const uint32_t e0 = (uint32_t)(blk * ER + tid / CPR) * nn + gcol;
    auto chunk_off = [&](int b, int scale) -> uint32_t {
      return col_ok ? (e0 + b * e_step) * scale : kOOB;
    };
    if (!accum) {
      if (p.out_f32 && p.rel_tab != nullptr) {
        // a chunk a copy engine sends once released: stores coherent at system scope (sc0 sc1)
        // leave less for the release's L2 write-back (Flash-RS in lockstep: 417 -> 413 us)
#pragma unroll
        for (int b = 0; b < CPT; ++b) {
          const float4 x = chunk_lds(b);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x), out_res,
                                                 chunk_off(b, 4), 0, 1 | 16);
          if (b % 4 == 3) __builtin_amdgcn_sched_barrier(0);
        }
      } else if (p.out_f32) {
#pragma unroll
        for (int b = 0; b < CPT; ++b) {
          const float4 x = chunk_lds(b);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x), out_res,
                                                 chunk_off(b, 4), 0, 0);
          if (b % 4 == 3) __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int b = 0; b < CPT; ++b) {
          const float4 x = chunk_lds(b);
          const uint32_t lo = cvt_bf16x2(x.x, x.y), hi = cvt_bf16x2(x.z, x.w);
          __builtin_amdgcn_raw_buffer_store_b64(i32x2{(int)lo, (int)hi}, out_res, chunk_off(b, 2),
                                                0, 0);
          if (b % 4 == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
      // the own chunk of Flash-RS (fp32 output): partial q at the same element offset in
      // recv[q] + row0 * N
#pragma unroll
      for (int b0 = 0; b0 < CPT; b0 += BATCH) {
        float4 x[BATCH];
#pragma unroll
        for (int b = 0; b < BATCH; ++b) x[b] = chunk_lds(b0 + b);
        for (int q0 = 0; q0 < p.n_recv; q0 += 4) {
          float4 t[4][BATCH];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (q0 + q < p.n_recv) {
              const __amdgpu_buffer_rsrc_t rr =
                  buffer_res(p.recv[q0 + q] + row0 * N, (uint32_t)a_rows * nn * 4);
#pragma unroll
              for (int b = 0; b < BATCH; ++b)  // streaming: the partials are read once
                t[q][b] = __builtin_bit_cast(
                    float4, __builtin_amdgcn_raw_buffer_load_b128(rr, chunk_off(b0 + b, 4), 0, 2));
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (q0 + q >= p.n_recv) break;
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
              x[b].x += t[q][b].x;
              x[b].y += t[q][b].y;
              x[b].z += t[q][b].z;
              x[b].w += t[q][b].w;
            }
          }
        }
#pragma unroll
        for (int b = 0; b < BATCH; ++b)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x[b]), out_res,
                                                 chunk_off(b0 + b, 4), 0, 0);
      }
    }
    lds_barrier();  // the next block, or the next tile's loads, overwrite the staging rows
  }
  release_tile(p, pos, grp);
}

// The call's copies wait for its start signal (fo_wait.h).
__device__ __forceinline__ void release_start(const Plan& p) { fo::release_start(p.start); }

// Flash-RS tail unit u: piece u % tail_per_group of row group g = u / tail_per_group of the own
// chunk. Once the group's tiles have stored their fp32 sums (own_done) and the group's partials
// have landed, out += recv[0], then recv[1], ... for each element, the fused epilogue's order,
// so the result is the same bit for bit. The last group's partials land together at the end of
// the call; spread over these workgroups their adds take a few microseconds instead of running
// through the group's own tiles alone. 16-byte pieces throughout (the host checks alignment).
__device__ __forceinline__ void rs_tail_unit(const Plan& p, int u) {
  const int g = u / p.tail_per_group, k = u % p.tail_per_group;
  const int64_t r0 = (int64_t)g * p.grid.group_rows * p.tail_bm;
  const int64_t r1 = (int64_t)(g + 1) * p.grid.group_rows * p.tail_bm < p.m
                         ? (int64_t)(g + 1) * p.grid.group_rows * p.tail_bm : p.m;
  if (r0 >= r1) return;
  if (threadIdx.x == 0) {
    wait_gen(p.own_done + g, p.gen, p.spin_limit, p.err);
    if (p.comp_tab != nullptr)
      for (int i = 0; i < p.n_recv; ++i)
        if (p.recv_slice[i] >= 0) wait_group(p, p.recv_slice[i], g);
  }
  __syncthreads();
  // No acquire fence: out and the partials are read with system-coherent loads (sc0 sc1), which
  // return what the other workgroups' released stores and the copy engines put in memory
  // whatever this CU's caches hold. (A system-scope acquire invalidates the L2 in every one of
  // these workgroups; the last group's invalidates serialized into a tail of tens of us.)
  constexpr int kSys = 1 | 16;  // cache policy sc0 | sc1
  const int64_t N = p.N;
  const int64_t e4 = (r1 - r0) * N / 4;  // 16-byte pieces of the group
  const int64_t lo = e4 * k / p.tail_per_group, hi = e4 * (k + 1) / p.tail_per_group;
  const uint32_t bytes = (uint32_t)((r1 - r0) * N * 4);
  const __amdgpu_buffer_rsrc_t out_r = buffer_res((float*)p.c_pos[p.accum_pos] + r0 * N, bytes);
  // two pieces per thread per pass; pieces past hi get an offset outside the range (kOOB): their
  // loads read zeros and their stores are dropped
  constexpr int TB = 2;
  for (int64_t j0 = lo + threadIdx.x; j0 < hi; j0 += TB * kThreads) {
    uint32_t off[TB];
    float4 x[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      const int64_t j = j0 + b * kThreads;
      off[b] = j < hi ? (uint32_t)(j * 16) : kOOB;
      x[b] = __builtin_bit_cast(float4,
                                __builtin_amdgcn_raw_buffer_load_b128(out_r, off[b], 0, kSys));
    }
    for (int q0 = 0; q0 < p.n_recv; q0 += 4) {  // four partials' loads in flight, then their adds
      float4 t[4][TB];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q0 + q < p.n_recv) {
          const __amdgpu_buffer_rsrc_t rr = buffer_res(p.recv[q0 + q] + r0 * N, bytes);
#pragma unroll
          for (int b = 0; b < TB; ++b)  // streaming (nt): the partials are read once
            t[q][b] = __builtin_bit_cast(
                float4, __builtin_amdgcn_raw_buffer_load_b128(rr, off[b], 0, kSys | 2));
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q0 + q >= p.n_recv) break;
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          x[b].x += t[q][b].x;
          x[b].y += t[q][b].y;
          x[b].z += t[q][b].z;
          x[b].w += t[q][b].w;
        }
      }
    }
#pragma unroll
    for (int b = 0; b < TB; ++b)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x[b]), out_r, off[b], 0, 0);
  }
}

// One workgroup per tile, or (grid smaller than the tile count) a persistent grid whose
// workgroups walk the tiles with a stride of the grid size, in the same order. With the Flash-RS
// tail, tail_units more workgroups follow the tiles.
template <int BM, int BN, bool ACT>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(Plan p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_ring[Cfg<BM, BN>::LDS];
  release_start(p);
  const int total = p.grid.npos * p.grid.tiles_m * p.grid.tiles_n;
  if ((int)blockIdx.x >= total) {
    rs_tail_unit(p, (int)blockIdx.x - total);
    return;
  }
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x)
    bf16_tile<BM, BN, ACT>(p, tile, lds_ring);
}

// ---------------------------------------------------------------- fp32 kernel ----------------

constexpr int F_BM = 64, F_BN = 64, F_BK = 16;

__device__ __forceinline__ void f32_tile(const Plan& p, const int tile, float (*sa)[F_BM + 4],
                                         float (*sb)[F_BN + 4]) {
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;

  int pos, grp, tm, tn;
  locate(p.grid, tile, pos, grp, tm, tn);
  const int64_t K = p.K, N = p.N;
  const int64_t row0 = (int64_t)tm * F_BM, col0 = (int64_t)tn * F_BN;
  const int64_t rows_valid = p.m - row0;
  const float* A = (const float*)p.a_pos[pos] + row0 * K;
  const float* B = (const float*)p.b + col0;

  if (p.gate_slice[pos] >= 0) wait_groups_wg(p, p.gate_slice + pos, 1, grp);

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int64_t k0 = 0; k0 < K; k0 += F_BK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // A tile: 64 rows x 16 k, B tile: 16 k x 64 cols
      const int idx = tid + q * kThreads;
      const int ar = idx / F_BK, ak = idx % F_BK;
      sa[ak][ar] = (ar < rows_valid && k0 + ak < K) ? A[(int64_t)ar * K + k0 + ak] : 0.f;
      const int bk = idx / F_BN, bn = idx % F_BN;
      sb[bk][bn] = (k0 + bk < K && col0 + bn < N) ? B[(k0 + bk) * N + bn] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < F_BK; ++k) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(sa[k][ty + 16 * i], sb[k][tx + 16 * j], acc[i][j]);
    }
    __syncthreads();
  }

  // the own chunk adds its partials here, unless the tail workgroups do (tail_units > 0)
  const bool accum = (pos == p.accum_pos) && p.tail_units == 0;
  if (accum) wait_groups_wg(p, p.recv_slice, p.n_recv, grp);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t r = ty + 16 * i, col = col0 + tx + 16 * j;
      if (r >= rows_valid || col >= N) continue;
      const int64_t off = (row0 + r) * N + col;
      float x = acc[i][j];
      if (accum)
        for (int q = 0; q < p.n_recv; ++q) x += p.recv[q][off];
      if (p.out_f32)
        ((float*)p.c_pos[pos])[off] = x;
      else
        ((uint16_t*)p.c_pos[pos])[off] = to_bf16_rne(x);
    }
  }
  release_tile(p, pos, grp);
}

__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(Plan p) {
  release_start(p);
  __shared__ float sa[F_BK][F_BM + 4];  // k-major so a thread's 4 rows are one broadcast read
  __shared__ float sb[F_BK][F_BN + 4];
  const int total = p.grid.npos * p.grid.tiles_m * p.grid.tiles_n;
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    f32_tile(p, tile, sa, sb);
    __syncthreads();  // the next tile refills sa / sb
  }
}

// e0 / e1 (may be null): events that take the kernel's own start and end times from its
// dispatch (hipExtLaunchKernel), with no marker packets around it on the stream
template <int BM, int BN>
hipError_t launch_bf16(const Plan& p, int64_t grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (p.act)
    hipExtLaunchKernelGGL((gemm_bf16_kernel<BM, BN, true>), dim3((unsigned)grid), dim3(kThreads),
                          0, s, e0, e1, 0, p);
  else
    hipExtLaunchKernelGGL((gemm_bf16_kernel<BM, BN, false>), dim3((unsigned)grid), dim3(kThreads),
                          0, s, e0, e1, 0, p);
  return hipGetLastError();
}

// Releases the copies that depend on a call's start signal: everything enqueued earlier on the
// stream is complete and, after the system-scope release, visible to the copy engines.
__global__ __launch_bounds__(64) void release_kernel(int64_t* v) {
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
    __hip_atomic_store(v, (int64_t)0, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

struct SliceList {
  int32_t s[FO_MAX_P];
  int32_t n, groups;
};

// Waits until every group of every listed slice has landed (the transfers alone, without a GEMM).
__global__ __launch_bounds__(64) void wait_kernel(const int64_t* const* comp_tab, SliceList l,
                                                  uint64_t limit, uint32_t* err, uint32_t gen) {
  if (threadIdx.x == 0)
    for (int i = 0; i < l.n; ++i)
      for (int g = 0; g < l.groups; ++g)
        wait_signal(comp_tab[l.s[i] * kMaxGroups + g], limit, err, gen);
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
}

typedef __attribute__((ext_vector_type(4))) float v4f;

// Loads that are coherent at system scope (sc0 sc1): they return what the copy engines wrote to
// memory whatever the L1 and L2 of this CU hold, so the reader needs no cache invalidation. Their
// completion is awaited with an explicit s_waitcnt (wait_loads) before the values are used.
__device__ __forceinline__ v4f ld_sys4(const float* p) {
  v4f v;
  asm volatile("global_load_dwordx4 %0, %1, off sc0 sc1" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ float ld_sys1(const float* p) {
  float v;
  asm volatile("global_load_dword %0, %1, off sc0 sc1" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Bounded wait of call `gen` until a device word holds `v` (or a wait of the call has failed).
__device__ __forceinline__ void wait_word(const uint32_t* w, uint32_t v, uint64_t limit,
                                          uint32_t* err, uint32_t gen) {
  const uint64_t t0 = wall_clock64();
  while (__hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != v) {
    if (wait_failed(err, gen)) return;
    if (wall_clock64() - t0 > limit) {
      wait_fail(err, 1u, gen);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// out += the received partials, in arrival order (the tail of Flash-RS in the data-slicing
// order). HBM-bound: one pass over out and each partial, 16-byte accesses when aligned. The grid
// is persistent (about two blocks per CU, all resident at once). Only block 0 polls the arrival
// signals (host memory: hundreds of pollers would slow the copy engines); it then sets a device
// word the other blocks wait on. The partials are read with system-coherent loads, so no block
// needs a cache invalidation (a system-scope acquire in every block costs more than the pass).
__global__ __launch_bounds__(256) void reduce_kernel(ReduceArgs a) {
  if (threadIdx.x == 0 && a.comp_tab != nullptr) {
    if (blockIdx.x == 0) {
      for (int i = 0; i < a.n_recv; ++i)
        if (a.recv_slice[i] >= 0)
          for (int g = 0; g < a.groups; ++g)
            wait_signal(a.comp_tab[a.recv_slice[i] * kMaxGroups + g], a.spin_limit, a.err, a.gen);
      __hip_atomic_store(a.go, a.go_value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    } else {
      wait_word(a.go, a.go_value, a.spin_limit, a.err, a.gen);
    }
  }
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  constexpr int B = 8;  // partials whose loads are in flight together
  if (a.vec4) {
    v4f* o = (v4f*)a.out;
    for (int64_t i = first; i < a.count / 4; i += stride) {
      v4f x = o[i];
      for (int q0 = 0; q0 < a.n_recv; q0 += B) {
        v4f t[B];
#pragma unroll
        for (int j = 0; j < B; ++j)
          if (q0 + j < a.n_recv) t[j] = ld_sys4(a.recv[q0 + j] + 4 * i);
        wait_loads();
#pragma unroll
        for (int j = 0; j < B; ++j)
          if (q0 + j < a.n_recv) x += t[j];
      }
      o[i] = x;
    }
  } else {
    for (int64_t i = first; i < a.count; i += stride) {
      float x = a.out[i];
      for (int q0 = 0; q0 < a.n_recv; q0 += B) {
        float t[B];
#pragma unroll
        for (int j = 0; j < B; ++j)
          if (q0 + j < a.n_recv) t[j] = ld_sys1(a.recv[q0 + j] + i);
        wait_loads();
#pragma unroll
        for (int j = 0; j < B; ++j)
          if (q0 + j < a.n_recv) x += t[j];
      }
      a.out[i] = x;
    }
  }
}

// Zeroes `words` 32-bit words with vector stores (a kernel, not hipMemsetAsync, so that a caller
// may capture it in a HIP graph).
__global__ __launch_bounds__(256) void zero_kernel(uint32_t* p, int words) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < words; i += gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace

hipError_t launch_zero(uint32_t* p, int words, hipStream_t s) {
  if (p == nullptr || words < 0) return hipErrorInvalidValue;
  if (words == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)std::min(64, (words + 255) / 256)), dim3(256), 0,
                     s, p, words);
  return hipGetLastError();
}

hipError_t launch_release(int64_t* v, hipStream_t s) {
  hipLaunchKernelGGL(release_kernel, dim3(1), dim3(64), 0, s, v);
  return hipGetLastError();
}

hipError_t launch_wait(const int64_t* const* comp_tab, const int32_t* slices, int n, int groups,
                       uint64_t spin_limit, uint32_t* err, uint32_t gen, hipStream_t s) {
  if (n < 0 || n > FO_MAX_P || groups < 1 || groups > kMaxGroups) return hipErrorInvalidValue;
  SliceList l{};
  for (int i = 0; i < n; ++i) l.s[i] = slices[i];
  l.n = n;
  l.groups = groups;
  hipLaunchKernelGGL(wait_kernel, dim3(1), dim3(64), 0, s, comp_tab, l, spin_limit, err, gen);
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s) {
  if (a.n_recv < 0 || a.n_recv > FO_MAX_P || a.groups < 1 || a.groups > kMaxGroups || a.count < 0 ||
      a.go == nullptr)
    return hipErrorInvalidValue;
  for (int i = 0; i < a.n_recv; ++i)
    if (a.recv_slice[i] >= FO_MAX_P || (a.recv_slice[i] >= 0 && a.comp_tab == nullptr))
      return hipErrorInvalidValue;
  const int64_t items = a.vec4 ? a.count / 4 : a.count;
  const int64_t blocks =
      std::max<int64_t>(1, std::min<int64_t>((items + 255) / 256, std::max(1, a.max_blocks)));
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

TileShape tile_shape(int tile) {
  switch (tile) {
    case FO_TILE_256x256: return {256, 256};
    case FO_TILE_256x128: return {256, 128};
    case FO_TILE_128x256: return {128, 256};
    case FO_TILE_128x128: return {128, 128};
    case FO_TILE_64x64: return {64, 64};
    default: return {0, 0};
  }
}

// Host-side check of what the kernels index: signal tables behind every gate, awaited partial
// and release; slice ids and positions inside the tables; row groups that tile the rows.
static bool plan_ok(const Plan& p) {
  const TileGrid& g = p.grid;
  if (g.npos < 1 || g.npos > FO_MAX_P || g.tiles_m < 1 || g.tiles_n < 1) return false;
  if (g.groups < 1 || g.groups > kMaxGroups || g.group_rows < 1) return false;
  if ((int64_t)g.groups * g.group_rows < g.tiles_m || (g.groups - 1) * g.group_rows >= g.tiles_m)
    return false;
  if (g.lead < 0 || g.trail < 0 || g.lead + g.trail > g.npos) return false;
  if (p.done == nullptr || p.err == nullptr) return false;
  if (p.comp_tab != nullptr && (p.lead == nullptr || p.ready == nullptr || p.gen == 0)) return false;
  for (int i = 0; i < g.npos; ++i)
    if (p.gate_slice[i] >= FO_MAX_P || (p.gate_slice[i] >= 0 && p.comp_tab == nullptr)) return false;
  if (p.accum_pos >= g.npos || p.n_recv < 0 || p.n_recv > FO_MAX_P) return false;
  if (p.accum_pos >= 0 && !p.out_f32) return false;  // partials are added in fp32 output only
  // the SwiGLU epilogue: bf16 output, no added partials, gate and up halves of 8-column chunks
  if (p.act && (p.out_f32 || p.accum_pos >= 0 || p.N % 16 != 0)) return false;
  if (p.accum_pos >= 0)
    for (int i = 0; i < p.n_recv; ++i)
      if (p.recv_slice[i] >= FO_MAX_P || (p.recv_slice[i] >= 0 && p.comp_tab == nullptr))
        return false;
  if (p.tail_units < 0) return false;
  if (p.tail_units > 0 &&
      (p.accum_pos < 0 || p.own_done == nullptr || p.tail_per_group < 1 || p.tail_bm < 1 ||
       p.tail_units != g.groups * p.tail_per_group || p.act || p.N % 4 != 0 ||
       g.groups * g.group_rows * (int64_t)p.tail_bm < p.m ||
       (p.m * p.N * 4) >= ((int64_t)1 << 31)))
    return false;
  return true;
}

hipError_t launch_gemm(const Plan& p, int in_dt, int tile, hipStream_t s, hipEvent_t e0,
                       hipEvent_t e1) {
  if (!plan_ok(p)) return hipErrorInvalidValue;
  int64_t grid = (int64_t)p.grid.npos * p.grid.tiles_m * p.grid.tiles_n;
  if (in_dt == FO_DT_F32) {
    // the fp32 kernel has no SwiGLU epilogue and adds its partials itself
    if (p.act || p.tail_units) return hipErrorInvalidValue;
    hipExtLaunchKernelGGL(gemm_f32_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, e0, e1, 0,
                          p);
    return hipGetLastError();
  }
  grid += p.tail_units;
  switch (tile) {
    case FO_TILE_256x256: return launch_bf16<256, 256>(p, grid, s, e0, e1);
    case FO_TILE_256x128: return launch_bf16<256, 128>(p, grid, s, e0, e1);
    case FO_TILE_128x256: return launch_bf16<128, 256>(p, grid, s, e0, e1);
    case FO_TILE_128x128: return launch_bf16<128, 128>(p, grid, s, e0, e1);
    case FO_TILE_64x64: return launch_bf16<64, 64>(p, grid, s, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fo
