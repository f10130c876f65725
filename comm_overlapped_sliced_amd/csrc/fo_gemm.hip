// Sliced GEMM kernels of libflashovl for gfx950 (MI355X).
//
// One launch computes every slice of a Flash-AG or Flash-RS call (FlashOverlap page, technical
// summary section 2): workgroups are laid out in schedule order, a tile of a slice that is still
// in flight waits on that slice's arrival flag before reading it, and the chunk that stays on the
// rank (Flash-RS) adds the partials received from the peers in its write-back.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 with fp32 accumulation. Each workgroup is 4 waves (2 x 2);
// each wave owns a (BM/2) x (BN/2) block of 32x32 MFMA fragments. K advances in steps of 64
// through two LDS stages: the next step's operands are fetched from HBM into registers with
// 128-bit loads while the current stage feeds the MFMAs. A (K-contiguous) is stored to LDS as
// is; W (N-contiguous) is transposed in registers on the way so that both operands are read
// from LDS as 16-byte K-runs. LDS rows are 128 bytes with an XOR swizzle of the 16-byte chunks
// so that the fragment reads and the transposed writes are free of bank conflicts.
//
// fp32 path: a plain LDS-tiled fp32 FMA kernel (exact fp32 products, fp32 sums in k order).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fo_internal.h"

namespace fo {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kThreads = 256;
constexpr int kBK = 64;  // K step (one 128-byte LDS row per operand row)

// ---------------------------------------------------------------- waits and flags -----------

// Bounded wait for flag == epoch. Once any wait of the call has run past the bound (err set),
// later waits give up at once, so a missing arrival costs one bound, not one per workgroup.
__device__ __forceinline__ void wait_flag(const uint32_t* flag, uint32_t epoch, uint64_t limit,
                                          uint32_t* err) {
  const uint64_t t0 = wall_clock64();
  while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != epoch) {
    if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0u) return;
    if (wall_clock64() - t0 > limit) {
      __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Thread 0 waits for every listed flag; then the whole workgroup acquires at system scope so
// that data written by the copy engine before the flag is seen (no stale cache lines).
__device__ __forceinline__ void wait_flags_wg(const Plan& p, const int32_t* ids, int n) {
  if (threadIdx.x == 0) {
    for (int i = 0; i < n; ++i)
      if (ids[i] >= 0) wait_flag(p.arr + ids[i], p.epoch, p.spin_limit, p.err);
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
}

// After a tile of position `pos` is stored: count it; the last tile of the position raises the
// position's release flag (read by the copy stream's wait) and re-arms the counter.
__device__ __forceinline__ void release_tile(const Plan& p, int pos, int tiles_per_pos) {
  if (p.rel[pos] == nullptr) return;
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
    const uint32_t old = __hip_atomic_fetch_add(p.done + pos, 1u, __ATOMIC_ACQ_REL,
                                                __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == (uint32_t)tiles_per_pos) {
      __hip_atomic_store(p.done + pos, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.rel[pos], p.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

// fp32 -> bf16, round to nearest, ties to even (quiet NaN kept).
__device__ __forceinline__ uint16_t to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Tile order inside one position. Workgroup b runs on XCD b % 8; when a position has a multiple
// of 8 tiles, XCD x is given the x-th contiguous run of tiles (column-major over the tile grid),
// so every XCD reuses the same W column blocks across slices in its own L2.
__device__ __forceinline__ int remap_tile(int u, int T) {
  if (T % 8) return u;
  return (u % 8) * (T / 8) + u / 8;
}

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// Writes one 32x32 accumulator fragment: lane (lr, lh) holds column lr and rows
// 8*(v/4) + 4*lh + v%4 of the fragment in element v. The accumulate epilogue adds the received
// partials in arrival order onto the fp32 value before the store.
__device__ __forceinline__ void store_fragment(const Plan& p, int pos, const f32x16 a,
                                               int64_t row0, int64_t rbase, int64_t rows_valid,
                                               int64_t col, bool accum) {
  if (col >= p.N) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t r = rbase + 8 * (v >> 2) + (v & 3);
    if (r >= rows_valid) continue;
    const int64_t off = (row0 + r) * p.N + col;
    float x = a[v];
    if (accum)
      for (int q = 0; q < p.n_recv; ++q) x += p.recv[q][off];
    if (p.out_f32)
      ((float*)p.c_pos[pos])[off] = x;
    else
      ((uint16_t*)p.c_pos[pos])[off] = to_bf16_rne(x);
  }
}

// ---------------------------------------------------------------- bf16 MFMA kernel ----------

template <int BM, int BN>
struct Cfg {
  static constexpr int WTM = BM / 2, WTN = BN / 2;  // wave tile (2 x 2 waves)
  static constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 fragments per wave
  static constexpr int A_CH = BM * kBK / 8 / kThreads;  // 16-byte A chunks per thread
  static constexpr int KB = BN / 32;                   // W rows per thread in the transposer
  static constexpr int NBLK = BN / 8;                  // 8-column blocks of a W tile row
  static constexpr int LDS_A = BM * kBK * 2;
  static constexpr int LDS_B = BN * kBK * 2;
  static constexpr int LDS_STAGE = LDS_A + LDS_B;
  static_assert(A_CH >= 1 && KB >= 2 && KB <= 8 && FM >= 1 && FN >= 1, "tile");
};

template <int KB>
struct WRegs {
  uint4 r[KB];
};

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int d) {
  return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

template <int BM, int BN>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(Plan p) {
  using C = Cfg<BM, BN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::LDS_STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int T = p.tiles_m * p.tiles_n;
  const int pos = blockIdx.x / T;
  const int t = remap_tile(blockIdx.x - pos * T, T);
  const int tm = t % p.tiles_m, tn = t / p.tiles_m;

  const int64_t K = p.K, N = p.N;
  const int64_t row0 = (int64_t)tm * BM;   // first row of the tile inside the slice
  const int64_t col0 = (int64_t)tn * BN;
  const int64_t rows_valid = p.m - row0;   // >= 1
  const uint16_t* A = (const uint16_t*)p.a_pos[pos] + row0 * K;
  const uint16_t* B = (const uint16_t*)p.b + col0;

  // Flash-AG: a received slice is read only after its arrival flag.
  if (p.gate[pos] >= 0) wait_flags_wg(p, p.gate + pos, 1);

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  uint4 ra[C::A_CH];
  WRegs<C::KB> rb;
  const int a_c = tid & 7;            // A: 16-byte chunk of the 128-byte K run
  const int a_r = tid >> 3;           // A: first row (then +32 per chunk)
  const int b_nb = tid % C::NBLK;     // W: 8-column block
  const int b_kg = tid / C::NBLK;     // W: group of KB consecutive k rows

  auto load_global = [&](int kt) {
    const int64_t k0 = (int64_t)kt * kBK;
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
      const int r = a_r + 32 * i;
      const int64_t k = k0 + a_c * 8;
      if (r < rows_valid && k < K)
        ra[i] = *(const uint4*)(A + (int64_t)r * K + k);
      else
        ra[i] = make_uint4(0, 0, 0, 0);
    }
    const int64_t n = col0 + b_nb * 8;
#pragma unroll
    for (int j = 0; j < C::KB; ++j) {
      const int64_t k = k0 + b_kg * C::KB + j;
      if (k < K && n < N)
        rb.r[j] = *(const uint4*)(B + k * N + b_nb * 8);
      else
        rb.r[j] = make_uint4(0, 0, 0, 0);
    }
  };

  auto store_lds = [&](int stage) {
    uint8_t* sa = smem + stage * C::LDS_STAGE;
    uint8_t* sb = sa + C::LDS_A;
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
      const int r = a_r + 32 * i;
      *(uint4*)(sa + r * 128 + ((a_c ^ swz(r)) << 4)) = ra[i];
    }
    // transpose the KB x 8 block of W: column e of the block becomes a K-run of row n.
    // dword d of row j holds columns 2d (low half) and 2d+1 (high half)
    const int kbyte = b_kg * C::KB * 2;         // byte offset of this K-run in the 128-byte row
    const int chunk = kbyte >> 4, intra = kbyte & 15;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int n = b_nb * 8 + e;
      uint32_t o[C::KB / 2];
#pragma unroll
      for (int q = 0; q < C::KB / 2; ++q) {
        const uint32_t lo = dword_of(rb.r[2 * q], e >> 1);
        const uint32_t hi = dword_of(rb.r[2 * q + 1], e >> 1);
        o[q] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      uint8_t* dst = sb + n * 128 + ((chunk ^ swz(n)) << 4) + intra;
      if constexpr (C::KB == 8)
        *(uint4*)dst = make_uint4(o[0], o[1], o[2], o[3]);
      else if constexpr (C::KB == 4)
        *(uint2*)dst = make_uint2(o[0], o[1]);
      else
        *(uint32_t*)dst = o[0];
    }
  };

  auto compute = [&](int stage) {
    const uint8_t* sa = smem + stage * C::LDS_STAGE;
    const uint8_t* sb = sa + C::LDS_A;
    const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int c = 2 * kk + lh;
      bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int r = wm * C::WTM + i * 32 + lr;
        af[i] = __builtin_bit_cast(bf16x8, *(const uint4*)(sa + r * 128 + ((c ^ swz(r)) << 4)));
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int n = wn * C::WTN + j * 32 + lr;
        bfr[j] = __builtin_bit_cast(bf16x8, *(const uint4*)(sb + n * 128 + ((c ^ swz(n)) << 4)));
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  const int KT = (int)((K + kBK - 1) / kBK);
  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_global(kt + 1);
    compute(cur);
    if (kt + 1 < KT) store_lds(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------------------
  const bool accum = (pos == p.accum_pos);
  if (accum) wait_flags_wg(p, p.recv_flag, p.n_recv);
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int64_t col = col0 + wn * C::WTN + j * 32 + lr;
      const int64_t rbase = (int64_t)wm * C::WTM + i * 32 + 4 * lh;
      store_fragment(p, pos, acc[i][j], row0, rbase, rows_valid, col, accum);
    }
  }
  release_tile(p, pos, T);
}

// ---------------------------------------------------------------- fp32 kernel ----------------

constexpr int F_BM = 64, F_BN = 64, F_BK = 16;

__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(Plan p) {
  __shared__ float sa[F_BK][F_BM + 4];  // k-major so a thread's 4 rows are one broadcast read
  __shared__ float sb[F_BK][F_BN + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;

  const int T = p.tiles_m * p.tiles_n;
  const int pos = blockIdx.x / T;
  const int t = blockIdx.x - pos * T;
  const int tm = t % p.tiles_m, tn = t / p.tiles_m;
  const int64_t K = p.K, N = p.N;
  const int64_t row0 = (int64_t)tm * F_BM, col0 = (int64_t)tn * F_BN;
  const int64_t rows_valid = p.m - row0;
  const float* A = (const float*)p.a_pos[pos] + row0 * K;
  const float* B = (const float*)p.b + col0;

  if (p.gate[pos] >= 0) wait_flags_wg(p, p.gate + pos, 1);

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

  const bool accum = (pos == p.accum_pos);
  if (accum) wait_flags_wg(p, p.recv_flag, p.n_recv);
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
  release_tile(p, pos, T);
}

template <int BM, int BN>
hipError_t launch_bf16(const Plan& p, hipStream_t s) {
  const int64_t grid = (int64_t)p.npos * p.tiles_m * p.tiles_n;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN>), dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

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

hipError_t launch_gemm(const Plan& p, int in_dt, int tile, hipStream_t s) {
  if (in_dt == FO_DT_F32) {
    const int64_t grid = (int64_t)p.npos * p.tiles_m * p.tiles_n;
    hipLaunchKernelGGL(gemm_f32_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
  }
  switch (tile) {
    case FO_TILE_256x256: return launch_bf16<256, 256>(p, s);
    case FO_TILE_256x128: return launch_bf16<256, 128>(p, s);
    case FO_TILE_128x256: return launch_bf16<128, 256>(p, s);
    case FO_TILE_128x128: return launch_bf16<128, 128>(p, s);
    case FO_TILE_64x64: return launch_bf16<64, 64>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fo
