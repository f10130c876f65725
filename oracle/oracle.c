/*
 * Oracle for the Flash-Overlap hot path: a plain, slow CPU implementation in fp64.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call this file;
 * only the tests, the smoke check and the benchmark's CPU-baseline leg use it. It shares no
 * code, header, table or helper with the HIP library.
 *
 * Source of truth: the FlashOverlap page (gist.science, paper 2604.24013), technical summary,
 * section 2 "Methodology (Flash-Overlap)":
 *   - Flash-AG: All-Gather is split into ring-based asynchronous point-to-point transfers; the rank
 *     computes the slice it already holds first and the slices it receives afterwards.
 *   - Flash-RS: Reduce-Scatter is split into point-to-point transfers; rank-adaptive scheduling
 *     puts the slice that stays on this rank (it needs no further transfer) at the very end.
 *   - Architectural instantiations: column-parallel projection (All-Gather, then GEMM) and
 *     row-parallel projection (GEMM, then Reduce-Scatter).
 * Section 3 "Key contributions" states the algorithm is exact, so the sliced result is the plain
 * result: the oracle is the definition written out, C[i][j] = sum_k A[i][k] * B[k][j], in fp64.
 *
 * Readings where the page is silent (all listed in the design notes of the repository):
 *   - ring direction: a rank receives from rank r-1, so at ring step t the slice (r - t) mod P
 *     arrives; the Flash-AG order is r, r-1, ..., r-P+1 (mod P).
 *   - order of the chunks that leave the rank: r+1, r+2, ..., r+P-1, then r (own chunk last).
 *     At step i every rank targets a distinct peer.
 *   - each incoming partial is one peer's un-summed [m, N] contribution (direct point-to-point);
 *     at step i the partial of peer (r - i) mod P arrives, i = 1..P-1; they are added onto the
 *     own chunk's product in that order.
 *
 * Inputs are decoded exactly to fp64 (bf16 and fp32 both embed exactly in fp64).
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC oracle.c -o liboracle.so
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BF16 0
#define ORC_F32 1

/* bf16 is the upper half of an IEEE-754 binary32 pattern. */
static double decode_bf16(uint16_t h) {
  uint32_t bits = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double decode_elem(const void* base, int dt, int64_t idx) {
  if (dt == ORC_BF16) return decode_bf16(((const uint16_t*)base)[idx]);
  return (double)((const float*)base)[idx];
}

/* Decode a whole row-major [rows, cols] operand to fp64. Caller frees. */
static double* decode_matrix(const void* base, int dt, int64_t rows, int64_t cols) {
  double* out = (double*)malloc(sizeof(double) * (size_t)(rows * cols));
  if (!out) return NULL;
  for (int64_t i = 0; i < rows * cols; ++i) out[i] = decode_elem(base, dt, i);
  return out;
}

static int valid_dt(int dt) { return dt == ORC_BF16 || dt == ORC_F32; }

/* Flash-AG computation order for rank r: the local slice first, then the slices in the order the
   ring delivers them (from rank r-1, then r-2, ...). */
int oracle_ag_order(int P, int r, int* out) {
  if (P < 1 || r < 0 || r >= P || !out) return 1;
  for (int t = 0; t < P; ++t) out[t] = ((r - t) % P + P) % P;
  return 0;
}

/* Flash-RS computation order for rank r: chunks bound for the other ranks, r+1 .. r+P-1, then the
   chunk that stays on this rank last. */
int oracle_rs_order(int P, int r, int* out) {
  if (P < 1 || r < 0 || r >= P || !out) return 1;
  for (int i = 0; i < P - 1; ++i) out[i] = (r + 1 + i) % P;
  out[P - 1] = r;
  return 0;
}

/* C[M,N] = A[M,K] . B[K,N], all row-major; C in fp64. Rows are independent, so OpenMP splits
   them across threads; each entry is summed over k in increasing order. */
static void gemm_f64(const double* A, const double* B, double* C, int64_t M, int64_t K, int64_t N) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; ++i) {
    double* c = C + i * N;
    for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double a = A[i * K + k];
      const double* b = B + k * N;
      for (int64_t j = 0; j < N; ++j) c[j] += a * b[j];
    }
  }
}

int oracle_gemm(const void* A, int a_dt, const void* B, int b_dt, double* C, int64_t M, int64_t K,
                int64_t N) {
  if (!A || !B || !C || M < 0 || K < 0 || N < 0 || !valid_dt(a_dt) || !valid_dt(b_dt)) return 1;
  double* a = decode_matrix(A, a_dt, M, K);
  double* b = decode_matrix(B, b_dt, K, N);
  if (!a || !b) { free(a); free(b); return 2; }
  gemm_f64(a, b, C, M, K, N);
  free(a);
  free(b);
  return 0;
}

/* Flash-AG (column-parallel projection, All-Gather then GEMM).
   x_slices[s] is slice s, a row-major [m, K] block (slice s = rows s*m .. s*m+m-1 of the gathered
   activation). Y is [P*m, N]. Slices are processed in `order` (NULL: the Flash-AG order of rank r);
   the values cannot depend on the order, since each slice's rows are an independent product. */
int oracle_ag(const void* const* x_slices, int x_dt, const void* W, int w_dt, double* Y, int P,
              int r, const int* order, int64_t m, int64_t K, int64_t N) {
  if (!x_slices || !W || !Y || P < 1 || r < 0 || r >= P || m < 0 || K < 0 || N < 0) return 1;
  if (!valid_dt(x_dt) || !valid_dt(w_dt)) return 1;
  int* ord = (int*)malloc(sizeof(int) * (size_t)P);
  if (!ord) return 2;
  if (order) {
    int* seen = (int*)calloc((size_t)P, sizeof(int));
    if (!seen) { free(ord); return 2; }
    for (int t = 0; t < P; ++t) {
      if (order[t] < 0 || order[t] >= P || seen[order[t]]) { free(seen); free(ord); return 1; }
      seen[order[t]] = 1;
      ord[t] = order[t];
    }
    free(seen);
  } else {
    oracle_ag_order(P, r, ord);
  }
  double* w = decode_matrix(W, w_dt, K, N);
  if (!w) { free(ord); return 2; }
  int rc = 0;
  for (int t = 0; t < P && rc == 0; ++t) {
    const int s = ord[t];
    if (!x_slices[s]) { rc = 1; break; }
    double* xs = decode_matrix(x_slices[s], x_dt, m, K);
    if (!xs) { rc = 2; break; }
    gemm_f64(xs, w, Y + (int64_t)s * m * N, m, K, N);
    free(xs);
  }
  free(w);
  free(ord);
  return rc;
}

/* Flash-RS (row-parallel projection, GEMM then Reduce-Scatter), as seen by rank r.
   x_shard is this rank's [P*m, K] activation (full token range, its share of K); W is [K, N].
   Chunk d (rows d*m .. d*m+m-1 of x_shard . W) is the partial sum destined for rank d. Chunks are
   computed in the Flash-RS order; chunk d != r is what would be sent to rank d and is written to
   send[d*m*N ...] when send is non-NULL. The own chunk r comes last, and
   out[m, N] = S_r + partial[(r-1) mod P] + partial[(r-2) mod P] + ... + partial[(r-P+1) mod P],
   added in that (arrival) order. partials[q] is peer q's [m, N] fp32 partial for chunk r;
   partials[r] is ignored. */
int oracle_rs(const void* x_shard, int x_dt, const void* W, int w_dt, const float* const* partials,
              double* out, double* send, int P, int r, int64_t m, int64_t K, int64_t N) {
  if (!x_shard || !W || !out || P < 1 || r < 0 || r >= P || m < 0 || K < 0 || N < 0) return 1;
  if (!valid_dt(x_dt) || !valid_dt(w_dt)) return 1;
  if (P > 1 && !partials) return 1;
  for (int q = 0; q < P; ++q)
    if (q != r && !partials[q]) return 1;
  int* ord = (int*)malloc(sizeof(int) * (size_t)P);
  if (!ord) return 2;
  oracle_rs_order(P, r, ord);
  double* w = decode_matrix(W, w_dt, K, N);
  double* chunk = (double*)malloc(sizeof(double) * (size_t)(m * N));
  if (!w || !chunk) { free(ord); free(w); free(chunk); return 2; }
  int rc = 0;
  for (int t = 0; t < P && rc == 0; ++t) {
    const int d = ord[t];
    const uint8_t* xb = (const uint8_t*)x_shard;
    const int64_t esz = (x_dt == ORC_BF16) ? 2 : 4;
    double* xd = decode_matrix(xb + (int64_t)d * m * K * esz, x_dt, m, K);
    if (!xd) { rc = 2; break; }
    gemm_f64(xd, w, chunk, m, K, N);
    free(xd);
    if (d != r) {
      if (send) memcpy(send + (int64_t)d * m * N, chunk, sizeof(double) * (size_t)(m * N));
    } else {
      for (int64_t e = 0; e < m * N; ++e) out[e] = chunk[e];
      for (int i = 1; i < P; ++i) {
        const int q = ((r - i) % P + P) % P;
        const float* pq = partials[q];
        for (int64_t e = 0; e < m * N; ++e) out[e] += (double)pq[e];
      }
    }
  }
  free(chunk);
  free(w);
  free(ord);
  return rc;
}

/* Single entries of A . B: out[t] = sum_k A[rows[t]][k] * B[k][cols[t]] in fp64, for checking
   products too large for the full oracle. A is [*, K], B is [K, N]. */
static double dot_entry(const void* A, int a_dt, const void* B, int b_dt, int64_t row, int64_t col,
                        int64_t K, int64_t N) {
  double s = 0.0;
  for (int64_t k = 0; k < K; ++k)
    s += decode_elem(A, a_dt, row * K + k) * decode_elem(B, b_dt, k * N + col);
  return s;
}

/* Sampled Flash-AG output entries: Y[rows[t]][cols[t]] with row i taken from slice i / m. */
int oracle_ag_sampled(const void* const* x_slices, int x_dt, const void* W, int w_dt, int P,
                      int64_t m, int64_t K, int64_t N, const int64_t* rows, const int64_t* cols,
                      int64_t n, double* out) {
  if (!x_slices || !W || !rows || !cols || !out || P < 1 || m < 1 || K < 0 || N < 1) return 1;
  if (!valid_dt(x_dt) || !valid_dt(w_dt)) return 1;
  for (int64_t t = 0; t < n; ++t)
    if (rows[t] < 0 || rows[t] >= P * m || cols[t] < 0 || cols[t] >= N || !x_slices[rows[t] / m])
      return 1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < n; ++t) {
    const int64_t s = rows[t] / m;
    out[t] = dot_entry(x_slices[s], x_dt, W, w_dt, rows[t] - s * m, cols[t], K, N);
  }
  return 0;
}

/* Sampled Flash-RS own-chunk entries: out[rows[t]][cols[t]] of rank r (rows index the [m, N]
   chunk), the product plus the incoming partials in arrival order. */
int oracle_rs_sampled(const void* x_shard, int x_dt, const void* W, int w_dt,
                      const float* const* partials, int P, int r, int64_t m, int64_t K, int64_t N,
                      const int64_t* rows, const int64_t* cols, int64_t n, double* out) {
  if (!x_shard || !W || !rows || !cols || !out || P < 1 || r < 0 || r >= P || m < 1 || N < 1)
    return 1;
  if (!valid_dt(x_dt) || !valid_dt(w_dt)) return 1;
  for (int q = 0; q < P; ++q)
    if (q != r && (!partials || !partials[q])) return 1;
  for (int64_t t = 0; t < n; ++t)
    if (rows[t] < 0 || rows[t] >= m || cols[t] < 0 || cols[t] >= N) return 1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < n; ++t) {
    double v = dot_entry(x_shard, x_dt, W, w_dt, (int64_t)r * m + rows[t], cols[t], K, N);
    for (int i = 1; i < P; ++i) {
      const int q = ((r - i) % P + P) % P;
      v += (double)partials[q][rows[t] * N + cols[t]];
    }
    out[t] = v;
  }
  return 0;
}

/* Sampled entries of one send chunk d != r of rank r: rows index the [m, N] chunk. */
int oracle_rs_send_sampled(const void* x_shard, int x_dt, const void* W, int w_dt, int d,
                           int64_t m, int64_t K, int64_t N, const int64_t* rows,
                           const int64_t* cols, int64_t n, double* out) {
  if (!x_shard || !W || !rows || !cols || !out || d < 0 || m < 1 || N < 1) return 1;
  if (!valid_dt(x_dt) || !valid_dt(w_dt)) return 1;
  for (int64_t t = 0; t < n; ++t)
    if (rows[t] < 0 || rows[t] >= m || cols[t] < 0 || cols[t] >= N) return 1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < n; ++t)
    out[t] = dot_entry(x_shard, x_dt, W, w_dt, (int64_t)d * m + rows[t], cols[t], K, N);
  return 0;
}

/* ---- The MLP block (NEXT: the workload of the page's MLP-layer latency) ------------------
 *
 * Section 4 of the technical summary reports the end-to-end latency of an MLP layer: the
 * column-parallel projection (Flash-AG), the activation, and the row-parallel projection
 * (Flash-RS). The workloads' shapes are Llama-3.1's, whose MLP activation is SwiGLU (a reading:
 * the page does not name it): h = silu(gate) * up with silu(g) = g / (1 + e^-g), gate and up
 * being the two halves [0, inter) and [inter, 2*inter) of the gate+up projection's columns.
 * Between the kernels the activations are bf16: each intermediate is rounded to the nearest bf16
 * value, ties to even. */

/* h[r][j] = silu(y[r][j]) * y[r][inter + j] in fp64; y is bf16 [rows, 2*inter]. */
int oracle_swiglu(const uint16_t* y, int64_t rows, int64_t inter, double* h) {
  if (!y || !h || rows < 0 || inter < 0) return 1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < inter; ++j) {
      const double g = decode_bf16(y[r * 2 * inter + j]);
      const double u = decode_bf16(y[r * 2 * inter + inter + j]);
      h[r * inter + j] = g / (1.0 + exp(-g)) * u;
    }
  return 0;
}

/* The same activation on an fp64 y [rows, 2*inter] (gate half, then up half): the fused form,
   where the activation reads the projection's sums before any rounding. */
int oracle_swiglu_f64(const double* y, int64_t rows, int64_t inter, double* h) {
  if (!y || !h || rows < 0 || inter < 0) return 1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < inter; ++j) {
      const double g = y[r * 2 * inter + j];
      const double u = y[r * 2 * inter + inter + j];
      h[r * inter + j] = g / (1.0 + exp(-g)) * u;
    }
  return 0;
}

/* x rounded to 8 significant bits (the bf16 precision), to nearest, ties to even, written as
   bf16 bit patterns. For finite x within bf16's normal range (or zero): x = f * 2^e with
   0.5 <= |f| < 1, f * 2^8 is rounded to an integer (nearbyint rounds ties to even in the default
   rounding mode) and scaled back; the result has at most 8 significant bits, so it is exact as a
   float, whose upper 16 bits are the bf16 pattern. */
int oracle_round_bf16(const double* x, int64_t n, uint16_t* out) {
  if (!x || !out || n < 0) return 1;
  for (int64_t i = 0; i < n; ++i) {
    int e = 0;
    const double f = frexp(x[i], &e);
    const double v = ldexp(nearbyint(ldexp(f, 8)), e - 8);
    const float fv = (float)v;
    uint32_t bits;
    memcpy(&bits, &fv, sizeof bits);
    out[i] = (uint16_t)(bits >> 16);
  }
  return 0;
}

/* Number of OpenMP threads a parallel region uses (reported beside the CPU timing). */
int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      extern int omp_get_num_threads(void);
      n = omp_get_num_threads();
#endif
    }
  }
  return n;
}

/* Attention of one rank after the All-to-All of Ulysses (sequence) parallelism. The page
   (technical summary section 2, "Query Split Attention" and "Flash All-to-All") splits the
   attention by query slices to overlap it with the arriving slices; the softmax is taken over
   all key positions a query sees, so the result is plain scaled dot-product attention whatever
   the split and order. This is that definition in fp64, per query position i and head h:
     s_j = (q_i,h . k_j,g) / sqrt(d) for key positions j (j <= i when causal), g = h / (hq / hkv);
     out[i, h] = sum_j exp(s_j - max s) v_j,g / sum_j exp(s_j - max s).
   qkv: bf16 [S, (hq + 2 hkv) * d], a token's row = [hq query heads | hkv key heads | hkv value
   heads]. rows: the nrows query positions to compute (NULL: all S, in order). out: fp64
   [nrows, hq * d]. */
int oracle_attn(const uint16_t* qkv, int64_t S, int hq, int hkv, int d, int causal,
                const int64_t* rows, int64_t nrows, double* out) {
  if (!qkv || !out || S < 0 || hq < 1 || hkv < 1 || hq % hkv || d < 1) return 1;
  if (!rows) nrows = S;
  if (nrows < 0) return 1;
  const int64_t W = (int64_t)(hq + 2 * hkv) * d;
  const double scale = 1.0 / sqrt((double)d);
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t t = 0; t < nrows; ++t) {
    const int64_t i = rows ? rows[t] : t;
    if (i < 0 || i >= S) { bad = 1; continue; }
    const int64_t nk = causal ? i + 1 : S;
    double* sc = (double*)malloc(sizeof(double) * (size_t)nk);
    if (!sc) { bad = 1; continue; }
    for (int h = 0; h < hq; ++h) {
      const int g = h / (hq / hkv);
      const uint16_t* q = qkv + i * W + (int64_t)h * d;
      double mx = -INFINITY;
      for (int64_t j = 0; j < nk; ++j) {
        const uint16_t* k = qkv + j * W + (int64_t)(hq + g) * d;
        double dot = 0.0;
        for (int e = 0; e < d; ++e) dot += decode_bf16(q[e]) * decode_bf16(k[e]);
        sc[j] = dot * scale;
        if (sc[j] > mx) mx = sc[j];
      }
      double den = 0.0;
      for (int64_t j = 0; j < nk; ++j) {
        sc[j] = exp(sc[j] - mx);
        den += sc[j];
      }
      double* o = out + t * (int64_t)hq * d + (int64_t)h * d;
      for (int e = 0; e < d; ++e) o[e] = 0.0;
      for (int64_t j = 0; j < nk; ++j) {
        const uint16_t* v = qkv + j * W + (int64_t)(hq + hkv + g) * d;
        for (int e = 0; e < d; ++e) o[e] += sc[j] * decode_bf16(v[e]);
      }
      for (int e = 0; e < d; ++e) o[e] /= den;
    }
    free(sc);
  }
  return bad ? 1 : 0;
}
