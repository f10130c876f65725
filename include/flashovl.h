/*
 * libflashovl — the Flash-Overlap hot path on AMD MI355X (gfx950): one tensor-parallel rank's
 * share of the MLP projections, computed slice by slice while the other slices are in flight.
 *
 * What is computed follows the FlashOverlap page (gist.science, paper 2604.24013), technical
 * summary section 2 "Methodology (Flash-Overlap)":
 *   - Flash-AG (Flash-All-Gather): All-Gather split into ring point-to-point transfers; the rank
 *     multiplies the slice it already holds first and each received slice after it arrives.
 *   - Flash-RS (Flash-Reduce-Scatter): Reduce-Scatter split into point-to-point transfers;
 *     rank-adaptive scheduling computes the chunk that stays on the rank last, and the partial
 *     sums received from the other ranks are added into it.
 *   - Architectural instantiations: the column-parallel projection (All-Gather, then GEMM) and
 *     the row-parallel projection (GEMM, then Reduce-Scatter) of MLP and attention layers.
 * Section 3 ("Key contributions") states the algorithm is exact: every result equals the plain
 * product, whatever the slice order.
 *
 * On one GPU the peer ranks are emulated: a "peer" buffer holds what the peer would send, and the
 * library copies it into the receive buffer with one of the GPU's SDMA engines (one engine
 * stands for one link). Kernels wait per slice on the copy's completion; there is no global
 * barrier, and neither a transfer nor its gating takes a compute unit from the GEMM.
 *
 * Conventions for every entry point:
 *   - All matrices are dense and row-major. X is [rows, K], W is [K, N] (N contiguous), outputs
 *     are [rows, N]. bf16 is the IEEE binary32 upper half; accumulation is fp32.
 *   - Device pointers are device memory on the current HIP device. Arrays "of P pointers" are
 *     host arrays of device pointers. The caller owns every buffer; the library never frees
 *     caller memory. bf16 operands must be 16-byte aligned with K and N multiples of 8; fp32
 *     buffers must be 4-byte aligned; the slice height m may be any value >= 0 (0: nothing to
 *     do) and K may be 0 (empty sums).
 *   - Streams are hipStream_t passed as void*; NULL = the null stream. Calls are stream-ordered
 *     and return after enqueueing. The transfers run on DMA engines outside any HIP stream, but a
 *     call's kernel completes only after every transfer it waits for has landed, so synchronizing
 *     the compute stream is enough (fo_check() also waits for transfers a timed-out kernel left
 *     behind). Calls on one device are serialized by the library: each waits for the previous
 *     call's kernel, whichever stream that was on.
 *   - Errors are return codes; nothing is enqueued when an argument is rejected. An in-kernel
 *     wait that exceeds opts->spin_timeout_us is recorded on the device and reported as
 *     FO_ERR_TIMEOUT by fo_check(); the kernel still runs to completion (no hang), but that
 *     call's results are then unspecified. The record names the call: its other waits give up
 *     at once, while the calls enqueued after it wait as usual and are unaffected.
 *   - Thread safety: entry points may be called from several host threads; each call holds a
 *     per-device lock while it enqueues.
 */
#ifndef FLASHOVL_H
#define FLASHOVL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FO_VERSION 1
#define FO_MAX_P 32     /* largest tensor-parallel degree (number of slices) */
#define FO_MAX_GROUPS 8 /* most row groups per slice (fo_opts.row_groups) */
#define FO_NOALLOC_SCRATCH_BYTES 4096 /* per-device static scratch of fo_gemm_rs_noalloc */

typedef enum fo_status {
  FO_OK = 0,
  FO_ERR_INVALID_ARG = 1, /* a NULL/misaligned pointer, bad size, rank, dtype or option */
  FO_ERR_UNSUPPORTED = 2, /* well-formed but not implemented (e.g. a dtype combination) */
  FO_ERR_HIP = 3,         /* a HIP or HSA runtime call or a DMA transfer failed; fo_last_error()
                             has the message */
  FO_ERR_TIMEOUT = 4      /* an in-kernel arrival wait ran past its bound */
} fo_status;

typedef enum fo_dtype { FO_DT_BF16 = 0, FO_DT_F32 = 1 } fo_dtype;

/* Slice order. FLASH: the page's schedule (AG: local slice first, then ring arrivals; RS: chunks
   for the other ranks first, own chunk last, partials added in its write-back). NATURAL: slices
   in index order 0..P-1, the data-slicing baseline of the page's problem statement; in fo_gemm_rs
   the own chunk is then written where it falls and the partials are added after the GEMM by a
   separate pass (the tail that data slicing cannot hide), with the same adds in the same order,
   so both orders give bitwise the same result. */
typedef enum fo_order { FO_ORDER_FLASH = 0, FO_ORDER_NATURAL = 1 } fo_order;

/* How emulated peer data arrives. NONE: the data is already resident in the receive buffer and
   no slice waits. EAGER: every copy is enqueued at the start of the call. LOCKSTEP (RS only): the
   partial that rank r receives at step i is released only when rank r has finished its own step
   i-1, modelling peers that progress in step with this rank. DEFAULT: EAGER for AG, LOCKSTEP for
   RS. */
typedef enum fo_arrival {
  FO_ARR_DEFAULT = 0,
  FO_ARR_NONE = 1,
  FO_ARR_EAGER = 2,
  FO_ARR_LOCKSTEP = 3
} fo_arrival;

/* Tile shape of the bf16 GEMM (rows x columns of one workgroup's output tile). AUTO picks one
   from the shape. */
typedef enum fo_tile {
  FO_TILE_AUTO = 0,
  FO_TILE_256x256 = 1,
  FO_TILE_256x128 = 2,
  FO_TILE_128x256 = 3,
  FO_TILE_128x128 = 4,
  FO_TILE_64x64 = 5
} fo_tile;

/* Epilogue of fo_ag_gemm. NONE: y = X . W. SWIGLU: the gate+up projection of the MLP block with
   its activation fused into the write-back: W is [K, N] with the gate projection in columns
   [0, N/2) and the up projection in [N/2, N); y receives h = silu(X . W_gate) * (X . W_up),
   [P*m, N/2] bf16, from the fp32 accumulators (one rounding; fo_swiglu on a bf16 y rounds
   twice). Needs bf16 operands and output and N a multiple of 16. */
typedef enum fo_epilogue { FO_EPI_NONE = 0, FO_EPI_SWIGLU = 1 } fo_epilogue;

typedef struct fo_opts {
  int32_t order;            /* fo_order */
  int32_t arrival;          /* fo_arrival */
  int32_t tile;             /* fo_tile */
  uint32_t spin_timeout_us; /* bound of each in-kernel wait; 0 = 2 000 000 us */
  int32_t links;            /* emulated links (DMA engines) the call's transfers use: the t-th
                               transfer goes over link t mod links, transfers on one link run
                               one after the other. 0 = P-1 (one link per peer, the full xGMI
                               mesh of an 8-GPU node); 1 = a single link, as in a ring whose
                               slices all come from one neighbour */
  int32_t row_groups;       /* granularity of transfer, gating and release: each slice (AG) or
                               chunk (RS) is cut into this many groups of whole tile rows,
                               each its own transfer that the tiles of those rows wait for; the
                               received slices (AG) and the chunks for other ranks (RS) are
                               then computed group by group across slices (all first groups,
                               then all second groups, ...), with the local slice (AG) first and
                               the own chunk (RS) last, each whole. 1 = whole slices, the page's
                               slice-by-slice order; 0 = one group per tile row, at most
                               FO_MAX_GROUPS */
  void* kernel_events[2];   /* optional hipEvent_t pair (created by the caller) that the GEMM
                               kernel's launch gives its own start and end times
                               (hipExtLaunchKernel; no marker packets on the stream): for
                               hipEventElapsedTime, not for ordering other work (profiling) */
  int32_t epilogue;         /* fo_epilogue (fo_ag_gemm only; else FO_ERR_INVALID_ARG) */
  int32_t k_chunks;         /* fo_ag_gemm only (else it must be 0 or 1): 0 or 1 = every X slice
                               row-major [m, K]. c in 2..FO_MAX_GROUPS = every X slice (x_local,
                               each x_peer[s], and slice s of x_recv) stored K-chunk-major: c
                               blocks one after another, block j holding columns j*K/c ..
                               (j+1)*K/c - 1 of the slice's m rows, row-major [m, K/c]. Each row
                               group of a received slice then travels as c transfers, block by
                               block, and its tiles start once block 0 has landed, waiting for
                               block j only before they read its columns. Needs bf16 operands,
                               K a multiple of 256*c and m*K*2 <= 2^30 bytes (else
                               FO_ERR_UNSUPPORTED); row groups are capped at FO_MAX_GROUPS / c */
  int32_t engines_per_link; /* DMA engines that carry one emulated link: 1 = one engine, the
                               link's transfers one after the other; 2 = the two engines of a
                               pair (which share one bandwidth) taking the link's transfers in
                               turn, so that one copy's start-up overlaps the other's data (a
                               link's transfers may then land out of issue order; every wait is
                               per transfer, so results do not change); 3 = the pair, every
                               transfer cut in two halves, one on each engine, landing when both
                               have; 0 = the default (3) */
  int32_t reserved;         /* must be 0 */
} fo_opts;

/* Fills *o with the defaults (FLASH order, DEFAULT arrival, AUTO tile, 2 s bound, one link per
   peer, one row group per tile row, no events). */
void fo_opts_init(fo_opts* o);

/*
 * Flash-AG: Y = [X_0; X_1; ...; X_{P-1}] . W for rank `rank` (column-parallel projection).
 *   x_local  device [m, K] in_dt: this rank's slice X_rank.
 *   x_peer   host array of P device pointers; x_peer[s] ([m, K] in_dt) is what peer s sends.
 *            Entry [rank] is ignored. NULL: no transfers, the slices are already in x_recv.
 *   x_recv   device [P*m, K] in_dt receive buffer; slice s arrives at x_recv + s*m*K. The rows of
 *            slice `rank` are neither read nor written.
 *   w        device [K, N] in_dt, this rank's column shard of the weight.
 *   y        device [P*m, N] out_dt; rows s*m .. s*m+m-1 hold X_s . W (with opts.epilogue
 *            FO_EPI_SWIGLU: [P*m, N/2] bf16 holding silu(X_s . W_gate) * (X_s . W_up)).
 * Slices are computed in the Flash-AG order (rank, rank-1, ..., rank-P+1 mod P); slice s != rank
 * is read only after its transfer has landed. in_dt and out_dt: BF16 or F32; out_dt BF16
 * rounds the fp32 accumulator to nearest-even. No output may overlap an input.
 * With opts.k_chunks = c > 1 every X slice (x_local, x_peer[s], slice s of x_recv, each m*K
 * values at the same places) is in the K-chunk-major layout described at fo_opts; y is
 * unchanged and equal, bit for bit, to the row-major call's.
 */
fo_status fo_ag_gemm(const void* x_local, const void* const* x_peer, void* x_recv, const void* w,
                     void* y, int32_t P, int32_t rank, int64_t m, int64_t K, int64_t N,
                     int32_t in_dt, int32_t out_dt, void* compute_stream, const fo_opts* opts);

/*
 * Flash-RS: the P row-chunks of X_shard . W for rank `rank` (row-parallel projection), own chunk
 * last, plus the partials received from the other ranks.
 *   x_shard      device [P*m, K] in_dt: this rank's activation (all tokens, its share of K).
 *   w            device [K, N] in_dt: this rank's row shard of the weight.
 *   send_buf     device [P*m, N] fp32; chunk d != rank (rows d*m..) receives X_shard[d rows] . W,
 *                the partial this rank would send to rank d. Chunk `rank` is not written.
 *   out          device [m, N] fp32: X_shard[rank rows] . W + sum of the incoming partials, added
 *                onto the fp32 accumulator in arrival order q = rank-1, rank-2, ... (mod P).
 *                With bf16 operands and 16-byte aligned out and recv_buf chunks the adds run in
 *                workgroups of the same launch after a row group's tiles have stored their sums
 *                (spread over the CUs the other chunks freed), else in the tiles' write-back;
 *                the order of the adds, and so every bit of out, is the same.
 *   peer_partial host array of P device pointers; peer_partial[q] ([m, N] fp32) is what peer q
 *                sends for this rank's chunk. Entry [rank] ignored. NULL: no transfers, the
 *                partials are already in recv_buf.
 *   recv_buf     device [P*m, N] fp32; peer q's partial arrives at recv_buf + q*m*N.
 * Chunks are computed in the Flash-RS order (rank+1, ..., rank+P-1, rank mod P), or in index order
 * with opts->order NATURAL. LOCKSTEP arrivals: peer rank-1-t sends its partial when this rank ends
 * its step t (FLASH), or when this rank ends the step of its own chunk (NATURAL, where every rank
 * computes chunk d at step d).
 */
fo_status fo_gemm_rs(const void* x_shard, const void* w, float* send_buf, float* out,
                     const float* const* peer_partial, float* recv_buf, int32_t P, int32_t rank,
                     int64_t m, int64_t K, int64_t N, int32_t in_dt, void* compute_stream,
                     const fo_opts* opts);

/*
 * fo_gemm_rs with every incoming partial already in recv_buf, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The result is that of fo_gemm_rs with peer_partial = NULL (the same kernels, the
 * same bits). The tile counters, the own chunk's row-group words and the wait record live in a
 * static device array of FO_NOALLOC_SCRATCH_BYTES that every device holds until the process
 * ends, instead of in memory the library allocates; the call allocates nothing and calls no
 * allocating routine (its first call on a device looks the array up and reads two device
 * attributes). Arguments as for fo_gemm_rs; opts: order, tile, row_groups, spin_timeout_us and
 * kernel_events are used, arrival must be DEFAULT or NONE (else FO_ERR_INVALID_ARG). Each call
 * first clears the counters and words it uses with a small kernel on compute_stream (no
 * hipMemsetAsync), then launches the GEMM there. All calls on a device share its array: calls
 * that overlap on one device (on two streams with no ordering between them) race on it and give
 * unspecified results; order them on one stream or with events. A call needing more scratch
 * than the array holds returns FO_ERR_UNSUPPORTED (P <= FO_MAX_P always fits). Waits that run
 * past their bound are reported by fo_check() like those of the other calls.
 */
fo_status fo_gemm_rs_noalloc(const void* x_shard, const void* w, float* send_buf, float* out,
                             float* recv_buf, int32_t P, int32_t rank, int64_t m, int64_t K,
                             int64_t N, int32_t in_dt, void* compute_stream, const fo_opts* opts);

/*
 * Plain monolithic GEMM C[M, N] = A[M, K] . B[K, N] with the same kernels (no slices, no waits):
 * the "pure GEMM" latency the overlap is measured against, and the unsliced product that the
 * page's exactness claim compares to. tile: a fo_tile value (AUTO = the choice fo_ag_gemm would
 * make for a single slice of M rows).
 */
fo_status fo_gemm_ref(const void* a, const void* b, void* c, int64_t M, int64_t K, int64_t N,
                      int32_t in_dt, int32_t out_dt, int32_t tile, void* stream);

/*
 * The activation of the MLP block between fo_ag_gemm (gate+up projection) and fo_gemm_rs (down
 * projection): h[r, j] = silu(y[r, j]) * y[r, inter + j] with silu(g) = g / (1 + e^-g), for
 * r < rows, j < inter. The FlashOverlap page measures its MLP-layer latency (technical summary
 * section 4) on the block these three make; for the Llama-3.1 shapes of the workloads the
 * activation is SwiGLU.
 *   y  device [rows, 2*inter] bf16: the gate+up output, gate in columns [0, inter) and up in
 *      [inter, 2*inter) (a plain concatenation of the two projections).
 *   h  device [rows, inter] bf16, not overlapping y.
 * fp32 arithmetic and one round-to-nearest-even to bf16. inter must be a multiple of 8 and both
 * pointers 16-byte aligned (else FO_ERR_INVALID_ARG, nothing enqueued). Enqueued on `stream`
 * (hipStream_t), ordered only by that stream.
 */
fo_status fo_swiglu(const void* y, void* h, int64_t rows, int64_t inter, void* stream);

/*
 * Query-split attention between the two All-to-Alls of Ulysses (sequence) parallelism, both
 * decomposed into point-to-point transfers: one rank's share. The FlashOverlap page (gist.science
 * paper 2604.24013, technical summary section 2 "Methodology") applies its sliced overlap to
 * attention by query slices and to the All-to-All of Ulysses parallelism. After the first
 * All-to-All, rank `rank` holds, for its own hq query heads and hkv key/value heads, the rows of
 * every peer's sequence chunk: slice s is the m tokens at sequence positions s*m .. s*m+m-1.
 * Slice `rank` is local; slice s != rank is copied from qkv_peer[s] into qkv_recv (emulated
 * arrival, in the Flash-AG arrival order). The attention runs by query slices: the work for the
 * queries of slice s starts once slice s has landed and reads key slices in arrival order as
 * each one lands (with causal masking only slices j <= s). Per head h (key head h / (hq / hkv))
 * and query position i:
 *     out[i, h] = sum_j softmax_j(q_i . k_j / sqrt(head_dim)) v_j, over key positions j (j <= i
 *     when causal).
 * The second All-to-All returns each query slice's output rows (this rank's heads) to the rank
 * that owns those positions: with out_peer given, the rows of slice s != rank are copied to
 * out_peer[s] as soon as every work item of a row group of slice s (the groups it arrived in)
 * has stored them, while the later work computes; in the FLASH order the own slice, whose rows
 * stay, is dispatched last (the Flash-RS order applied to the outgoing exchange). The call ends
 * when every sent row has landed. Under causal masking the work items (slice, 128-query tile,
 * head) differ in length up to P*m/64 key tiles; the workgroups (two per CU) then take lists
 * that give every CU the same work, the longest items cut in two along their keys and the two
 * halves combined in a fixed order (the same bits whichever half ends last), and the dispatch
 * order above no longer applies.
 *   qkv_local  device [m, (hq + 2*hkv) * head_dim] bf16: one row per token, [hq query heads |
 *              hkv key heads | hkv value heads], each head_dim values.
 *   qkv_peer   host array of P device pointers (entry [rank] ignored), each [m, row] like
 *              qkv_local; NULL = the slices are already in qkv_recv (no arrivals).
 *   qkv_recv   device [P*m, row] bf16; slice s at rows s*m (the rows of slice `rank` unused).
 *   out        device [P*m, hq * head_dim] bf16: row i is query position i, heads side by side.
 *   out_peer   host array of P device pointers (entry [rank] ignored), each [m, hq * head_dim]
 *              bf16, not overlapping out, the inputs or one another: out_peer[s] stands for
 *              rank s's receive buffer and gets out's rows s*m .. s*m+m-1. NULL = no return
 *              exchange. Needs 2*P <= FO_MAX_P (else FO_ERR_UNSUPPORTED).
 * Computed in fp32 (bf16 MFMA products, fp32 sums, fp32 softmax in base 2); the probabilities
 * enter the value product as bf16; one round to nearest even of the output.
 * head_dim must be 128 (else FO_ERR_UNSUPPORTED); hq a multiple of hkv; causal 0 or 1; every
 * pointer 16-byte aligned; out must not overlap an input (else FO_ERR_INVALID_ARG, nothing
 * enqueued). opts: order (FLASH: local slice first, then rank-1, rank-2, ...; NATURAL: index
 * order, own slice included, for the data-slicing baseline), arrival (NONE, EAGER or DEFAULT =
 * EAGER), links, row_groups (each slice sent in that many row groups, group by group, of a
 * whole number of 128-row query tiles, both ways; 0 = whole slices), spin_timeout_us and
 * kernel_events are used: a query tile waits for the group holding its rows, and the walk over a
 * key slice for the groups holding the keys it reads. tile must be AUTO, epilogue NONE.
 * Enqueued on compute_stream like fo_ag_gemm, with the same ordering, timeout and error
 * reporting through fo_check.
 */
fo_status fo_attn(const void* qkv_local, const void* const* qkv_peer, void* qkv_recv, void* out,
                  void* const* out_peer, int32_t P, int32_t rank, int64_t m, int32_t hq,
                  int32_t hkv, int32_t head_dim, int32_t causal, void* compute_stream,
                  const fo_opts* opts);

/*
 * The same attention with every slice resident (one sequence of S tokens, no transfers): the
 * pure-attention latency of the exposed-transfer fraction and the unsliced result of the
 * exactness check. qkv [S, (hq + 2*hkv) * head_dim] bf16, out [S, hq * head_dim] bf16; the
 * checks of fo_attn apply. Enqueued on `stream`; a causal call cuts long items in two like
 * fo_attn and keeps their halves in the device's buffers, so it is also ordered after the
 * device's previous call as fo_attn is.
 */
fo_status fo_attn_ref(const void* qkv, void* out, int64_t S, int32_t hq, int32_t hkv,
                      int32_t head_dim, int32_t causal, void* stream);

/*
 * The emulated transfers of one fo_ag_gemm (kind 0) or fo_gemm_rs (kind 1) call on their own,
 * without the GEMM: the same copies, links and arrival order (RS releases are not awaited). On
 * `stream` it enqueues the release of the copies and a one-workgroup kernel that waits until all
 * of them have landed, so the stream's time from the release to that kernel's end is the transfer
 * time of the exposed-transfer fraction (sliced latency minus pure-GEMM latency, over transfer
 * time).
 *   src    host array of P device pointers; src[s] is slice s (slice_bytes bytes). Entry [rank]
 *          is ignored.
 *   dst    device buffer of P*slice_bytes bytes; slice s lands at dst + s*slice_bytes.
 * opts: order, links, row_groups (each slice cut into that many equal pieces, issued group by
 * group like the calls; 0 = whole slices) and spin_timeout_us are used. slice_bytes must be a
 * multiple of 4.
 */
fo_status fo_transfer_ref(int32_t kind, const void* const* src, void* dst, int32_t P,
                          int32_t rank, int64_t slice_bytes, void* stream, const fo_opts* opts);

/* Synchronizes `stream` (hipStream_t), waits (on the host, at most 30 s) until every transfer the
   library issued on the current device has landed, and reports what happened since the previous
   fo_check in any call on the device (fo_gemm_rs_noalloc's included): FO_ERR_TIMEOUT if an
   in-kernel wait ran past its bound or a transfer did not land in time, FO_ERR_HIP if a DMA
   engine reported a failed copy. The record is then cleared. */
fo_status fo_check(void* stream);

/* Host-side slice scheduler. kind 0 = AG, 1 = RS; order a fo_order. Writes P slice/chunk ids in
   computation order to out[0..P-1]. */
fo_status fo_slice_order(int32_t kind, int32_t order, int32_t P, int32_t rank, int32_t* out);

/* The tile shape the bf16 kernel would use for slices of m rows, K, N with output out_dt (fp32 for
   fo_gemm_rs) and the tile request `tile` (a fo_tile). Writes the tile rows/columns and the
   number of tile workgroups one call over P slices launches (a fo_gemm_rs launch may append
   workgroups that add the partials after them). */
fo_status fo_tile_info(int32_t P, int64_t m, int64_t K, int64_t N, int32_t in_dt, int32_t out_dt,
                       int32_t tile, int32_t* bm, int32_t* bn, int64_t* workgroups);

/* The dispatch order of one fo_ag_gemm (kind 0) or fo_gemm_rs (kind 1) launch for these sizes,
   output dtype (fo_gemm_rs always writes fp32) and options (order, tile, row_groups are used):
   workgroup u computes position out[4u], row group
   out[4u+1], tile row out[4u+2] and tile column out[4u+3] of that position. Writes the first
   min(capacity, count) workgroups; *count receives the number of workgroups. */
fo_status fo_tile_order(int32_t kind, int32_t P, int64_t m, int64_t K, int64_t N, int32_t in_dt,
                        int32_t out_dt, const fo_opts* opts, int32_t* out, int64_t capacity,
                        int64_t* count);

/* The work lists of a causal fo_attn / fo_attn_ref launch for P slices of m tokens, hq query heads
   and n_cu CUs (host only, no device needed): entry k (in launch order) is out[5k] = the
   workgroup that takes it, out[5k+1] = slice, out[5k+2] = 128-query tile, out[5k+3] = head and
   out[5k+4] = -1 for a whole item, else 2 * pair + part for one of the two halves (the first or
   the second half of its key walk) of a split item. Workgroup b takes its entries in order;
   workgroups b and b + n_cu share a CU. Writes the first min(capacity, count) entries; *count
   receives the number of entries, *workgroups the number of workgroups (0 and 0: the shape has
   no table and the launch takes one workgroup per item). */
fo_status fo_attn_schedule(int32_t P, int64_t m, int32_t hq, int32_t n_cu, int32_t* out,
                           int64_t capacity, int64_t* count, int32_t* workgroups);

const char* fo_status_str(fo_status s);
/* Detail of the last failure on the calling thread (empty string if none). */
const char* fo_last_error(void);
int32_t fo_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASHOVL_H */
