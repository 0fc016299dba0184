/*
 * fedavg.h -- C ABI of the MI355X FedAvg aggregation library (libfedavg.so).
 *
 * Server-side federated averaging: the server combines the models (or model
 * deltas) sent by K clients into one global model, weighting client k by its
 * sample count n_k.  For every parameter i
 *
 *     out_i = sum_{k in C_i} n_k * x_{k,i} / W_i           (FA_WEIGHTS)
 *     out_i = base_i + sum_{k in C_i} n_k * d_{k,i} / W_i  (FA_DELTAS)
 *     W_i   = sum_{k in C_i} n_k
 *
 * where C_i is the set of clients with n_k > 0 that sent parameter i.  A
 * parameter that no such client sent keeps its global value: out_i = base_i.
 *
 * Sources of the definition:
 *   - plain or contribution-weighted averaging of the clients' models by the
 *     server: "NVIDIA Clara implements federated learning" (epnc.co.kr),
 *     introduction and section "Server-side workflow" (weighted aggregation
 *     algorithm);  n_k is the per-round sample count each participant reports
 *     (gist.science summary of the measurement-based adaptive data
 *     partitioning paper, section "The adaptive controller");
 *   - component-level updates averaged over the clients that sent them, and
 *     adapter-only federation: "Building Federated Multimodal AI Workflows with
 *     NVIDIA FLARE" (ai-thai.com), sections "Client Update Contract" and the
 *     FedUMM example;
 *   - partial sharing, each client choosing the fraction of its update it
 *     sends: the Clara page, introduction and section "Client-side workflow";
 *   - streamed, chunk-at-a-time transfer with a tunable chunk size, and server
 *     memory that must not grow linearly with the number of clients: the FLARE
 *     page, sections on tensor streaming (Tensor Downloader) and "Offload
 *     Aggregation to Disk" (Tensor Disk Offload);
 *   - fp32 master weights, round-to-nearest-even (never stochastic rounding)
 *     for weights: "NVFP4 training with JAX and MaxText" (ai-thai.com),
 *     training-recipe section and the linear-layer data-flow figure.
 *
 * Arithmetic contract.  Accumulation is fp32 with one fused multiply-add per
 * contributing client, in client order (resident lists: list order; streaming:
 * arrival order), starting from 0; then one IEEE division by fp32(W_i); then,
 * in delta mode, one fp32 addition of base_i; then round-to-nearest-even to
 * the output type.  Results are deterministic (no floating-point atomics), and
 * a streamed aggregation is bit-identical to the resident one over the same
 * clients in the same order.  NaN/Inf in a contributing client propagate;
 * fp32 denormals are kept.
 *
 * Conventions for every call:
 *   - Return value: FA_OK (0) or a negative fa_status; the message of the most
 *     recent failure on the calling thread is available from
 *     fedavg_last_error().  No C++ exception crosses the ABI.
 *   - Argument errors are detected and returned before any device work is
 *     enqueued.  Device work is asynchronous on the stream(s) given (a
 *     hipStream_t passed as void*; NULL is the default stream).
 *   - The caller owns every device buffer, pinned host buffer and stream.
 *     Only the streaming handle (host memory and its HIP events, plus one
 *     internal copy stream when the caller passes none) belongs to the
 *     library; fedavg_destroy releases it.
 *   - Threads: the resident calls may run on several threads at once, each
 *     on its own buffers.  A streaming handle is used by one thread at a
 *     time (its calls update host-side coverage and staging slots).
 *   - Limits: K <= FA_MAX_CLIENTS resident clients per call;
 *     0 <= n_k <= FA_MAX_WEIGHT (so fp32(n_k) is exact); sums of weights
 *     below 2^32; at most FA_MAX_N parameters per buffer and chunk_bytes at
 *     most FA_MAX_N (FA_ERR_RANGE beyond: no byte count can overflow).
 *   - Aliasing: `out` may be the same buffer as `base` or as one client input
 *     (every element is read before it is written); partial overlap is not
 *     allowed.
 *   - Alignment: 16-byte aligned buffers take the vector path; others a
 *     slower element-wise path with identical results.
 */
#ifndef FEDAVG_H
#define FEDAVG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FEDAVG_ABI_VERSION 1
#define FA_MAX_CLIENTS 64
#define FA_MAX_WEIGHT (1 << 24)
#define FA_MAX_STREAM_CLIENTS 255
#define FA_MAX_N (1ll << 40)

typedef enum {
    FA_OK = 0,
    FA_ERR_ARG = -1,         /* bad pointer, size, count or combination */
    FA_ERR_DTYPE = -2,       /* unsupported element type */
    FA_ERR_RANGE = -3,       /* a limit above is exceeded */
    FA_ERR_ZERO_WEIGHT = -4, /* dense weights mode with sum of n_k == 0 */
    FA_ERR_STATE = -5,       /* streaming call out of order */
    FA_ERR_INCOMPLETE = -6,  /* dense streaming: a client did not cover [0,N) */
    FA_ERR_INDEX = -7,       /* unsorted, duplicate or out-of-range index */
    FA_ERR_WORKSPACE = -8,   /* workspace missing or too small */
    FA_ERR_HIP = -9          /* HIP runtime error */
} fa_status;

typedef enum { FA_F32 = 0, FA_BF16 = 1 } fa_dtype;
/*
 * FA_WEIGHTS: clients send weights; out_i = sum n_k x_k / W_i.
 * FA_DELTAS:  clients send deltas;  out_i = base_i + sum n_k d_k / W_i.
 * FA_DELTAS_ZERO_FILL: clients send deltas and a parameter a client did not
 *     send counts as a zero delta from it: out_i = base_i + sum n_k d_k / S,
 *     S = sum of n_k over every client with n_k > 0 (in streaming: every
 *     client accumulated so far, merged partials by their W).  A parameter no
 *     client sent keeps base_i exactly.  With every client sending every
 *     parameter this equals FA_DELTAS.  This is the other reading of
 *     averaging partially shared updates (Clara page, client-side workflow:
 *     each client sends a fraction of its update); the divisor is fp32(S).
 */
typedef enum { FA_WEIGHTS = 0, FA_DELTAS = 1, FA_DELTAS_ZERO_FILL = 2 } fa_mode;
typedef enum { FA_COUNT_U8 = 0, FA_COUNT_U32 = 1 } fa_count_dtype;

/* FEDAVG_ABI_VERSION of the loaded library. */
int fedavg_abi_version(void);

/* Message of the last failed call on this thread ("" if none). The pointer
   stays valid until the next call on this thread. */
const char *fedavg_last_error(void);

/*
 * fedavg_aggregate -- resident K-client aggregation in one pass over HBM.
 *
 * x        host array of K device pointers; x[k] holds N elements of x_dtype
 *          (client models in FA_WEIGHTS mode, client deltas in FA_DELTAS).
 * n        host array of K sample counts.  n_k == 0: client k is skipped and
 *          x[k] is never read (it may be NULL).
 * N        parameters per client (N == 0 is a no-op; every pointer may then
 *          be NULL).
 * base     device, N elements of base_dtype.  Required in FA_DELTAS mode and
 *          whenever T > 0; unused in dense FA_WEIGHTS mode (may be NULL).
 * out      device, N elements of out_dtype.
 * T        0: dense -- every client sent every parameter (FA_WEIGHTS then
 *          needs sum n_k > 0, else FA_ERR_ZERO_WEIGHT).
 *          T > 0: per-segment (per-tensor) masks, for adapter-only or
 *          partially shared updates: parameters are split into T contiguous
 *          segments and client k sent segment t iff present[k*T + t] != 0.
 *          Segments no client sent are never read and copy base.
 * seg_bounds device int64[T+1]: seg_bounds[0] = 0, nondecreasing,
 *          seg_bounds[T] = N; segment t is [seg_bounds[t], seg_bounds[t+1]).
 *          Device data is not validated on the host; a malformed table gives
 *          unspecified values but every access stays inside the buffers.
 * present  device uint8[K*T], row-major by client.
 * stream   hipStream_t the work is enqueued on.
 * Traffic: one read of every element of every contributing (segment of a)
 * client, one write of out, plus base where it is used.
 */
int fedavg_aggregate(int K, const void *const *x, fa_dtype x_dtype, const int64_t *n, int64_t N,
                     fa_mode mode, const void *base, fa_dtype base_dtype, void *out,
                     fa_dtype out_dtype, int T, const int64_t *seg_bounds, const uint8_t *present,
                     void *stream);

/*
 * fedavg_arena_layout -- where to put the buffers of one resident
 * aggregation (the K client updates the server holds for a round, Clara
 * page, section "Server-side workflow", and the output) inside a single
 * device allocation that the caller makes.  The dense pass reads the same
 * parameter of every client at the same moment; buffers from separate
 * allocations start at the same position within a 2 MiB page, so those
 * addresses share their low 21 bits.  Here buffer j starts at
 *     offsets[j] = j * (round_up(bytes, 2 MiB) + 32 KiB),
 * that is 32 KiB further into its page than buffer j - 1 (modulo 2 MiB).
 * Measured on MI355X with 16 bf16 clients of 1.92e9 parameters and the
 * output: about 5% faster than separate allocations, on every allocation
 * tried; with 8 or 32 clients the two were within their run-to-run spread.
 * count        buffers, 1 to FA_ARENA_MAX_BUFFERS.
 * bytes        bytes per buffer, >= 0.
 * offsets      host int64[count], written (multiples of 32 KiB: every buffer
 *              is 16-byte aligned when the allocation is).
 * total_bytes  host, written: the allocation's size, offsets[count-1] + bytes.
 * Host only, no device work and no allocation.  FA_ERR_ARG for a count out of
 * range, a negative size or a NULL pointer; FA_ERR_RANGE when the total would
 * exceed 2^62 bytes.
 */
#define FA_ARENA_MAX_BUFFERS 4096
int fedavg_arena_layout(int count, int64_t bytes, int64_t *offsets, int64_t *total_bytes);

/* ------------------------------------------------------------------------
 * Streaming: clients arrive one after another, each as chunks, into one
 * resident fp32 accumulator, so device memory does not grow with K.
 * ------------------------------------------------------------------------ */
typedef struct fa_stream_state *fa_handle;

/*
 * fedavg_workspace_size -- device bytes the caller must provide.
 * partial      0: dense (every client covers [0,N) exactly once);
 *              1: partial (clients send ranges, masked ranges or index lists;
 *                 each parameter is averaged over the clients that sent it).
 * chunk_bytes  largest chunk payload per call (values), > 0.
 * n_slots      staging slots for host-resident chunks (1 to 64; 2 or more lets
 *              the next copy overlap the current accumulate).
 * acc_bytes    N fp32;  wsum_bytes  N uint32 (partial only, else 0);
 * count_bytes  N uint8 (partial only, else 0);
 * staging_bytes per-slot staging plus a small header (error flag).
 */
int fedavg_workspace_size(int64_t N, int partial, int64_t chunk_bytes, int n_slots,
                          size_t *acc_bytes, size_t *wsum_bytes, size_t *count_bytes,
                          size_t *staging_bytes);

/*
 * fedavg_begin -- start an aggregation; zeroes acc (and wsum, count) on
 * compute_stream.
 * acc, wsum, count, staging: caller device buffers of at least the sizes from
 *     fedavg_workspace_size (wsum/count only in partial mode; count may be
 *     NULL in partial mode when per-parameter client counts are not wanted).
 * compute_stream: where accumulate and finalize kernels run.  The buffers are
 *     taken in this stream's order: work queued on it before the call may
 *     still write them (the copies into staging wait for that work too).
 * copy_stream: where host-to-device chunk copies run (NULL: the handle creates
 *     its own stream).  Copies and kernels are ordered with HIP events.
 */
int fedavg_begin(fa_handle *h, int64_t N, fa_mode mode, int partial, float *acc, uint32_t *wsum,
                 uint8_t *count, void *staging, size_t staging_bytes, int64_t chunk_bytes,
                 int n_slots, void *compute_stream, void *copy_stream);

/*
 * fedavg_accumulate -- add one chunk of one client: acc[i] += n_k * value_i
 * for every parameter i the chunk carries (and, in partial mode,
 * wsum[i] += n_k, count[i] += 1).
 *
 * client_id   caller's id of the client (>= 0); a client keeps one n_k.
 * n_k         the client's sample count; n_k == 0 returns FA_OK, no work.
 * chunk       pinned host memory (staged with hipMemcpyAsync on the copy
 *             stream) or device memory (read in place).  Pageable host memory
 *             is rejected with FA_ERR_ARG.
 * offset,len  without mask/indices: the chunk holds parameters
 *             [offset, offset+len); a range reaching past N (tested without
 *             forming offset+len, so huge values cannot wrap) is
 *             FA_ERR_RANGE.  Dense mode: each client's chunks must arrive in
 *             ascending order and tile [0,N) exactly.  Partial mode: a
 *             client's ranges must be ascending and non-overlapping.
 * mask        partial mode only, nullable: len bytes, nonzero = sent.
 * indices     partial mode only, nullable: len strictly increasing int64
 *             indices relative to offset (parameter offset+indices[j] gets
 *             value j).  Violations are detected on the device and reported
 *             by fedavg_sync as FA_ERR_INDEX; the bad entries are skipped.
 *             The caller must not send one parameter twice for a client.
 *             A list dense enough (FA_OPT_INDEX_TILES) is checked first and
 *             then applied by reading and writing the accumulator's
 *             2048-parameter tiles that hold it (a device word in the
 *             staging header carries the check's verdict); other lists, and
 *             lists the check refuses, are scattered.  Both give the same
 *             bits.
 *             mask and indices live where chunk lives.
 * An empty chunk (len == 0) enters the client but carries no parameter, so
 * the ordering and tiling rules above do not apply to it.
 * A host buffer passed here may be reused once n_slots further calls of
 * fedavg_accumulate or fedavg_accumulate_partial on this handle have
 * returned -- calls of every kind count: device or empty chunks, n_k == 0,
 * refused calls -- or after fedavg_sync.  (Each call waits, if need be, for
 * the host-to-device copy of the call n_slots before it.)
 */
int fedavg_accumulate(fa_handle h, int client_id, int64_t n_k, const void *chunk, fa_dtype dtype,
                      int64_t offset, int64_t len, const uint8_t *mask, const int64_t *indices);

/*
 * fedavg_accumulate_partial -- two-level (hierarchical) aggregation: add the
 * unnormalised partial sums of a lower-level aggregation as one pseudo-client
 * of h.  The regime this serves groups devices into fixed silos that
 * aggregate inside and whose models are then aggregated at the federated
 * round boundary (HFL-DDP: gist.science summary of the measurement-based
 * adaptive data partitioning paper, section "Execution regimes").  Regrouping
 * the sum makes this equal, in exact arithmetic, to aggregating all the
 * silos' clients in one flat pass:
 *     sum_s sum_{k in s} n_k x_k / sum_s W_s,   W_s = sum_{k in s} n_k.
 *
 * client_id  the pseudo-client's id in h (>= 0); it keeps one W and
 *            n_clients, and follows a client's range rules (dense mode: its
 *            calls arrive in ascending order and tile [0,N) exactly; partial
 *            mode: ascending, non-overlapping ranges).
 * W          the silo's total weight (fedavg_partial_info of the silo's
 *            handle), in [0, 2^32); W == 0 returns FA_OK, no work.  It enters
 *            the dense divisor S the way a client's n_k does.
 * n_clients  clients behind the partial, in [1, 255]; in partial mode the
 *            handle's clients, counted this way, stay at most 255.
 * acc_src    float[len]: the silo's sums over parameters [offset, offset+len),
 *            i.e. its accumulator after fedavg_sync and before (or after)
 *            its finalize.
 * wsum_src   uint32[len], required when h is in partial mode (the silo's
 *            per-parameter weight sums); ignored otherwise.
 * count_src  uint8[len], required when h has a count buffer; else ignored.
 * Residence: all device, or all pinned host (staged like chunks; then 4*len
 * must not exceed chunk_bytes).  Pageable host memory: FA_ERR_ARG.
 * Arithmetic: acc_i = acc_i + acc_src_i, one IEEE fp32 addition (RNE); the
 * weight sums and counts add exactly.  The silo's own order of FMAs is kept
 * inside acc_src; partials enter in call order.
 */
int fedavg_accumulate_partial(fa_handle h, int client_id, int64_t W, int n_clients,
                              const float *acc_src, const uint32_t *wsum_src,
                              const uint8_t *count_src, int64_t offset, int64_t len);

/* Total weight (sum of the clients' n_k and the partials' W) and number of
   clients (a partial counts n_clients) accumulated so far in h.  Either
   output pointer may be NULL. */
int fedavg_partial_info(fa_handle h, int64_t *W, int *n_clients);

/*
 * fedavg_finalize -- out_i = base_i + acc_i / W_i (FA_DELTAS) or acc_i / W_i
 * (FA_WEIGHTS), W_i = sum of n_k (dense) or wsum_i (partial); parameters with
 * W_i == 0 copy base_i.  base (device, N of base_dtype) is required in
 * FA_DELTAS and partial modes when N > 0; out may alias base.  Dense mode returns
 * FA_ERR_INCOMPLETE if some client has not covered [0,N).  The accumulator is
 * left intact, so finalize may be repeated; no accumulate may follow a
 * successful finalize (FA_ERR_STATE).  A finalize refused by its checks
 * (FA_ERR_ARG, FA_ERR_DTYPE, FA_ERR_INCOMPLETE, FA_ERR_ZERO_WEIGHT) leaves the
 * handle as it was.
 */
int fedavg_finalize(fa_handle h, const void *base, fa_dtype base_dtype, void *out,
                    fa_dtype out_dtype);

/*
 * Spill and resume.  Server memory must not have to hold every client's
 * update at once, and partial aggregation state may live on disk between
 * uses (FLARE page, section "Offload Aggregation to Disk": incoming updates
 * go to temporary files and are read back when needed).  Here the running
 * aggregate is the whole state: the caller's acc (and wsum, count) buffers
 * plus the handle's host-side record -- mode, N, and per client its id,
 * weight, coverage and client count.
 *
 * fedavg_state_size   bytes fedavg_export_state writes for h now.
 * fedavg_export_state waits for h's work (as fedavg_sync, returning
 *                     FA_ERR_INDEX if a deferred index error was raised,
 *                     without writing), then writes the host-side record to
 *                     buf (host memory, at least fedavg_state_size bytes).  The
 *                     caller then copies acc/wsum/count out (e.g. to disk) and
 *                     may destroy h and free the device buffers.
 * fedavg_resume       opens a handle like fedavg_begin, except that acc, wsum
 *                     and count are NOT cleared: the caller has restored them
 *                     bit for bit from the export, and the client record comes
 *                     from state.  Accumulating on and finalizing then gives
 *                     exactly the bits an uninterrupted run gives.  The state
 *                     is checked (format, version, checksum, limits) before
 *                     anything is created: FA_ERR_ARG when it fails.  count
 *                     must be non-NULL exactly when the exported handle kept
 *                     client counts.  chunk_bytes, n_slots and the streams may
 *                     differ from the exporting handle's; N, mode and
 *                     partial must equal the exported ones (they size the
 *                     caller's buffers), else FA_ERR_ARG.
 * The record is versioned, little-endian and ends with a 64-bit FNV-1a
 * checksum of its bytes.
 */
int fedavg_state_size(fa_handle h, size_t *bytes);
int fedavg_export_state(fa_handle h, void *buf, size_t bytes);
int fedavg_resume(fa_handle *h, const void *state, size_t state_bytes, int64_t N, fa_mode mode,
                  int partial, float *acc, uint32_t *wsum, uint8_t *count, void *staging,
                  size_t staging_bytes, int64_t chunk_bytes, int n_slots, void *compute_stream,
                  void *copy_stream);

/* Wait for all work of the handle; returns a deferred device error
   (FA_ERR_INDEX) if one was raised, else FA_OK. */
int fedavg_sync(fa_handle h);

/* Wait for the handle's work, then release its host state and events. */
int fedavg_destroy(fa_handle h);

/* ------------------------------------------------------------------------
 * Resident sparse partial sharing.
 * ------------------------------------------------------------------------ */

/* Device workspace bytes sparse_masked_accumulate needs for K clients, N. */
int sparse_workspace_size(int K, int64_t N, size_t *bytes);

/*
 * sparse_masked_accumulate -- K clients each send a sorted list of
 * (index, value) pairs, e.g. the top p% of their |delta| (partial sharing,
 * Clara page, introduction and client-side workflow).  One pass:
 *     count_i = |C_i|, W_i = sum_{k in C_i} n_k,
 *     out_i   = W_i > 0 ? base_i + sum_{k in C_i} n_k v_{k,i} / W_i : base_i
 * (FA_DELTAS; FA_WEIGHTS drops base_i from the first branch), accumulating
 * client by client in list order.
 *
 * idx, val   host arrays of K device pointers: nnz[k] int64 indices, strictly
 *            increasing, in [0,N), and nnz[k] fp32 values (SoA layout).
 * nnz, n     host arrays of K (nnz[k] >= 0; n_k as for fedavg_aggregate).
 * base, out  device fp32[N]; out may alias base.
 * counts     device, N of counts_dtype (nullable): per-parameter client count.
 * wsum       device uint32[N] (nullable): per-parameter weight sum W_i.
 * workspace  device, >= sparse_workspace_size bytes (may be NULL when
 *            N == 0).
 * err_flag   device int (nullable): set to 0 by this call, then to
 *            FA_ERR_INDEX if some list is unsorted, has duplicates or an
 *            index outside [0,N) (those entries are skipped).
 */
int sparse_masked_accumulate(int K, const int64_t *const *idx, const float *const *val,
                             const int64_t *nnz, const int64_t *n, int64_t N, fa_mode mode,
                             const float *base, float *out, void *counts,
                             fa_count_dtype counts_dtype, uint32_t *wsum, void *workspace,
                             size_t workspace_bytes, int *err_flag, void *stream);

/*
 * sparse_masked_accumulate_noalloc -- for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.  The same merge, results and arguments
 * as sparse_masked_accumulate, without the workspace: the list offsets
 * (and the error flag when err_flag is NULL) live in a static device array
 * of FA_SPARSE_SCRATCH_BYTES per GPU, held until the process ends.  The
 * call allocates and frees nothing.  It needs 256 + 8 * Kc * (ranges + 1)
 * bytes of that array, Kc the clients with n_k > 0 and nnz > 0 and ranges
 * the parameter ranges the merge uses (by default N / 8192 for N beyond
 * about 3.4e7, 122,071 at N = 10^9, so up to 34 clients there; at most
 * 2^19, which every N admits for Kc <= 7);
 * beyond FA_SPARSE_SCRATCH_BYTES it returns FA_ERR_RANGE before any device
 * work.  All calls on one GPU share its array: calls that overlap in time
 * on one GPU (other streams, other threads) race on it and must be
 * serialized by the caller.  The flag is reset by each call; the offsets
 * are rewritten by each call before they are read.
 */
#define FA_SPARSE_SCRATCH_BYTES (32ll << 20)
int sparse_masked_accumulate_noalloc(int K, const int64_t *const *idx, const float *const *val,
                                     const int64_t *nnz, const int64_t *n, int64_t N, fa_mode mode,
                                     const float *base, float *out, void *counts,
                                     fa_count_dtype counts_dtype, uint32_t *wsum, int *err_flag,
                                     void *stream);

/* ------------------------------------------------------------------------
 * Per-round sample counts (host only, no device work).
 * ------------------------------------------------------------------------ */

typedef struct {
    double w_time;   /* weight of the time cost, >= 0 */
    double w_energy; /* weight of the energy cost, >= 0 (not both 0) */
    double ema;      /* smoothing: s <- ema * x + (1 - ema) * s, in (0, 1] */
    double deadband; /* keep the current counts when no count would change by
                        more than this fraction of itself, >= 0 */
} fa_controller;

/*
 * fedavg_controller_step -- the n_k of the next round from this round's
 * measurements, after the measurement-based adaptive controller (gist.science
 * summary of the adaptive data partitioning paper, section "The adaptive
 * controller"): per-sample costs tau_i = t_i / n_i and eps_i = e_i / n_i,
 * smoothed by an exponential moving average; a combined cost
 *     c_i = w_time * tau_i / median(tau) + w_energy * eps_i / median(eps)
 * (a term with weight 0 is left out; the median of an even count is the mean
 * of the middle two); samples in inverse proportion to c_i.  These n_k are the
 * FedAvg weights of the next round.
 * P participants; t, e: their time and energy this round (>= 0); n: their
 * counts this round (> 0); total: samples to hand out (>= P).
 * tau_state, eps_state: the smoothed costs, P doubles each, read unless
 * first_round and always written back.
 * n_next (P): largest-remainder integers summing to total (ties to the lower
 * index), at least 1 each (taken from the largest count, lowest index) so
 * every cost stays measurable; but if total equals the current sum and no
 * count would move by more than deadband * n_i, n_next = n.
 * All arithmetic is IEEE binary64 in the order written.  Errors: FA_ERR_ARG
 * (bad pointer, value or a zero median), FA_ERR_RANGE (total < P).
 */
int fedavg_controller_step(int P, const double *t, const double *e, const int64_t *n,
                           int64_t total, const fa_controller *c, double *tau_state,
                           double *eps_state, int first_round, int64_t *n_next);

/* ------------------------------------------------------------------------
 * Client-side top-k selection (partial sharing).
 * ------------------------------------------------------------------------ */

/* Device workspace bytes topk_select needs to keep k of N values of dtype
   (it grows with k: while k < N/3 for fp32, N/4 for bf16, it holds a
   staging copy of the entries near and above the threshold, 6 or 4 bytes
   each).  FA_ERR_RANGE unless 0 <= k <= N. */
int topk_workspace_size(fa_dtype dtype, int64_t N, int64_t k, size_t *bytes);

/*
 * topk_select -- the client's side of partial sharing: of its update x
 * (device, N values of dtype) keep the k entries of largest magnitude, the
 * fraction p of the update it chooses to send (k = floor(p*N); Clara page,
 * introduction and client-side workflow section).  Order: by the magnitude
 * bit pattern (the fp32 bits with the sign cleared; bf16 is widened to fp32
 * exactly) -- |x| order, with NaNs above infinity and -0 tied with +0; ties go
 * to the lower index.  The k kept indices are written to idx_out (device
 * int64[k]) in increasing order and their values, widened to fp32, to val_out
 * (device float[k]): exactly the per-client lists sparse_masked_accumulate
 * takes.  The result is unique, hence deterministic.
 * k == 0 returns FA_OK with no work; k > N or N > 2^36 is FA_ERR_RANGE.  workspace:
 * device, 16-byte aligned, topk_workspace_size(dtype, N, k) bytes,
 * overwritten.  Outputs must not overlap x.  Asynchronous on `stream`.
 * The threshold is bounded first from a sample of about 2^20 values, so that
 * the update is read once; when the bound fails (or FA_OPT_TOPK_SAMPLED is
 * 0) the call finishes with three passes over it instead, on the device and
 * with the same result.
 */
int topk_select(const void *x, fa_dtype dtype, int64_t N, int64_t k, int64_t *idx_out,
                float *val_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * fedavg_checksum -- order-independent checksum of a device buffer of `count`
 * elements: *hash_dev = sum over i of fmix64(i * 0x9E3779B97F4A7C15 XOR
 * bits_i) mod 2^64 (bits_i: the element's raw 16- or 32-bit pattern; fmix64:
 * the 64-bit finalizer of MurmurHash3).  Lets a caller compare large outputs
 * or chunks bit for bit without copying them back.  hash_dev: device uint64,
 * overwritten.
 */
int fedavg_checksum(const void *buf, int64_t count, fa_dtype dtype, uint64_t *hash_dev,
                    void *stream);

/*
 * fedavg_sum_workspace_size -- bytes of workspace fedavg_checksum_sum needs
 * for `count` elements: 8 per tile of 8192 elements (count/1024 bytes),
 * 0 for count == 0.  count > FA_MAX_N: FA_ERR_RANGE.
 *
 * fedavg_checksum_sum -- in one read of the buffer, the checksum above (when
 * hash_dev is not NULL) and a deterministic fp64 sum of the element values
 * into *sum_dev (device double, overwritten).  The additions run in an order
 * fixed by `count` alone: tiles of 8192 elements; in a tile, each of 256
 * threads adds its 32 elements (those of 16-byte vectors j, j + 256, ...)
 * in order from +0, then a butterfly over each wavefront and
 * (w0 + w1) + (w2 + w3) over the four; the tile sums are added by 1024
 * threads (thread j: sums j, j + 1024, ... in order), a butterfly, and a
 * pairwise tree over the 16 wavefronts.  So the result is the same bits on
 * every call and every launch shape.  It differs from the exact sum by at
 * most g * (sum of |x_i|), g = h * 2^-53 / (1 - h * 2^-53), where
 * h = 48 + ceil(T / 1024) is the longest chain of roundings for T tiles.
 * NaN, or infinities of both signs, give NaN; a zero sum is +0.  workspace:
 * device memory of fedavg_sum_workspace_size bytes, 8-byte aligned, holding
 * the tile sums.  The buffer, the workspace and the results must not overlap
 * (FA_ERR_ARG); a short workspace is FA_ERR_WORKSPACE.
 */
int fedavg_sum_workspace_size(int64_t count, size_t *bytes);
int fedavg_checksum_sum(const void *buf, int64_t count, fa_dtype dtype, uint64_t *hash_dev,
                        double *sum_dev, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Launch-shape options (process-wide, for tuning and measurement).  They
 * change how work is spread over the GPU, never the results.
 * ------------------------------------------------------------------------ */
typedef enum {
    FA_OPT_BLOCKS_PER_CU = 1,          /* cap on the grid of the streaming
                                          kernels, in workgroups per CU, each
                                          thread then striding over the data
                                          (default 0: no cap, one 8-parameter
                                          vector per thread) */
    FA_OPT_MASK_VECTORS_PER_BLOCK = 2, /* masked aggregate: 8-parameter vectors
                                          per workgroup, which sets the grid
                                          (default 2048) */
    FA_OPT_SPARSE_BLOCKS = 3,          /* sparse merge: parameter ranges, i.e.
                                          workgroups (default 0: ranges of 4
                                          tiles, but at least 4096 ranges while
                                          there are that many tiles, at most
                                          2^19; max 2^19) */
    FA_OPT_RESIDENT_PER_CU = 4,        /* resident dense kernel: workgroups of
                                          256 threads resident per CU (default
                                          -1: chosen by the number of
                                          contributing clients, 2 for 16;
                                          0 = hardware limit) */
    FA_OPT_SPARSE_TILE = 5,            /* sparse merge: parameters per LDS tile,
                                          512, 1024, 2048 (default), 4096 or
                                          8192 */
    FA_OPT_TOPK_SAMPLED = 6,           /* top-k: 1 (default) bounds the
                                          threshold from a sample first; 0
                                          always takes the three-pass path */
    FA_OPT_INDEX_TILES = 7             /* fedavg_accumulate with indices:
                                          0 (default) reads and writes the
                                          accumulator in dense tiles when the
                                          list holds at least 2^16 entries
                                          and one parameter in 16 of
                                          [offset, N), else scatters; 1
                                          always scatters; 2 always tiles.
                                          Tiles need N % 4 == 0 and 16-byte
                                          aligned sums and weight sums
                                          (4-byte aligned counts); otherwise
                                          the call scatters */
} fa_option;

/* Set one option; FA_ERR_ARG for an unknown option, FA_ERR_RANGE for a value
   outside the option's range.  Not thread-safe with concurrent launches. */
int fedavg_set_option(int option, int64_t value);

#ifdef __cplusplus
}
#endif

#endif /* FEDAVG_H */
