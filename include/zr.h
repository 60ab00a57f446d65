/*
 * zr.h - gradient-bucket reduction for data-parallel training, MI355X (gfx950).
 *
 * K data-parallel ranks are K buffers in one GPU's HBM. The library flattens
 * fragmented gradients into a flat bucket, reduce-scatters the bucket across
 * the K ranks in the ring's chunk order with fp32 accumulation, averages by
 * K and writes each rank's partition in one pass, gathers full parameters
 * back from 1/K shards, and composes the two into an all-reduce. A small
 * scheduler keeps the reduction on its own stream with per-buffer
 * completion events.
 *
 * Pages the operations follow (title, then section):
 *  [RING]  "图解 Ring All-Reduce：分布式训练梯度同步的核心算法": Phase 1
 *          (Scatter-Reduce) and Phase 2 (All-Gather).
 *  [L14]   CMU 11-868 lecture 14 notes, "Distributed Training I:
 *          Communication and Data Parallelism": 2.1 (every operation is bound
 *          to a stream), 2.2 (primitives; all-reduce = reduce-scatter +
 *          all-gather), 3.2 (ring rounds and placement), 4.1 (average =
 *          SUM / world size).
 *  [ZERO3] "DeepSpeed ZeRO-3 源码解析：前向与反向": 1 (data-flow overview:
 *          bucket -> reduce -> partition copy -> single bf16->fp32 cast),
 *          2.1/2.2 (parameter fetch and prefetch, its two caps and the
 *          limit on queued fetches), 2.4 (conservative release), 3.1/3.2
 *          (bucketing, contiguous flat buffer), 5.1-5.4 (bucket insert,
 *          reduce paths, partition write, epilogue).
 *  [ISSUE] "ZeRO-1/2 average_tensor serializes backward compute behind the
 *          preceding reduction" (DeepSpeed issue 8364): Proposed design
 *          direction (per-buffer reduction-complete events) and Validation
 *          requirements.
 *
 * Conventions for every call
 *  - Pointer tables (`in`, `out`, `shards`, ...) are HOST arrays of K DEVICE
 *    pointers; rank r's buffer is entry r. The library copies the tables
 *    into kernel arguments at launch; it keeps no reference after returning.
 *  - Sizes are element counts. bf16 data is raw 16-bit patterns.
 *  - Chunking: C = ceil(N / K); chunk j covers global indices [jC, jC + C)
 *    of every rank's buffer; indices >= N are zero padding.
 *  - chunk_shift s: after reduce-scatter rank q holds chunk (q + s) mod K,
 *    i.e. chunk j lands on rank (j - s) mod K. s = 1 is where the ring
 *    leaves each fully reduced chunk [RING Phase 1; L14 3.2]; s = 0 is the
 *    "rank r keeps slice r" convention of the contiguous path [ZERO3 5.2].
 *  - Ring order: chunk j is summed as (((x_j + x_{j+1}) + x_{j+2}) + ...
 *    + x_{j-1}) with ranks mod K, each input widened exactly to fp32, one
 *    fp32 round-to-nearest-even add per hop [RING Phase 1 rule].
 *  - Streams are hipStream_t passed as void*; NULL is the null stream. Work
 *    is enqueued asynchronously [L14 2.1]; buffers must stay alive until
 *    the stream has finished with them. No call allocates device memory.
 *  - Workspaces: the calls that take a table of fragments or segments
 *    (flatten, discrete reduce-scatter and its plans, all-gather) carry up
 *    to min(32, 256 / K) fragments (32 segments) per launch in kernel
 *    arguments; a larger table goes out as several launches, or, when the
 *    caller passes a device workspace (owned by the caller, at least
 *    zr_workspace_bytes(K, n) bytes, 8-byte aligned, not overlapping any
 *    buffer of the call), is copied into it and the whole call is one launch
 *    [ZERO3 3.1: one operation per bucket, not one per parameter]. A one-shot
 *    call copies its table with hipMemcpyAsync on `stream` from a host
 *    buffer, which HIP performs synchronously for pageable memory (the call
 *    returns once `stream` has reached the copy); a plan copies it once, at
 *    creation. Calls on one stream may share a workspace; calls on different
 *    streams that run at the same time must not. Under stream capture a
 *    one-shot call never records the copy: it goes out as argument launches
 *    (plans are created outside capture and may then be captured).
 *  - Errors: every call returns a zr_status; nothing throws or aborts across
 *    the boundary. Arguments are validated before any HIP call, so a bad
 *    argument enqueues nothing. zr_last_error() describes the last failure
 *    on the calling thread. N == 0 (or no work) returns ZR_OK and enqueues
 *    nothing.
 *  - Environment, read once, at the library's first launch or plan; for
 *    debugging and tests only. Ring-order results are bit-identical under
 *    every setting (ZR_ORDER_FREE results stay within their bound):
 *      ZR_DEBUG=1        every call waits for its stream after its launches
 *                        (not under stream capture), so an error a kernel
 *                        raises is returned, as ZR_ERR_HIP, by the call that
 *                        launched it;
 *      ZR_FORCE_PATH=element | small | large
 *                        element: the reduce-scatter, discrete reduce-scatter,
 *                        all-reduce and all-gather fold or copy element by
 *                        element even where their inputs allow 16-byte access
 *                        (the flatten has no such choice: its whole 16-byte
 *                        units always move as vectors); small: every ring-order
 *                        reduce-scatter uses one-slice tiles; large: none does;
 *                        other values are reported on stderr and ignored;
 *      ZR_MAX_GRID=n     at most n blocks per launch (default 2^30), the
 *                        blocks striding over the tiles beyond them.
 */
#ifndef ZR_H
#define ZR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ZR_OK = 0,
    ZR_ERR_INVALID = 1,     /* bad count, rank, shift, null pointer, state */
    ZR_ERR_ALIGN = 2,       /* pointer not aligned to its element size */
    ZR_ERR_ALIAS = 3,       /* overlapping buffers that must not overlap */
    ZR_ERR_UNSUPPORTED = 4, /* dtype or dtype pair not supported */
    ZR_ERR_WORKSPACE = 5,   /* workspace too small for the table it must hold */
    ZR_ERR_HIP = 6,         /* a HIP runtime call or launch failed */
    ZR_ERR_NOMEM = 7        /* host memory ran out, or a caller-provided arena
                               cannot hold what must be live */
} zr_status;

/* The _MIN_/_MAX_ enumerators make every int a value of the enum type in C
 * and C++ alike, so any int a caller passes is well defined; the library
 * rejects values other than the named ones with ZR_ERR_UNSUPPORTED (dtypes)
 * or ZR_ERR_INVALID (orders). */
typedef enum {
    ZR_BF16 = 0,
    ZR_FP32 = 1,
    ZR_DTYPE_MIN_ = -2147483647 - 1,
    ZR_DTYPE_MAX_ = 2147483647
} zr_dtype;

/* ZR_ORDER_RING: the ring order above, bit-exact and deterministic.
 * ZR_ORDER_FREE: ranks summed in an order of the library's choosing (fp32
 * accumulation); the result is within the usual fp32 summation error bound
 * of the exact sum but need not match the ring order bit for bit.
 * ZR_ORDER_RING_WIRE: the ring order with each hop's partial sum rounded to
 * the input dtype before the next hop, as on a ring that carries bf16
 * partial sums between ranks (the issue page's setup communicates in bf16):
 * acc = x_j; acc = RNE_bf16(acc + x_{j+1}); ...; bit-exact and deterministic.
 * For fp32 input it is the same as ZR_ORDER_RING. */
typedef enum {
    ZR_ORDER_RING = 0,
    ZR_ORDER_FREE = 1,
    ZR_ORDER_RING_WIRE = 2,
    ZR_ORDER_MIN_ = -2147483647 - 1,
    ZR_ORDER_MAX_ = 2147483647
} zr_order;

/* One tensor of an all-gather: its shard starts at element shard_off of
 * every rank's shard buffer and holds C = ceil(numel / K) elements; the
 * full tensor starts at element full_off of every rank's full buffer. */
typedef struct {
    int64_t shard_off;
    int64_t full_off;
    int64_t numel;
} zr_seg;

#define ZR_MAX_RANKS 64
/* Largest element count of any one buffer, fragment, bucket, segment or
 * offset (2^40); larger sizes are ZR_ERR_INVALID. */
#define ZR_MAX_ELEMS (1LL << 40)

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* zr_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int zr_version(void);

/* Bytes of device workspace that let a flatten, discrete reduce-scatter (or
 * its plan) with n fragments, or an all-gather with n segments, go out as one
 * launch on K ranks; 0 when such a call always fits one kernel-argument block
 * (n <= min(32, 256 / K)) and needs none. Host only. A multiple of 256; 0 for
 * K outside [1, ZR_MAX_RANKS] or n < 0. (A flatten fragment larger than
 * 2^28 / K tiles of 4 KiB per rank still takes more than one launch without
 * a workspace.) */
size_t zr_workspace_bytes(int K, int n);

/*
 * Bucket flatten [ZERO3 3.2, 5.1]: on every rank r, fragment p is copied to
 * bucket_r at element offset n_0 + ... + n_{p-1}, then positions
 * n_0 + ... + n_{F-1} .. padded_numel - 1 are set to +0.
 *
 *  K            ranks, 1..ZR_MAX_RANKS
 *  n_frag       fragments per rank F (>= 0); every rank has the same sizes
 *  frags        host array [K * n_frag] of device pointers, rank-major:
 *               frags[r * n_frag + p] is fragment p of rank r (may be NULL
 *               only when numels[p] == 0)
 *  numels       host array [n_frag] of fragment sizes (>= 0)
 *  buckets      host array [K] of device pointers, padded_numel elements each
 *  padded_numel >= sum(numels); callers pad to a multiple of K for the
 *               reduce-scatter that follows
 *  dt           ZR_BF16 or ZR_FP32 (a bitwise copy either way)
 *  workspace    NULL, or a device workspace of ws_bytes bytes (see the
 *               conventions above): with more than min(32, 256 / K)
 *               fragments the table is staged there and the flatten is one
 *               launch; without it, min(32, 256 / K) fragments per launch
 * Buckets must not overlap each other or any fragment (ZR_ERR_ALIAS).
 * ZR_ERR_WORKSPACE when the workspace is smaller than the table.
 */
zr_status zr_flatten_bucket(int K, int n_frag, const void* const* frags, const int64_t* numels,
                            void* const* buckets, int64_t padded_numel, zr_dtype dt,
                            void* workspace, size_t ws_bytes, void* stream);

/* A bucket flatten prepared once and launched many times (fragments and
 * buckets at fixed addresses): validation, entries and launch arguments are
 * built at create; with a workspace (needed only above min(32, 256 / K)
 * fragments) the table is copied into it at create, with a blocking copy,
 * and every launch is one kernel. The plan keeps the buffers' addresses and
 * the workspace, which it uses until destroyed. Arguments and results are
 * those of zr_flatten_bucket. zr_flatten_plan_info reports the kernel
 * launches per zr_flatten_plan_launch and the staged table's size (either
 * pointer may be NULL). */
typedef struct zr_flatten_plan zr_flatten_plan;

zr_status zr_flatten_plan_create(int K, int n_frag, const void* const* frags, const int64_t* numels,
                                 void* const* buckets, int64_t padded_numel, zr_dtype dt,
                                 void* workspace, size_t ws_bytes, zr_flatten_plan** plan);
zr_status zr_flatten_plan_launch(const zr_flatten_plan* plan, void* stream);
zr_status zr_flatten_plan_info(const zr_flatten_plan* plan, int* launches, size_t* table_bytes);
zr_status zr_flatten_plan_destroy(zr_flatten_plan* plan);

/* Flags of the reduce-scatter calls. */
#define ZR_AVERAGE 1    /* divide the sum by K */
#define ZR_ACCUMULATE 2 /* add into the existing partition instead of overwriting it */

/*
 * Fused reduce-scatter + average + cast [RING Phase 1; L14 3.2, 4.1;
 * ZERO3 1, 5.2, 5.3, 6]. For every holder rank q and o in [0, C), with
 * j = (q + chunk_shift) mod K and g = j*C + o:
 *     S        = ring-order fp32 fold of in_{j}[g], in_{j+1}[g], ..., in_{j-1}[g]
 *                (0 when g >= N)
 *     A        = S / K if (flags & ZR_AVERAGE) else S   (one IEEE fp32 divide;
 *                exact multiply by 1/K when K is a power of two)
 *     out_q[o] = A, or old + A in fp32 if (flags & ZR_ACCUMULATE), where old is
 *                the value already in out_q[o] widened to fp32
 * written as fp32 (no intermediate bf16 rounding) or rounded once to bf16.
 * ZR_ACCUMULATE is gradient accumulation over micro-steps: the first
 * micro-step overwrites the partition, later ones add to it in place
 * [ZERO3 5.3, 6]. Positions with g >= N receive +0 (or keep old + 0).
 *
 *  in        host array [K] of device pointers, N elements each (in_dt)
 *  out       host array [K] of device pointers, C elements each (out_dt)
 *  in_dt     ZR_BF16 or ZR_FP32; out_dt ZR_FP32 or ZR_BF16
 *  flags     0..3: ZR_AVERAGE and/or ZR_ACCUMULATE; other bits are ZR_ERR_INVALID
 *  order     ZR_ORDER_RING (bit-exact ring order) or ZR_ORDER_FREE
 * Outputs must be distinct and must not overlap any input (ZR_ERR_ALIAS).
 * Reads K*N elements once (plus the K*C old outputs when accumulating) and
 * writes K*C elements.
 */
zr_status zr_reduce_scatter_avg(int K, const void* const* in, zr_dtype in_dt, int64_t N,
                                void* const* out, zr_dtype out_dt, int chunk_shift,
                                int flags /* ZR_AVERAGE | ZR_ACCUMULATE */, zr_order order,
                                void* stream);

/* A reduce-scatter prepared once and launched many times, for a bucket whose
 * buffers keep their addresses from step to step: zr_rs_plan_create
 * validates the arguments and builds the launch (vector chunks, heads, tile
 * numbering, kernel), and each zr_rs_plan_launch only enqueues it. Arguments
 * and results are exactly those of zr_reduce_scatter_avg (flags fixed at
 * create). The plan keeps the buffers' addresses, not their contents; it owns
 * only host memory; N == 0 gives a plan that launches nothing. */
typedef struct zr_rs_plan zr_rs_plan;

zr_status zr_rs_plan_create(int K, const void* const* in, zr_dtype in_dt, int64_t N, void* const* out,
                            zr_dtype out_dt, int chunk_shift, int flags, zr_order order,
                            zr_rs_plan** plan);
zr_status zr_rs_plan_launch(const zr_rs_plan* plan, void* stream);
zr_status zr_rs_plan_destroy(zr_rs_plan* plan);

/*
 * Reduce-scatter straight from fragmented gradients, the discrete path
 * [ZERO3 5.2 (discrete path), 3.2]: bit for bit the result of
 * zr_flatten_bucket(K, n_frag, frags, numels, buckets, N) followed by
 * zr_reduce_scatter_avg(K, buckets, in_dt, N, out, ...), without writing the
 * bucket: every fragment element is read once where it lies.
 *
 *  frags     host array [K * n_frag] of device pointers, rank-major as in
 *            zr_flatten_bucket (NULL only where numels[p] == 0)
 *  numels    host array [n_frag]; N >= sum(numels); positions past the last
 *            fragment are zero padding
 *  out, flags, order, chunk_shift: as zr_reduce_scatter_avg
 *  workspace NULL, or a device workspace of ws_bytes bytes (see the
 *            conventions above): with more than min(32, 256 / K) fragments
 *            the table (fragments and their (fragment, chunk) pieces) is
 *            staged there and the call is one launch; without it, each
 *            launch carries min(32, 256 / K) fragments, the zero padding
 *            when it comes next, and the pieces they form
 * Outputs must be distinct and must not overlap any fragment (ZR_ERR_ALIAS).
 * ZR_ERR_WORKSPACE when the workspace is smaller than the table.
 */
zr_status zr_reduce_scatter_frags(int K, int n_frag, const void* const* frags,
                                  const int64_t* numels, int64_t N, zr_dtype in_dt,
                                  void* const* out, zr_dtype out_dt, int chunk_shift, int flags,
                                  zr_order order, void* workspace, size_t ws_bytes, void* stream);

/*
 * zr_reduce_scatter_frags for callers that cannot allocate device memory or
 * hold a workspace (code under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without the workspace, the same
 * results bit for bit. A table that needs staging is copied into a staging
 * array of ZR_NOALLOC_TABLE_BYTES bytes that the library keeps on every GPU
 * it runs on until the process ends (a file-scope device array; nothing is
 * allocated at run time: no hipMalloc, no hipFree). A table larger than that
 * is ZR_ERR_WORKSPACE, with nothing enqueued; zr_workspace_bytes(K, n_frag)
 * <= ZR_NOALLOC_TABLE_BYTES is always accepted (up to 1,910 fragments at
 * K = 64, 10,483 at K = 8). Every call on one GPU shares that GPU's array:
 * calls on one stream are ordered, but calls that overlap in time on
 * different streams of one GPU race for it. Each call rewrites the part it
 * uses, so no contents need clearing between calls. Under stream capture the
 * call goes out as argument launches, as zr_reduce_scatter_frags does.
 */
#define ZR_NOALLOC_TABLE_BYTES (1 << 20)
zr_status zr_reduce_scatter_frags_noalloc(int K, int n_frag, const void* const* frags,
                                          const int64_t* numels, int64_t N, zr_dtype in_dt,
                                          void* const* out, zr_dtype out_dt, int chunk_shift,
                                          int flags, zr_order order, void* stream);

/*
 * All-gather of sharded tensors into full tensors [RING Phase 2; L14 3.2;
 * ZERO3 1, 2.1]. For each segment and every destination rank r:
 *     full_r[full_off + j*C + o] = shard_{(j - chunk_shift) mod K}[shard_off + o]
 * for every j*C + o < numel, C = ceil(numel / K). Shard padding beyond
 * numel is never read into a full tensor.
 *
 *  shards    host array [K] of device pointers
 *  fulls     host array [K] of device pointers
 *  segs      host array [n_segs], n_segs >= 0; numel >= 0, offsets >= 0;
 *            segments must not write overlapping full ranges; each shard
 *            buffer must hold shard_off + C elements
 *  workspace NULL (32 segments per launch), or a device workspace of
 *            ws_bytes bytes: above 32 segments the segment table is staged
 *            there and the call is one launch
 * The written extent of each full buffer (lowest full_off to highest
 * full_off + numel) must not overlap another rank's, nor any shard extent
 * (ZR_ERR_ALIAS). Reads each shard element once and writes it K times.
 */
zr_status zr_all_gather(int K, const void* const* shards, void* const* fulls, zr_dtype dt,
                        const zr_seg* segs, int n_segs, int chunk_shift, void* workspace,
                        size_t ws_bytes, void* stream);

/*
 * All-reduce = reduce-scatter followed by all-gather [L14 2.2; RING].
 * Every rank receives, at every g < N, the ring-order fp32 fold of chunk
 * j = g / C (divided by K if average), stored once in dt: the same bits on
 * all K ranks.
 *
 *  in, out   host arrays [K] of device pointers, N elements of dt each;
 *            out[r] == in[r] for every r is allowed (in place); any other
 *            overlap is ZR_ERR_ALIAS
 *  fused     1: one pass that reads K values and writes the result to all K
 *            ranks; 0: zr_reduce_scatter_avg into `scratch`, then
 *            zr_all_gather from it (same bits either way)
 *  scratch   device buffer of K * C elements of dt when fused == 0, else
 *            ignored; must not overlap in/out
 */
zr_status zr_allreduce(int K, const void* const* in, void* const* out, zr_dtype dt, int64_t N,
                       int average, zr_order order, int fused, void* scratch, void* stream);

/*
 * Greedy bucket plan (host only, no GPU) [ZERO3 2.1 step 3, 2.2]: walk the
 * sizes in order; a bucket keeps taking the next item while its running total
 * is below `cap`, so the item that reaches or crosses the cap still joins it
 * (one oversized item may make a bucket larger than the cap). bucket_of[i]
 * receives the bucket index of item i (host array [n]); *n_buckets the number
 * of buckets. numels >= 0, cap >= 1.
 */
zr_status zr_plan_buckets(int n, const int64_t* numels, int64_t cap, int32_t* bucket_of,
                          int32_t* n_buckets);

/* ------------------------------------------------------------ cost model
 * alpha-beta model of collective time [L14 3.1, 3.4, 4.4], host only, no
 * GPU: a message of n bytes costs alpha + n / beta. Times in seconds, sizes
 * in bytes, alpha in seconds, beta in bytes per second. Invalid arguments
 * (K < 1, negative size or alpha, beta <= 0) return NaN (-1 for the segment
 * search).
 *   ring all-reduce       2(K-1)(alpha + N/(K beta))
 *   ring reduce-scatter   (K-1)(alpha + N/(K beta))
 *   tree all-reduce       2 ceil(log2 K)(alpha + N/beta)
 *   naive all-reduce      2(alpha + (K-1) N/beta)
 *   pipelined broadcast   (K-2+S)(alpha + N/(S beta)), K >= 2, S >= 1
 *   dp speedup            t1 / (t1/K + ring all-reduce of the gradients)
 */
double zr_cost_ring_allreduce(int K, double bytes, double alpha, double beta);
double zr_cost_ring_reduce_scatter(int K, double bytes, double alpha, double beta);
double zr_cost_tree_allreduce(int K, double bytes, double alpha, double beta);
double zr_cost_naive_allreduce(int K, double bytes, double alpha, double beta);
double zr_cost_pipelined_broadcast(int K, double bytes, int segments, double alpha, double beta);
/* Best power-of-two segment count in [1, max_segments]; its time in *time. */
int zr_cost_best_broadcast_segments(int K, double bytes, double alpha, double beta,
                                    int max_segments, double* time);
/* Message sizes (bytes) where ring equals tree / naive all-reduce. */
double zr_cost_ring_tree_crossover(int K, double alpha, double beta);
double zr_cost_ring_naive_crossover(int K, double alpha, double beta);
double zr_cost_dp_speedup(int K, double t1, double grad_bytes, double alpha, double beta);

/* A discrete reduce-scatter prepared once and launched many times: for a
 * bucket whose fragments stay at the same addresses from step to step (the
 * usual ZeRO layout), zr_rsf_plan_create validates everything and builds the
 * launches' kernel arguments, and each zr_rsf_plan_launch only enqueues
 * them. With a workspace (needed only above min(32, 256 / K) fragments) the
 * table is copied into it at create, with a blocking copy, and every launch
 * is one kernel; the plan uses the workspace until destroyed. Arguments and
 * results are exactly those of zr_reduce_scatter_frags with the same
 * arguments (the flags, including ZR_ACCUMULATE, are fixed at create). The
 * plan keeps the fragment and output addresses, not their contents: the
 * buffers must stay allocated while the plan is launched. The plan owns only
 * host memory; N == 0 gives a plan that launches nothing. zr_rsf_plan_info
 * reports the kernel launches per zr_rsf_plan_launch and the staged table's
 * size (either pointer may be NULL). */
typedef struct zr_rsf_plan zr_rsf_plan;

zr_status zr_rsf_plan_create(int K, int n_frag, const void* const* frags, const int64_t* numels,
                             int64_t N, zr_dtype in_dt, void* const* out, zr_dtype out_dt,
                             int chunk_shift, int flags, zr_order order, void* workspace,
                             size_t ws_bytes, zr_rsf_plan** plan);
zr_status zr_rsf_plan_launch(const zr_rsf_plan* plan, void* stream);
zr_status zr_rsf_plan_info(const zr_rsf_plan* plan, int* launches, size_t* table_bytes);
zr_status zr_rsf_plan_destroy(zr_rsf_plan* plan);

/* ------------------------------------------------------------- scheduler
 * Bucket/stream scheduler with per-buffer completion events [ISSUE,
 * Proposed design direction; ZERO3 3.3, 5.4].
 *
 * The reduction runs on `reduction_stream`. Buffer indices 0..n_buffers-1
 * name the physical IPG buffers (2 = ping-pong). Life of a buffer index:
 *   zr_sched_acquire(buf, producer): the producer stream waits on the event
 *       recorded after the last reduction that read this buffer, and on
 *       nothing else (not at all when the producer is the reduction stream,
 *       or a stream that a flush already ordered after that reduction); the
 *       producer may then write the buffer;
 *   zr_sched_submit_rs(buf, producers, ...): the reduction stream waits on
 *       every listed producer stream (all streams that wrote the bucket;
 *       the reduction stream itself needs no wait), runs
 *       zr_reduce_scatter_avg, and records the buffer's completion event.
 *       Until a stream other than the reduction stream has produced, no
 *       completion event is recorded; an acquire that then needs one
 *       records it at that point, after every reduction submitted so far;
 *   zr_sched_flush(caller): the caller stream waits for all reduction work
 *       submitted so far (epilogue of the backward pass).
 * acquire on a buffer already acquired, or submit on one not acquired, is
 * ZR_ERR_INVALID. The scheduler owns only its HIP events (created in
 * zr_sched_create, destroyed in zr_sched_destroy); it is not thread-safe.
 * zr_sched_destroy does not wait for queued reductions: flush into a stream
 * the caller synchronises before freeing the buffers they read or write.
 */
typedef struct zr_sched zr_sched;

zr_status zr_sched_create(zr_sched** out, int n_buffers, int max_producers,
                          void* reduction_stream);
zr_status zr_sched_acquire(zr_sched* s, int buf, void* producer_stream);
zr_status zr_sched_submit_rs(zr_sched* s, int buf, void* const* producer_streams, int n_prod,
                             int K, const void* const* in, zr_dtype in_dt, int64_t N,
                             void* const* out, zr_dtype out_dt, int chunk_shift,
                             int flags /* as zr_reduce_scatter_avg */, zr_order order);
zr_status zr_sched_flush(zr_sched* s, void* caller_stream);
zr_status zr_sched_destroy(zr_sched* s);

/* ------------------------------------------------- prefetch coordinator
 * ZeRO-3 parameter fetch and prefetch [ZERO3 2.1, 2.2]. Full parameters are
 * gathered from their 1/K shards (zr_all_gather's layout) into a caller-
 * provided arena per rank, only while they are live.
 *
 * The trace is fixed: step t (a module visit; forward then backward) uses
 * parameters step_params[step_offsets[t] .. step_offsets[t+1]). Per step:
 *   zr_pf_fetch(t): (1) gathers, on gather_stream, every parameter of step t
 *       that is not live; (2) makes compute_stream wait for the gathers that
 *       produce step t's parameters (none for gathers the host has seen
 *       finish); (3) prefetches: walks the trace after step t, skips live
 *       parameters, and gathers the others as one batch, stopping once the
 *       batch reaches min(max_live_numel - live, prefetch_bucket_numel)
 *       elements (the parameter that crosses the cap is included; nothing
 *       is prefetched while live >= max_live_numel). `live` is the element
 *       count of every gathered or in-flight full parameter.
 *   (the caller enqueues step t's compute on compute_stream, reading the
 *       addresses from zr_pf_full)
 *   zr_pf_release(t): step t's parameters stop being live, except those
 *       used again within max_reuse_numel elements of parameters after step
 *       t (the steps after t are scanned in order, a step at a time, until
 *       the parameters seen reach max_reuse_numel; the scan stays within this
 *       pass of the trace) [ZERO3 2.4]; the arena ranges of released
 *       parameters are reused only after compute_stream has passed this
 *       point.
 * At most max_ongoing_fetches gathers are outstanding (the page's value is
 * 2): before a new gather the host drops finished ones and blocks on the
 * oldest until fewer remain. Steps are fetched and released in trace order;
 * after the last step is released the trace starts over at step 0. Calls out
 * of order are ZR_ERR_INVALID.
 *
 * Arena: arena_numel elements in every rank's buffer, handed out in
 * 256-byte-aligned ranges at the same offsets on every rank. A gather takes
 * the free range released longest ago (never-used memory first), so it waits
 * only for the compute that last read that memory; a larger arena is used
 * whole before memory is reused. It must hold every single step's
 * parameters (checked at create, else ZR_ERR_NOMEM). A prefetch that does
 * not fit is cut to the part that fits; a step whose parameters cannot be
 * placed fails with ZR_ERR_NOMEM. Sizing: max_live_numel plus the largest
 * step and the largest parameter, plus room for fragmentation; zr_pf_plan
 * runs a trace on the host and reports whether a capacity works (no
 * ZR_ERR_NOMEM) and how many prefetches it trims.
 * gather_stream == compute_stream runs gathers and compute in series (no
 * overlap). The coordinator owns its HIP events and its copy of the trace;
 * it keeps the shard, arena and stream handles; it is not thread-safe.
 * zr_pf_destroy blocks until the gathers it issued have finished; the
 * caller frees the arenas once its own compute that reads them is done.
 */
typedef struct zr_pf zr_pf;

typedef struct {
    int K;                         /* ranks, 1..ZR_MAX_RANKS */
    zr_dtype dtype;
    int n_params;
    const int64_t* numels;         /* [n_params] full sizes, each >= 1 */
    const int64_t* shard_offsets;  /* [n_params] offset of each shard in every
                                      rank's shard buffer */
    const void* const* shards;     /* [K] shard buffers; parameter p's shard
                                      holds ceil(numels[p] / K) elements */
    void* const* arenas;           /* [K] arena buffers of arena_numel elements */
    int64_t arena_numel;
    int chunk_shift;               /* rank r holds chunk (r + s) mod K; ZeRO-3: 0 */
    int n_steps;
    const int32_t* step_offsets;   /* [n_steps + 1], step_offsets[0] = 0 */
    const int32_t* step_params;    /* parameter ids, trace order */
    int64_t prefetch_bucket_numel; /* >= 1 */
    int64_t max_live_numel;        /* >= 1 */
    int64_t max_reuse_numel;       /* conservative-release window, >= 0 */
    int max_ongoing_fetches;       /* >= 1 */
    void* gather_stream;           /* hipStream_t */
    void* compute_stream;          /* hipStream_t */
} zr_pf_config;

typedef struct {
    int64_t gathers;            /* gather batches issued */
    int64_t immediate_gathers;  /* batches of part (1): parameters not prefetched */
    int64_t immediate_numel;
    int64_t prefetch_numel;
    int64_t host_syncs;         /* host blocked on the oldest gather */
    int64_t stream_waits;       /* compute_stream waits on a gather */
    int64_t live;               /* elements live now */
    int64_t peak_live;
    int64_t peak_ongoing;       /* most gathers outstanding at once */
    int64_t arena_peak;         /* highest arena element offset used */
    int64_t prefetch_trimmed;   /* prefetches cut short by a full arena */
    int64_t retained;           /* releases skipped: the parameter is reused soon */
} zr_pf_stats;

/* Validates the whole config (buffers distinct and disjoint from the shard
 * ranges, trace ids in range) and creates the coordinator's events. */
zr_status zr_pf_create(const zr_pf_config* cfg, zr_pf** out);
zr_status zr_pf_fetch(zr_pf* pf, int step);
zr_status zr_pf_release(zr_pf* pf, int step);
/* Device address of live parameter `param` in rank `rank`'s arena;
 * ZR_ERR_INVALID when it is not live. */
zr_status zr_pf_full(const zr_pf* pf, int param, int rank, void** full);
zr_status zr_pf_get_stats(const zr_pf* pf, zr_pf_stats* out);
zr_status zr_pf_destroy(zr_pf* pf);
/* Host only (no GPU): runs the trace `iterations` times through the same
 * coordinator with gathers that finish at once, and reports the resulting
 * counters (peak live elements, arena peak, ...). Uses only the sizes, the
 * trace, the caps and arena_numel of cfg; pointers and streams may be NULL. */
zr_status zr_pf_plan(const zr_pf_config* cfg, int iterations, zr_pf_stats* out);

#ifdef __cplusplus
}
#endif

#endif /* ZR_H */
