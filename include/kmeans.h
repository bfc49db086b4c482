/*
 * kmeans.h -- C ABI of the MI355X (gfx950) exact Lloyd K-Means library.
 *
 * Citations name the page "Flash-KMeans: Fast and Memory-Efficient Exact
 * K-Means" (gist.science summary of paper 2603.09229): "tech §n" is a section
 * of its technical summary, "pop §n" one of its popular explainer.
 *
 * What the library computes.  Standard Lloyd K-Means, exactly (the page keeps
 * the K-Means formula and adds no approximation: tech §2 opening, tech §3).
 * The page leaves these rules open; this library fixes them:
 *   - distance: squared Euclidean;
 *   - assignment: nearest centroid, the LOWEST index wins a tie;
 *   - update: new centroid = mean of its assigned points; a cluster with no
 *     point keeps its previous centroid bit for bit;
 *   - one iteration = one assignment followed by one update; `iters` runs
 *     exactly that many (no tolerance, no early exit).
 *
 * Precision.  X may be fp32, bf16 or fp16.  Centroids are always fp32.  For
 * 16-bit X the distance contraction runs on the matrix cores with fp32
 * accumulation against the fp32 centroids rounded once per assignment to X's
 * type (round to nearest, ties to even); sums and means are accumulated in
 * fp32.  Near-equal distances (relative gap around 1e-6 of ||x||^2 + ||c||^2)
 * may resolve differently from exact arithmetic.
 *
 * Conventions for every entry point:
 *   - Layout: X is N x D row-major (element type `dt`), C is K x D row-major
 *     fp32, assignment vectors are int32[N], counts int32[K].  X must be
 *     4-byte aligned (16-byte alignment with D*sizeof(elem) % 16 == 0 enables
 *     vector loads); every other pointer 4-byte aligned (`objective` 8).
 *   - Memory: "device" pointers are HIP device memory (e.g. torch CUDA tensors
 *     on ROCm); "pinned host" pointers come from hipHostMalloc (torch's
 *     pin_memory()).  The caller owns every buffer; the library never
 *     allocates or frees memory.  Scratch space is the caller's workspace
 *     `ws` (device memory of at least kmeans_workspace_bytes() bytes, any
 *     content, 256-byte aligned); it must not be used by anything else while
 *     the call's work runs.
 *   - Streams: `stream` is a hipStream_t (NULL = the default stream).  All
 *     work is enqueued asynchronously on it; results are ready once the
 *     stream is synchronised.  The library never synchronises the host
 *     (kmeans_fit_streamed returns once its last chunk is enqueued).
 *   - Limits: 1 <= N < 2^31, 1 <= K < 2^31, 1 <= D <= 2^24 and K*D < 2^37
 *     (beyond: KM_ERR_UNSUPPORTED).  The page has N, K and D change from call
 *     to call (tech §1); every D is served: rows of up to 512 16-bit / 256
 *     fp32 values are held whole in registers, longer rows are walked in
 *     depth chunks by the assignment and in column strips by the update
 *     (same results, same rules).  K > N is allowed (the extra clusters stay
 *     empty).  N = 0 is accepted and does nothing except the documented
 *     output of an empty update.
 *   - Errors: arguments, dtype and workspace size are checked synchronously
 *     before any HIP call, so a failed check enqueues nothing.  A failed
 *     launch returns KM_ERR_HIP.  Faults inside kernels surface at the
 *     caller's next synchronisation.  No C++ exception crosses this ABI.
 *     kmeans_last_error() gives a message for the last failure on the
 *     calling thread.
 *   - Reentrancy: calls are thread-safe given distinct workspaces.  Global
 *     state, all of it behind a lock or atomic: the per-device property
 *     cache (filled on a device's first call), the planner overrides (for
 *     measurement), the optional kernel-timing registry, and the
 *     no-allocation fit's per-GPU scratch (whose overlapping calls race).
 */
#ifndef MEANS_CLUSTERING_AMD_KMEANS_H
#define MEANS_CLUSTERING_AMD_KMEANS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations are plain ints on the C side (a C caller may pass any int);
 * the C++ implementation gives them int as their fixed underlying type, so an
 * out-of-range value from such a caller is a valid value it can reject. */
#ifdef __cplusplus
#define KM_ENUM_INT : int
#else
#define KM_ENUM_INT
#endif

typedef enum km_dtype KM_ENUM_INT { KM_F32 = 0, KM_BF16 = 1, KM_F16 = 2 } km_dtype;

typedef enum km_status KM_ENUM_INT {
  KM_OK = 0,
  KM_ERR_INVALID_VALUE = 1, /* null pointer, size out of range, misalignment, bad dtype */
  KM_ERR_UNSUPPORTED = 2,   /* valid but beyond a size limit (D > 2^24, K*D, B*N; no-alloc scratch) */
  KM_ERR_WORKSPACE = 3,     /* ws is NULL or ws_bytes smaller than required */
  KM_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} km_status;

typedef enum km_op KM_ENUM_INT {
  KM_OP_ASSIGN = 0,
  KM_OP_UPDATE = 1,
  KM_OP_FIT = 2,
  KM_OP_FIT_STREAMED = 3,
  KM_OP_SORT = 4,
  KM_OP_FIT_STREAMED_WARM = 5, /* kmeans_fit_streamed with room for every chunk's warm-start order */
  KM_OP_FIT_STREAMED_RESIDENT = 6 /* ... and for a device copy of all of X */
} km_op;

/*
 * Workspace bytes needed by entry point `op` for the given sizes (N is the
 * number of points; for KM_OP_FIT_STREAMED `chunk_rows` is the chunk size).
 * KM_OP_FIT_STREAMED_WARM: the streamed fit's workspace plus 8 bytes per row
 * of X, where each chunk keeps its sorted order from one iteration to the
 * next so that later iterations assign it warm (faster, same results bit for
 * bit); kmeans_fit_streamed uses that room whenever ws_bytes holds it.
 * KM_OP_FIT_STREAMED_RESIDENT: the KM_OP_FIT_STREAMED_WARM workspace plus
 * N * D * sizeof(dt) bytes (rounded up to 256) for a device copy of X.
 * kmeans_fit_streamed keeps in the workspace beyond the warm layout as many
 * leading chunks of X as fit whole: each is uploaded once, in the first
 * iteration, and read from device memory in later ones (same results, bit
 * for bit; only host-link traffic changes).
 * Returns 0 if the arguments are invalid.
 */
size_t kmeans_workspace_bytes(km_op op, int64_t N, int64_t D, int64_t K, km_dtype dt, int64_t chunk_rows);

/*
 * kmeans_assign -- FlashAssign (tech §2.1): nearest centroid of every point,
 * fused with the distance computation so that no N x K distance matrix is
 * ever written (HBM traffic O(Nd + Kd), tech §2.1 "effect").
 *   X        device, N x D, type dt                         (read)
 *   C        device, K x D fp32 centroids                   (read)
 *   assign   device int32[N]: index of the nearest centroid (written)
 *   min_dist device fp32[N] or NULL: squared distance to that centroid,
 *            computed as ||x||^2 - 2 x.c + ||c||^2 in fp32, clamped at 0
 * When N is small against the GPU and K is large, the centroid sweep is split
 * over several workgroups and merged in index order (workspace: a score and an
 * index per point and range); the result is bit for bit the unsplit one.
 */
km_status kmeans_assign(const void* X, km_dtype dt, int64_t N, int64_t D, const float* C, int64_t K,
                        int32_t* assign, float* min_dist, void* ws, size_t ws_bytes, void* stream);

/*
 * kmeans_sort_by_cluster -- the explicit inverse map of Sort-Inverse Update
 * (tech §2.2 "explicit inverse mapping"): a stable argsort of the assignment
 * vector by cluster id, plus each cluster's segment boundaries.
 *   assign   device int32[N] cluster ids                    (read)
 *   perm     device int32[N]: point indices grouped by ascending cluster id,
 *            ascending point index within a cluster; a point whose id is
 *            outside [0, K) is listed inside cluster K-1's range with bit 31
 *            set (its index is perm & 0x7fffffff)           (written)
 *   offsets  device int32[K+1] or NULL: cluster k occupies perm[offsets[k] ..
 *            offsets[k+1]); offsets[K] = N                  (written)
 */
km_status kmeans_sort_by_cluster(const int32_t* assign, int64_t N, int64_t K, int32_t* perm, int32_t* offsets,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * kmeans_update -- Sort-Inverse Update (tech §2.2): argsort of the assignment
 * vector, segment boundaries, then a segmented reduction over the sorted
 * order with no atomic operation anywhere (the page's variant issues atomics
 * only at segment boundaries; here boundary pieces are summed by a fixed-
 * order pass, so results are deterministic).
 *   X       device, N x D, type dt                          (read)
 *   assign  device int32[N] cluster ids; ids outside [0, K) are ignored
 *   C_prev  device K x D fp32: centroids kept by empty clusters (read)
 *   C_new   device K x D fp32: means (written; may alias C_prev)
 *   counts  device int32[K] or NULL: points per cluster     (written)
 */
km_status kmeans_update(const void* X, km_dtype dt, int64_t N, int64_t D, const int32_t* assign, int64_t K,
                        const float* C_prev, float* C_new, int32_t* counts, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * kmeans_fit -- `iters` Lloyd iterations with X resident in device memory
 * (the page's end-to-end K-Means: the assignment step of tech §2.1 followed
 * by the centroid step of tech §2.2, repeated; tech §1 states the two steps
 * and tech §4 times them end to end); each iteration is kmeans_assign
 * followed by kmeans_update, all enqueued on `stream` with no host
 * synchronisation.
 *   C          device K x D fp32: initial centroids in, C^iters out
 *   assign     device int32[N] or NULL: assignment of the last iteration
 *   counts     device int32[K] or NULL: counts that formed C^iters
 *   objective  device double[iters] or NULL: objective[t] = sum of squared
 *              distances of iteration t's assignment (fp32 terms, fp64 sum)
 *   iters = 0 leaves every output untouched.
 */
km_status kmeans_fit(const void* X, km_dtype dt, int64_t N, int64_t D, int64_t K, float* C, int32_t iters,
                     int32_t* assign, int32_t* counts, double* objective, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * kmeans_fit_streamed -- Lloyd iterations for X that stays in host memory
 * (tech §2.3 "chunked stream overlap"; tech §1 names data larger than device
 * memory): every iteration copies X to the device in chunks of `chunk_rows`
 * rows on `copy_stream`, two device buffers in rotation, while
 * `compute_stream` assigns the previous chunk and accumulates its per-cluster
 * sums; the means are formed once per iteration.  A workspace of
 * KM_OP_FIT_STREAMED_WARM size or more adds the warm start; beyond that size
 * the leading chunks that fit whole are kept on the device after their first
 * upload (KM_OP_FIT_STREAMED_RESIDENT: all of X), and later iterations read
 * them there instead of copying them again.
 *   X_host       host, N x D, type dt                        (read)
 *                With stage_host == NULL it must be pinned (hipHostMalloc /
 *                torch pin_memory) and is read by the DMA engine directly.
 *                With a staging buffer it may be ordinary pageable memory:
 *                host threads of the library copy it slot by slot into the
 *                staging buffer, from which it is uploaded.
 *   C            device K x D fp32: initial centroids in, C^iters out
 *   assign_host  pinned host int32[N] or NULL: assignment of the last
 *                iteration (copied back chunk by chunk)
 *   counts       device int32[K] or NULL
 *   objective    device double[iters] or NULL (as kmeans_fit)
 *   compute_stream, copy_stream: distinct hipStream_t (NULL allowed for
 *                compute_stream only).
 *   stage_host, stage_bytes: pinned host staging buffer or NULL.  It is split
 *                into 4 slots of floor(stage_bytes / 4) bytes rounded down to
 *                whole rows (at least one row each, else
 *                KM_ERR_INVALID_VALUE); a few tens of MiB per slot keep the
 *                host link busy.  The number of copying threads is
 *                min(8, cores - 1) + the caller, or KM_STAGE_THREADS.
 * On return all work is enqueued.  With staging the call blocks while the
 * upload proceeds and returns once every byte of X has left the staging
 * buffer, so X_host and the staging buffer are free again on return; without
 * staging, keep X_host unchanged until compute_stream has been synchronised.
 * On an error return the same holds: with staging, uploads already issued
 * from the staging buffer have finished; work already enqueued on the two
 * streams still runs, and the outputs are undefined until a later call
 * succeeds (restart from the last good centroids: a fit of T - t
 * iterations from C^t equals the uninterrupted one bit for bit).  Tests
 * force the error path with the environment variable
 * KM_FAULT_INJECT_UPLOAD=n, which fails the n-th chunk upload of a call
 * before it is issued.
 * Synchronise compute_stream before reading any output.  Uploads into the
 * workspace start only after the work enqueued on compute_stream before the
 * call, so a workspace may be reused in compute-stream order.
 */
km_status kmeans_fit_streamed(const void* X_host, km_dtype dt, int64_t N, int64_t D, int64_t K, float* C,
                              int32_t iters, int64_t chunk_rows, int32_t* assign_host, int32_t* counts,
                              double* objective, void* ws, size_t ws_bytes, void* compute_stream,
                              void* copy_stream, void* stage_host, size_t stage_bytes);

/*
 * kmeans_workspace_bytes_batched -- workspace bytes for kmeans_fit_batched
 * (B problems of N points, D dimensions and K clusters each).  Returns 0 if
 * the arguments are invalid.
 */
size_t kmeans_workspace_bytes_batched(int64_t B, int64_t N, int64_t D, int64_t K, km_dtype dt);

/*
 * kmeans_fit_batched -- Lloyd iterations of B independent problems of one
 * shape in the same launches.  The page treats K-Means as an online
 * primitive called at high frequency inside AI pipelines (tech §1, tech §5);
 * a single small problem leaves the GPU idle between short kernels, so here
 * every phase of an iteration covers all B problems at once: one centroid
 * preparation, one FlashAssign launch (workgroups split over the problems),
 * and one sort-inverse update over B*N points whose cluster ids are made
 * distinct per problem (b*K + k), so each problem's clusters get their own
 * segments.  Each problem follows the same rules as kmeans_fit.
 *   X          device, B x N x D, type dt (problem b is rows b*N .. b*N+N-1)
 *   C          device B x K x D fp32: initial centroids in, C^iters out
 *   assign     device int32[B*N] or NULL: per-problem ids in [0, K) of the
 *              last iteration
 *   counts     device int32[B*K] or NULL: counts that formed C^iters
 *   objective  device double[iters*B] or NULL: objective[t*B + b] = sum of
 *              squared distances of problem b in iteration t (fp32 terms,
 *              fp64 sum)
 *   Limits: as kmeans_fit per problem, and B >= 1, B*N < 2^31, B*K < 2^31.
 *   iters = 0 leaves every output untouched.  Centroid sums of different
 *   problems never mix; the summation order inside a problem may differ
 *   from kmeans_fit on that problem alone (fp32 rounding only), and the
 *   assignment of a given centroid state is the same bit for bit.
 */
km_status kmeans_fit_batched(const void* X, km_dtype dt, int64_t B, int64_t N, int64_t D, int64_t K, float* C,
                             int32_t iters, int32_t* assign, int32_t* counts, double* objective, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * kmeans_fit_noalloc -- kmeans_fit for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, arguments and results as
 * kmeans_fit (bit for bit), with no workspace argument.  Its scratch space is
 * a fixed device array of KMEANS_NOALLOC_SCRATCH_BYTES inside the library
 * (one per GPU, held from library load until the process ends); the call
 * never allocates or frees memory.  Shapes whose kmeans_fit workspace
 * (kmeans_workspace_bytes(KM_OP_FIT, ...)) exceeds that size are rejected
 * with KM_ERR_UNSUPPORTED before any HIP call.  `stream` must belong to the
 * current device (else KM_ERR_INVALID_VALUE).  All calls on one GPU share the
 * array: calls that may overlap on one GPU (other streams, other threads)
 * race and must be serialised by the caller; calls in order on one stream
 * are safe.
 */
#define KMEANS_NOALLOC_SCRATCH_BYTES (64u << 20)
km_status kmeans_fit_noalloc(const void* X, km_dtype dt, int64_t N, int64_t D, int64_t K, float* C, int32_t iters,
                             int32_t* assign, int32_t* counts, double* objective, void* stream);

/*
 * Planner (for measurement).  The library chooses every launch shape itself
 * from N, K, D, the dtype and the device (compute units and last-level cache
 * size, read once per device); there is no tuning run and no compiled-at-
 * first-use code.  kmeans_plan_override(key, value) replaces one of those
 * choices for every later call of this process (value 0 restores the
 * planner's choice); it is meant for comparing the static choice against
 * the alternatives, not for production use, and must not change while a
 * call is being enqueued.  Keys and values:
 *   "assign_kernel"  1 pipelined four-wavefront kernel, 2 single-accumulator
 *                    kernel (16-bit X, D <= 128)
 *   "assign_fold"    1 exact argmax per score, 2 folded argmax (cold launches)
 *   "assign_split"   1 never split the centroid sweep, 2..64 ranges
 *   "reduce_tile"    1 long segment tiles, 2 short ones
 *   "radix_items"    8, 16 or 32 keys per thread in the argsort
 *   "small_update"   1 never the on-chip small-codebook update
 *   "sort_scan"      1 scan the argsort's larger (digit, block) count
 *                    tables as a whole (three launches), 2 scan every
 *                    table digit by digit (one launch); by default small
 *                    tables are summed by every scatter workgroup and
 *                    larger ones scanned digit by digit
 *   "sort_rank"      1 rank a block's keys with per-thread digit counters,
 *                    2 with wavefront ballots
 *   "radix_bits"     5 to 8: the widest digit of an argsort pass (above 6
 *                    the ballot ranking is used); by default 8 where that
 *                    saves one of at most three passes in blocks of up to
 *                    4,096 keys, else 6
 * Every choice gives the same assignments; sums may differ in fp32 rounding.
 * kmeans_plan_describe(N, D, K, dt, buf, len) writes a one-line description
 * of the plan of kmeans_fit for that shape (NUL-terminated, truncated to len).
 */
km_status kmeans_plan_override(const char* key, int64_t value);
km_status kmeans_plan_describe(int64_t N, int64_t D, int64_t K, km_dtype dt, char* buf, size_t len);

/* Short constant description of a status code. */
const char* kmeans_status_string(km_status s);

/* Message describing the last failed call on this thread ("" if none). */
const char* kmeans_last_error(void);

/*
 * Kernel timing (for measurement, off by default).  kmeans_timing_enable(1):
 * every kernel phase a call enqueues is bracketed by HIP events on the stream
 * it runs on; kmeans_timing_enable(2): only the FlashAssign launches ("assign"
 * phase), so the events barely perturb the rest; 0: off.  The events carry
 * no system-scope fence (they only take timestamps), but each record still
 * costs a marker packet and some host time, so throughput is measured with 2
 * or 0.  The mode can change between calls.  kmeans_timing_read() waits for
 * the recorded events and returns the
 * summed milliseconds and the number of timed launches of one phase:
 * "prep", "assign", "sort", "segments", "reduce", "finalize", "objective",
 * "h2d", "d2h".  kmeans_timing_reset() forgets all records.
 */
km_status kmeans_timing_enable(int enable);
km_status kmeans_timing_read(const char* phase, double* total_ms, int64_t* launches);
km_status kmeans_timing_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* MEANS_CLUSTERING_AMD_KMEANS_H */
