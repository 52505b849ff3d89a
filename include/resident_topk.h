/*
 * resident_topk.h -- C ABI of libresident_topk: exact brute-force top-K over a
 * device-resident fp32 corpus on an AMD Instinct MI355X (gfx950).
 *
 * The method ("GPU-Resident Top-K for Agentic RAG", A. Banerjee):
 *   - the corpus is copied into device memory once and stays there (section 3,
 *     "keep the corpus on the GPU"; section 4, Step 1);
 *   - per query, every corpus row is scored by inner product (section 4, Step 2),
 *     each block of rows keeps its own best-K list (Step 3), and the per-block
 *     lists are merged into the global best-K (Step 4);
 *   - only K indices and K scores come back (section 3; section 4, Step 6).
 * The order is the pages' comparator (section 3, "Problem B"): a larger score
 * wins; on an exact tie (float ==, so -0.0 ties +0.0) the lower index wins.
 * The same two-stage selector is exported as a plain top-K over raw int32/fp32
 * arrays ("CUDA Programming Model Series 9: Efficient TopK, two-stage
 * reduction kernel design", sections 2 and 3: per-block partial top-K, then a
 * second-stage merge).
 *
 * Conventions for every entry point
 *   - Pointers named "device" must point to device memory of the engine's GPU
 *     (hipMalloc, or a torch CUDA tensor).  They stay owned by the caller and
 *     must remain valid until the work queued on `stream` has finished.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     search_resident and topk_select only enqueue work; the caller
 *     synchronises the stream before reading outputs.
 *   - All device memory the engine needs is allocated by rt_engine_create.  No
 *     other entry point allocates (the pages' "Problem C": no allocation on the
 *     hot path).
 *   - Argument errors are detected on the host before anything is enqueued;
 *     outputs are then left untouched.
 *   - One engine runs one search or select at a time: calls on one engine that
 *     overlap on different streams race on the engine's scratch memory.  For
 *     concurrent searches use several engines sharing one corpus
 *     (rt_engine_create_shared).
 *   - Results are best-first.  Indices are int32 (0-based row / element
 *     positions), so n is limited to 2^31 - 1.
 *   - Inputs must be NaN-free; the comparator does not order NaN.
 */
#ifndef RESIDENT_TOPK_H
#define RESIDENT_TOPK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct rt_engine rt_engine; /* opaque; owns every device buffer */

typedef enum {
    RT_OK = 0,
    RT_EINVAL = 1, /* bad argument: null pointer, size out of range, k > n, ... */
    RT_ESTATE = 2, /* wrong state: search before upload, dimension mismatch */
    RT_ENOMEM = 3, /* device allocation failed in rt_engine_create */
    RT_EHIP = 4    /* a HIP runtime call failed; see rt_last_hip_error */
} rt_status;

typedef enum { RT_DTYPE_INT32 = 0, RT_DTYPE_FLOAT32 = 1 } rt_dtype;

/* Similarity used by search_resident_metric ("GPU-Resident Top-K for Agentic
 * RAG", section 4, Step 2: the scoring kernel computes an inner product and,
 * with cosine enabled, divides it by the query's and the row's L2 norms). */
typedef enum { RT_METRIC_DOT = 0, RT_METRIC_COSINE = 1 } rt_metric;

/* The first pass of a single-query filtered search (rt_set_filter_storage). */
typedef enum { RT_FILTER_AUTO = 0, RT_FILTER_BF16 = 1, RT_FILTER_FP8 = 2 } rt_filter_storage;

/* What the last search_resident_filtered call ran (rt_filter_path_used). */
typedef enum {
    RT_FILTER_PATH_NONE = 0,        /* no filtered search yet */
    RT_FILTER_PATH_PLAIN = 1,       /* the plain fp32 scan: copy unusable, depth not covered, or one
                                       query over a small corpus under RT_FILTER_AUTO */
    RT_FILTER_PATH_BF16 = 2,        /* bf16 first pass, one query per segment */
    RT_FILTER_PATH_FP8 = 3,         /* fp8 first pass, one query per segment */
    RT_FILTER_PATH_BF16_MATRIX = 4  /* bf16 matrix-core first pass for the whole batch */
} rt_filter_path;

/*
 * Create an engine on HIP device `device` and allocate, once, everything later
 * calls need, sized for the worst case: a corpus of max_n x max_d fp32, results
 * up to max_k per query, batches up to max_q queries ("GPU-Resident Top-K for
 * Agentic RAG", section 3 "Problem C" and section 4 Step 0: all device
 * allocations happen at engine initialisation).
 * Limits: 1 <= max_n <= 2^31-1; 1 <= max_d <= 65536; 1 <= max_k <= 1024;
 * 1 <= max_q <= 32.  On success *out receives the engine (RT_OK); otherwise
 * *out is set to NULL and RT_EINVAL / RT_ENOMEM / RT_EHIP is returned.
 */
rt_status rt_engine_create(int64_t max_n, int32_t max_d, int32_t max_k, int32_t max_q,
                           int32_t device, rt_engine **out);

/*
 * Create an engine that searches the same resident corpus as `other` without a
 * copy: the corpus and its row norms are shared (reference-counted: they stay
 * allocated until the last engine sharing them is destroyed, in any order),
 * while the new engine has scratch memory of its own (merge tree, counters,
 * batch buffers, timing events), sized for results up to max_k and batches up
 * to max_q.  Searches and selects on different engines may therefore run at
 * the same time on different streams -- several agents querying one corpus
 * concurrently, the use case of "GPU-Resident Top-K for Agentic RAG" (section
 * 1: many micro-agents, each retrieving top-K from the same corpus; section 9
 * lists query concurrency within one engine as missing).  An upload through any of the sharing engines
 * replaces the corpus for all of them; the caller must not upload while a
 * search on any of them is in flight.
 * Limits as rt_engine_create (1 <= max_k <= 1024, 1 <= max_q <= 32); the
 * device is other's.  RT_EINVAL for NULL arguments or limits out of range,
 * RT_ENOMEM / RT_EHIP if the scratch cannot be allocated (then *out = NULL).
 */
rt_status rt_engine_create_shared(rt_engine *other, int32_t max_k, int32_t max_q, rt_engine **out);

/* Free the engine's own device buffers, and the resident corpus if no other
 * engine shares it (waits for pending work on the device).  NULL is ignored. */
void rt_engine_destroy(rt_engine *e);

/*
 * Copy an n x d row-major fp32 corpus into the engine's device memory and make
 * it the resident corpus, replacing any previous one ("GPU-Resident Top-K for
 * Agentic RAG", section 4, Step 1).  `corpus` may be host or device memory
 * (hipMemcpyDefault); the caller keeps ownership.  The L2 norm of every row is
 * computed on the device as part of the upload (for the cosine metric; section
 * 4, Step 2 keeps a precomputed per-row norm).  Synchronous: when it returns
 * RT_OK the copy and the norms are complete.  RT_EINVAL if e or corpus is NULL, n < 1,
 * n > max_n, d < 1 or d > max_d (the pages return "invalid value" for
 * N > max_n or D > max_d).  On failure the previous corpus stays resident
 * unless the copy itself failed (RT_EHIP), in which case no corpus is resident.
 */
rt_status upload_corpus_rowmajor(rt_engine *e, const float *corpus, int64_t n, int32_t d);

/*
 * Exact top-k by inner product for q queries against the resident corpus
 * ("GPU-Resident Top-K for Agentic RAG", section 4, Steps 2-5).
 *   queries    device, q x d fp32 row-major, d = the resident dimension
 *   out_idx    device, q x k int32: row indices, best-first per query
 *   out_scores device, q x k fp32: the matching scores (fp32 dot products)
 * Order: larger score first, exact ties to the lower row index.
 * RT_EINVAL: null pointer, q < 1, q > max_q, k < 1, k > max_k, k > n.
 * RT_ESTATE: no corpus resident.  RT_EHIP: a launch failed.
 * Asynchronous on `stream`.
 */
rt_status search_resident(rt_engine *e, const float *queries, int32_t q, int32_t k,
                          int32_t *out_idx, float *out_scores, void *stream);

/*
 * search_resident with a choice of similarity ("GPU-Resident Top-K for Agentic
 * RAG", section 4, Step 2, and section 7 on dot product versus cosine):
 *   RT_METRIC_DOT     score = <row, query> (exactly search_resident);
 *   RT_METRIC_COSINE  score = <row, query> / (|query| |row|), computed in fp32
 *                     from the inner product, the row's L2 norm (computed at
 *                     upload) and the query's L2 norm (computed on the device
 *                     per call); -inf when |query| |row| is not positive (a
 *                     zero row or a zero query), so such rows rank last and,
 *                     among themselves, by lower index.
 * Arguments, layouts, ordering and errors are those of search_resident, plus
 * RT_EINVAL for an unknown metric.
 */
rt_status search_resident_metric(rt_engine *e, const float *queries, int32_t q, int32_t k, int32_t metric,
                                 int32_t *out_idx, float *out_scores, void *stream);

/*
 * Prepare an engine for search_resident_filtered: allocate, once, a bf16 copy
 * of the resident corpus (max_n x max_d x 2 bytes) with 4 bytes per row of
 * bf16 error norms, and an fp8 copy (max_n x max_d bytes of e4m3 codes and 8
 * bytes per row: the scale and the row's part of the fp8 bound),
 * shared by every engine that shares the corpus and refreshed by each upload,
 * and this engine's scratch for the filtered search (4 x max_q x
 * roundup(max_n, 64) bytes of row bounds).
 * Like rt_engine_create, it allocates: call it at set-up, not per query.
 * RT_EINVAL for NULL, RT_ENOMEM if the memory is not available.
 */
rt_status rt_enable_filtered(rt_engine *e);

/*
 * Exact top-k by inner product: for each query, the answer search_resident
 * gives for that query alone (indices, order and fp32 scores, bit for bit),
 * reading the fp32 rows only where they can matter.  "Reduced-precision
 * storage with exact re-rank" ("CUDA Programming Model Series 9: Efficient
 * TopK", section 4.3): a first pass scores every row from the bf16 copy (half
 * the bytes) and bounds the difference to the fp32 score from the rounding to
 * bf16 and the fp32 summation error of both sums (with the rows' and the
 * query's L2 norms, Cauchy-Schwarz); a threshold T certified to be at most the
 * k-th largest fp32 score follows from the lower bounds, so only rows whose
 * upper bound reaches T are scored in fp32 by the second pass -- with the
 * single-query scan's arithmetic -- and ranked.  A batch (q > 1) on an engine
 * created with max_q > 1 and a depth of 256, 384, 512, 768 or 1024 runs the
 * first pass once for all queries on bf16 matrix cores, with the query split
 * into two bf16 parts (constants: rt_filter_bounds_batched) and T the k-th
 * largest of the per-query maxima of the lower bounds over 32-row tiles.
 * Arguments, layouts and errors as search_resident; RT_ESTATE also when
 * rt_enable_filtered was not called on this engine.  If the depth is not a
 * multiple of 8 or above 2048, or a corpus value is not finite in bf16, the
 * call runs the plain fp32 scan instead, one query at a time (same answers).
 * Asynchronous on `stream`.  search_resident_filtered_metric(RT_METRIC_DOT)
 * is the same call.
 */
/*
 * Which first pass a single-query filtered search takes (host-only setting of
 * the engine): RT_FILTER_BF16, RT_FILTER_FP8 (rows stored as e4m3 codes of
 * row / s with a power-of-two scale s per row: a quarter of the fp32 bytes,
 * bound e = |q| (cr |x - x~| + cx |x|) + delta max(|q|, 1) max(s, 1), constants
 * from rt_filter_bounds_fp8; wider than bf16's, so more rows reach the
 * re-rank), or RT_FILTER_AUTO (the default: for a single query, the plain
 * fp32 scan below 44 x 2^20 corpus elements, where the two passes cost more
 * than they save, and the fp8 pass from there on).  The fp8 pass covers d in
 * {256, 384, 512, 768, 1024, 1536, 2048} and a corpus whose values are finite;
 * otherwise the bf16 pass runs.  Batches on an
 * engine with batch buffers always take the bf16 matrix-core pass.  The answer
 * is the same in every case.  RT_EINVAL for NULL or an unknown value.
 */
rt_status rt_set_filter_storage(rt_engine *e, int32_t storage);

/* The rt_filter_path of the last search_resident_filtered call (host-only). */
int32_t rt_filter_path_used(const rt_engine *e);

rt_status search_resident_filtered(rt_engine *e, const float *queries, int32_t q, int32_t k,
                                   int32_t *out_idx, float *out_scores, void *stream);

/*
 * search_resident_filtered with a metric: RT_METRIC_DOT as above, or
 * RT_METRIC_COSINE, whose answer is search_resident_metric's cosine answer for
 * that query alone (indices, order and fp32 scores, bit for bit: the cosine
 * sum / (|q| |x|), -inf where that product is not positive).  The first pass
 * turns each row's inner-product bounds into cosine bounds through the same
 * fp32 product |q| |x| that the scan divides by (widened by 2^-20 relative and
 * FLT_MIN absolute for the roundings of the divisions); the second pass
 * re-scores with the scan's arithmetic.  A cosine batch runs the single-query
 * passes with one segment per query.  Arguments, layouts and errors as
 * search_resident_metric; RT_ESTATE also when rt_enable_filtered was not
 * called on this engine.  Asynchronous on `stream`.
 */
rt_status search_resident_filtered_metric(rt_engine *e, const float *queries, int32_t q, int32_t k, int32_t metric,
                                          int32_t *out_idx, float *out_scores, void *stream);

/*
 * Plain top-k of a raw device array, no scoring ("CUDA Programming Model
 * Series 9: Efficient TopK", sections 2-3: two-stage selection).
 *   values     device, n elements of `dtype` (RT_DTYPE_INT32 or
 *              RT_DTYPE_FLOAT32), 4-byte aligned
 *   out_idx    device, k int32: element positions, best-first
 *   out_values device, k elements of `dtype`: the selected values, bit-for-bit
 *              copies of the input elements
 * Order: larger value first (int32 compared as integers, fp32 as floats so -0.0
 * ties +0.0), ties to the lower position.
 * RT_EINVAL: null pointer, unknown dtype, misaligned values, n < 1,
 * n > 2^31-1, k < 1, k > max_k, k > n.  Does not need a resident corpus.
 * Asynchronous on `stream`.
 */
rt_status topk_select(rt_engine *e, const void *values, int32_t dtype, int64_t n, int32_t k,
                      int32_t *out_idx, void *out_values, void *stream);

/*
 * topk_select for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same selection, kernels and answers as topk_select, with no engine.  It
 * allocates nothing -- no hipMalloc, hipFree or allocating library call -- and
 * keeps the kernels' scratch (merge-tree lists and arrival counters) in a
 * static device array of 4 MiB + 8 KiB that each GPU holds from the first call
 * on it until the process ends.
 *   values     device, n elements of `dtype`, 4-byte aligned, on the calling
 *              thread's current HIP device (as are the outputs and `stream`)
 *   out_idx    device, k int32: element positions, best-first
 *   out_values device, k elements of `dtype`: bit-for-bit copies of the input
 * Order and ties as topk_select.  RT_EINVAL: null pointer, unknown dtype,
 * misaligned values, n < 1, n > 2^31-1, k < 1, k > 1024, k > n (checked
 * before anything is enqueued; outputs untouched).  RT_EHIP: a HIP call or
 * launch failed (the next call first clears the counters with a fill kernel).
 * The array's size bounds the number of workgroups a call runs (fewer for
 * k > 256), not n.  Every call on one GPU shares that GPU's array and leaves
 * its counters zero: calls that overlap on one GPU (other streams, other
 * threads) race and must not be issued.  Asynchronous on `stream`.
 */
rt_status topk_select_noalloc(const void *values, int32_t dtype, int64_t n, int32_t k, int32_t *out_idx,
                              void *out_values, void *stream);

/*
 * Dynamic batching of concurrent single-query searches ("GPU-Resident Top-K
 * for Agentic RAG", section 1: many small agents retrieving against one
 * corpus; section 9: no concurrency between queries inside one engine).
 *
 * A batcher owns engine `e` from creation to rt_batcher_destroy: nothing else
 * may call `e` meanwhile (use rt_engine_create_shared for a second engine on
 * the same corpus).  Any number of host threads submit single queries; one
 * dispatcher thread gathers up to max_batch of them (1..min(32, e's max_q)),
 * waiting at most max_wait_us (0..1e6) after the first arrives, and runs them
 * as one batched search with k = the largest k in the batch; each request gets
 * the first k entries of its row.
 *   exact = 1: search_resident_filtered (requires rt_enable_filtered on e, else
 *     RT_ESTATE); every request's answer is bit for bit the plain single-query
 *     scan's.
 *   exact = 0: search_resident; scores from the batched fp32 matrix-core
 *     path, equal to the single-query scan's within fp32 rounding.
 * The corpus must be resident (RT_ESTATE otherwise); a request whose batch
 * finds the corpus changed (another depth, or fewer than k rows) fails with
 * RT_ESTATE.  RT_ENOMEM / RT_EHIP: allocation (pinned staging, a stream,
 * device buffers, the thread) failed.
 */
typedef struct rt_batcher rt_batcher; /* opaque */
rt_status rt_batcher_create(rt_engine *e, int32_t max_batch, int32_t max_wait_us, int32_t exact,
                            rt_batcher **out);
/*
 * Queue one query: `query` is host memory with the corpus depth's d floats,
 * copied before the call returns; 1 <= k <= min(e's max_k, resident rows).
 * out_idx / out_scores: host memory of k entries each, written before the
 * request completes; keep them valid until rt_batcher_wait returns for the
 * ticket, or until rt_batcher_destroy returns.  *out_ticket identifies the
 * request.  Thread-safe.  RT_EINVAL: bad argument; RT_ESTATE: the batcher is
 * being destroyed.
 */
rt_status rt_batcher_submit(rt_batcher *b, const float *query, int32_t k, int32_t *out_idx, float *out_scores,
                            uint64_t *out_ticket);
/*
 * Block until the request completes; returns its status (the search's, or
 * RT_ESTATE as above).  Wait for every ticket exactly once (RT_EINVAL for an
 * unknown or already-waited ticket).  Thread-safe.
 */
rt_status rt_batcher_wait(rt_batcher *b, uint64_t ticket);
/* out4 = {batches run, queries served, largest batch, queries waiting}. */
rt_status rt_batcher_stats(rt_batcher *b, int64_t *out4);
/* Serve every queued request (its outputs are written, as if waited for),
 * stop the dispatcher and free the batcher (not the engine).  No other thread
 * may be inside, or enter, any rt_batcher_* call on `b` once this is called. */
void rt_batcher_destroy(rt_batcher *b);

/* Static, human-readable name of a status code. */
const char *rt_status_string(rt_status s);

/* The last hipError_t value recorded by the engine (0 if none). */
int32_t rt_last_hip_error(const rt_engine *e);

/*
 * Kernel timing for measurement.  While enabled (on != 0), every search or
 * select records HIP events on its stream around its kernels; after the stream
 * has finished, rt_profile_read returns the last call's device times in
 * milliseconds: [0] = the whole call, [1] = its first kernel when it ran two
 * (the batched scoring kernel of a batch, the first (bf16 or fp8) pass of a
 * filtered search, the bound pass of a filtered batch; 0 otherwise), [2] = the rest (the streaming top-K kernel: scoring or
 * raw-array selection, per-block lists and the merge tree), i.e. [0] - [1].  The events
 * are created by rt_engine_create.  RT_EINVAL on NULL arguments.
 */
rt_status rt_profile_enable(rt_engine *e, int32_t on);
rt_status rt_profile_read(rt_engine *e, float *ms3);

/*
 * Read-bandwidth reference for measurements (the achievable ceiling that the
 * scan is compared with): `reps` launches on `stream` of a plain streaming
 * kernel that reads the resident fp32 corpus once each (its first
 * 16 * floor(n * d / 4) bytes, a contiguous chunk per wave, non-temporal
 * 16-byte loads, eight in flight per lane, 4 waves per CU) and does no other
 * work; the launches are timed with
 * the engine's events (so the last call's rt_profile_read times are replaced)
 * and synchronised, and *out_ms receives the average device time per launch.
 * The engine's merge-tree scratch may receive one word per wave.  RT_EINVAL on a
 * NULL engine or out_ms or reps < 1; RT_ESTATE before an upload.
 */
rt_status rt_read_probe(rt_engine *e, int32_t reps, void *stream, float *out_ms);

/*
 * Engine limits and state, for callers and tests: out7 receives
 * [max_n, max_d, max_k, max_q, resident_n, resident_d, device].
 */
rt_status rt_engine_info(const rt_engine *e, int64_t *out7);

/*
 * Host-side argument checks, exported so they can be tested without a GPU.
 * They apply exactly the rules the entry points above apply before enqueuing
 * anything, given the engine limits and resident sizes as plain numbers
 * (resident_n = 0 means no corpus).  Pointers are only tested for NULL.
 */
rt_status rt_check_create(int64_t max_n, int32_t max_d, int32_t max_k, int32_t max_q);
rt_status rt_check_upload(int64_t max_n, int32_t max_d, const void *corpus, int64_t n, int32_t d);
rt_status rt_check_search(int32_t max_k, int32_t max_q, int64_t resident_n, const void *queries,
                          int32_t q, int32_t k, const void *out_idx, const void *out_scores);
rt_status rt_check_search_metric(int32_t max_k, int32_t max_q, int64_t resident_n, const void *queries,
                                 int32_t q, int32_t k, int32_t metric, const void *out_idx, const void *out_scores);
rt_status rt_check_select(int32_t max_k, const void *values, int32_t dtype, int64_t n, int32_t k,
                          const void *out_idx, const void *out_values);

/*
 * The two constants of search_resident_filtered's bound for depth d, host-only
 * (no GPU needed): out2 = [cb, delta], where a row x with bf16 score a and
 * fp32 score s satisfies |a - s| <= cb |q| |x| + delta max(|q|, 1).
 * cb = (2^-8 + gamma_d (2 + 2^-8)) (1 + 2^-10), rounded up to fp32, with
 * gamma_d = d 2^-24 / (1 - d 2^-24): bf16 keeps 8 significant bits, so
 * rounding to nearest changes an element by at most 2^-8 of its magnitude, and
 * gamma_d bounds the fp32 summation error of each sum relative to the sum of
 * |terms| <= |q| |x| (Cauchy-Schwarz); the factor (1 + 2^-10) absorbs the fp32
 * rounding of the bound itself.  delta = 4 d 2^-126 covers values and partial
 * results below 2^-126.  RT_EINVAL for d < 1 or a NULL out2.
 */
rt_status rt_filter_bounds(int32_t d, float *out2);

/*
 * The constants of the batched first pass of search_resident_filtered,
 * host-only: out3 = [cr, cx, delta] with
 *   |a - s| <= |q| (cr |x - bf16(x)| + cx |x|) + delta max(|q|, 1) max(|x|, 1),
 * where a is the bf16 matrix-core sum of bf16(x) against the query split into
 * two bf16 parts (hi = bf16(q), lo = bf16(q - hi)) and s the single-query
 * scan's fp32 score.  |x - bf16(x)| is computed per row with the bf16 copy and
 * rounded up.  cr = (1 + 2^-16) (1 + 2^-10) and cx = (2^-16 + gamma_d + 1.02 g)
 * (1 + 2^-10), each rounded up to fp32: Cauchy-Schwarz on the row's rounding
 * error against the split query (|hi + lo| <= (1 + 2^-16) |q|), 2^-16 for the
 * split's own error, gamma_d = d 2^-24 / (1 - d 2^-24) for the scan's fp32 sum,
 * and g = 8 d 2^-24 / (1 - 8 d 2^-24) for the matrix core's fp32 accumulation
 * of the 2 d exact products in any order and rounding direction, with room to
 * spare, on sum |bf16(x)| (|hi| + |lo|) <= 1.02 |x| |q|; the factor (1 + 2^-10)
 * absorbs the fp32 evaluation of the bound.  delta = 16 d 2^-126 covers
 * values, products and partial sums below 2^-126.  RT_EINVAL for d < 1 or a
 * NULL out3.
 */
rt_status rt_filter_bounds_batched(int32_t d, float *out3);

/*
 * The constants of the fp8 first pass, host-only: out3 = [cr, cx, delta] with
 *   |a - s| <= |q| (cr |x - x~| + cx |x|) + delta max(|q|, 1) max(sc, 1),
 * where x~ = sc dec(codes) is the stored row (sc its power-of-two scale,
 * |x - x~| computed per row from the codes and rounded up), a = sc times the
 * fp32 sum of dec(codes) q and s the single-query scan's fp32 score.  The row's
 * part cr |x - x~| + cx |x| is computed once per upload (rounded up to fp32).
 * cr = (1 + gamma_d) (1 + 2^-10), cx = 2 gamma_d (1 + 2^-10), each rounded up
 * to fp32, gamma_d = d 2^-24 / (1 - d 2^-24): Cauchy-Schwarz on the rounding
 * error vector, gamma_d for a's fp32 sum over sum |x~ q| <= (|x| + |x - x~|) |q|
 * and gamma_d for the scan's.  delta = 4 d 2^-126 covers underflow.  RT_EINVAL
 * for d < 1 or a NULL out3.
 */
rt_status rt_filter_bounds_fp8(int32_t d, float *out3);

/*
 * The cosine arithmetic of the scans and of the filtered search, evaluated on
 * the host by the same source the kernels compile (host-only, no GPU needed;
 * for tests and for callers reproducing a decision of the filter).
 * rt_cosine_score: acc / (qnorm rnorm) in fp32, or -inf when that fp32
 * product is not positive (search_resident_metric's cosine epilogue).
 * rt_filter_cosine_bounds: out2 = [hi, lo], the bounds the first pass of the
 * filtered cosine search derives from inner-product bounds a - e <= acc <= a + e
 * ("GPU-Resident Top-K for Agentic RAG", section 4, Step 2, the cosine
 * branch): fl(a +- e) / fl(qnorm rnorm) widened by 2^-20 relative and FLT_MIN
 * absolute; (+inf, -inf) when known == 0 (an overflowed bound), (-inf, -inf)
 * when the product of norms is not positive; a quotient that overflows gives
 * the infinite bound on its side.  RT_EINVAL for a NULL out2.
 * Range of the cosine (both paths): the fp32 inner product and the fp32
 * product of the norms must be normal numbers; a pair whose |q| |x|
 * underflows in fp32 (below ~1e-45) scores -inf like a zero row.
 */
float rt_cosine_score(float acc, float qnorm, float rnorm);
rt_status rt_filter_cosine_bounds(int32_t known, float a, float e, float qnorm, float rnorm, float *out2);

#ifdef __cplusplus
}
#endif
#endif /* RESIDENT_TOPK_H */
