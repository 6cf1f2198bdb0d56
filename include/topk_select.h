/*
 * topk_select.h - C ABI of the MI355X (gfx950) index-only TopK selector.
 *
 * What is computed.  The web article "How to Use FlagOS's New Triton-TLE
 * Language to Build a TopK Selector Faster Than FlashInfer" (below: the TopK
 * article) describes the selector of DeepSeek-Sparse-Attention-style
 * decoding: in section 01, per query row of indexer logits over the
 * historical tokens, return the indices of the k largest logits, indices
 * only, without a full sort; in section 02, a radix select that maps floats to
 * order-preserving unsigned integers, histograms their digits from the most
 * significant end, keeps the bucket holding the k-th element, and finally
 * collects every element above the threshold value T followed by elements
 * equal to T in scan order (so ties at T go to the lowest index); in section
 * 5, -1 as the value of an output slot that holds no index.
 *
 * Readings of points the article leaves open (fixed by this ABI):
 *  - logits are fp32, row-major [rows, n], row stride n;
 *  - the valid length of row r is lengths[r] clamped to [0, n] (n for every
 *    row when lengths is NULL); positions at or past it are never returned;
 *  - when a row's valid length L is below k, the row's output holds every
 *    index 0..L-1 followed by k-L entries of -1;
 *  - -0.0 and +0.0 are equal (they tie); infinities and subnormals are
 *    ordinary values; NaN logits are outside the contract (no error is
 *    raised, the result for such a row is unspecified but memory-safe);
 *  - the output order within a row is unspecified, but it is a function of
 *    the row's values and the launch shape alone (every position comes from
 *    a block scan or an exact rank, none from the order in which atomic
 *    operations or workgroups complete), so repeated calls on the same input
 *    write identical bytes; the selected set is exact and unique.
 *    topk_select_sorted gives the set ordered by value.
 *
 * All pointers named "device" point to memory on the calling thread's current
 * HIP device.  The library never takes ownership of caller memory.
 * No C++ exception crosses this interface.
 */
#ifndef TOPK_SELECT_H_
#define TOPK_SELECT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TOPK_SELECT_VERSION 1

/* Status codes returned by every entry point. */
enum {
    TOPK_SELECT_SUCCESS = 0,
    TOPK_SELECT_ERROR_INVALID_VALUE = 1, /* bad argument; nothing was enqueued */
    TOPK_SELECT_ERROR_OUT_OF_MEMORY = 2, /* workspace allocation failed; nothing was enqueued */
    TOPK_SELECT_ERROR_LAUNCH = 3,        /* a HIP call or the kernel launch failed */
    TOPK_SELECT_ERROR_NO_DEVICE = 4,     /* no usable HIP device is current */
    TOPK_SELECT_ERROR_DEVICE_FLAG = 5,   /* a kernel raised a device-side error flag */
    TOPK_SELECT_ERROR_CAPTURE = 6,       /* scratch would have to be allocated while the stream is
                                            being captured into a graph; nothing was enqueued */
    TOPK_SELECT_ERROR_SCRATCH_LIMIT = 7  /* topk_select_no_alloc: the input needs more than its fixed
                                            scratch; nothing was enqueued */
};

/* hipStream_t, passed as an opaque pointer so this header needs no HIP headers.
 * NULL is the default (null) stream of the current device. */
typedef void* topk_select_stream_t;

/*
 * topk_select - per row, the indices of the k largest valid logits (the TopK
 * article, sections 01, 02 and 5; readings above).
 *
 *   logits   device, const float[rows * n], row-major, row stride n, at least
 *            4-byte aligned (16-byte alignment of rows is used when present,
 *            but not required).  Read only.
 *   rows     number of rows, >= 0.  rows == 0 is a successful no-op.
 *   n        row length, 1 <= n <= 2^30.
 *   lengths  device, const int32_t[rows], or NULL.  Valid length per row; read
 *            on the device and clamped to [0, n].
 *   k        number of indices per row, 1 <= k <= n.
 *   out_idx  device, int32_t[rows * k], row-major.  Written only by the
 *            enqueued work; must not overlap logits or lengths.
 *   stream   stream the work is enqueued on.  The call returns without
 *            waiting; results are ready when the stream reaches this point.
 *
 * Returns TOPK_SELECT_SUCCESS when the work was enqueued.  Host-checkable
 * arguments are checked before any HIP call; on INVALID_VALUE nothing is
 * enqueued and out_idx is untouched.  The library keeps a scratch workspace
 * per (device, stream), allocated on first use and grown as needed (the first
 * call for a new (device, stream) or a larger shape allocates and clears it
 * with hipMalloc/hipMemsetAsync; later calls of that size allocate nothing).
 * A buffer replaced by a larger one is kept until
 * topk_select_release_workspace, so graphs captured earlier stay valid.
 * While the stream is being captured into a graph, a call that would have to
 * allocate returns TOPK_SELECT_ERROR_CAPTURE and enqueues nothing: call once
 * with the same (or a larger) shape on that stream before capturing.
 * Thread-safe: calls from several host threads are serialised on the host
 * while they enqueue; calls on different streams use different workspaces
 * and may run concurrently on the device (a row's workgroups wait only for
 * workgroups of the same launch that were dispatched before them, so no
 * co-residency is required).  Calls on one stream run in stream order.
 */
int topk_select(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k,
                int32_t* out_idx, topk_select_stream_t stream);

/*
 * topk_select_no_alloc - topk_select for callers that cannot allocate device
 * memory (code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * topk_select, with the same launch shapes, so the same output bytes.
 *
 * Scratch: a static device array of TOPK_SELECT_NO_ALLOC_SCRATCH_BYTES
 * (32 MiB) per device, held until the process ends; the call allocates
 * nothing (no hipMalloc/hipFree, no allocating library routine).  The first
 * call on a device looks the array up and clears it with a kernel on
 * `stream`, waiting for that kernel (returns TOPK_SELECT_ERROR_CAPTURE if
 * the stream is being captured then: make one call before capturing).
 * Shapes with one workgroup per row (rows >= the device's CU count) need
 * only 256 bytes of it; shapes that split a row over G workgroups need
 * rows * G * region * 8 bytes of candidate stage (region = the candidate
 * capacity of one workgroup, at most 7168) plus a row table, and are limited
 * to 256 rows.  An input beyond the limit returns
 * TOPK_SELECT_ERROR_SCRATCH_LIMIT and enqueues nothing (for example, one
 * row of n = 2^30, or 64 rows of n = 2^20; the configurations up to 64 rows
 * of n = 131072 and any row count >= the CU count fit).
 *
 * Every call on a device shares that device's array, and each call leaves
 * it cleared for the next: calls that overlap in time on one device (on
 * different streams, or from different host threads without ordering) race
 * on it and give wrong results.  Serialise them, e.g. on one stream.
 * topk_select_device_status reports (and clears) flags raised by these calls
 * as well, on the device current when it is called.
 */
#define TOPK_SELECT_NO_ALLOC_SCRATCH_BYTES (32u << 20)
int topk_select_no_alloc(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k,
                         int32_t* out_idx, topk_select_stream_t stream);

/*
 * topk_select_sorted - the same selection, each row in order: values
 * descending, equal values by index ascending, the -1 slots (rows whose
 * valid length L is below k) last.  The TopK article, section 02: the
 * radix_topk pseudocode's need_sorted option sorts the collected output in
 * descending order; the order among equal values is not stated there, the
 * one taken is the rule that selects them (lowest index first).
 *
 *   out_val  device, float[rows * k], or NULL (indices only).  out_val[j] is
 *            the logit at out_idx[j] bit for bit (-0.0 stays -0.0), and
 *            -INFINITY where out_idx[j] is -1.  Must not overlap logits,
 *            lengths or out_idx.
 *   other arguments, ownership and errors as for topk_select.
 *
 * The order is fully determined, so repeated calls give identical outputs.
 * Besides the workspace of topk_select, the (device, stream) keeps a second
 * scratch area (grown as needed with hipMalloc; no clearing): rows*k*4 bytes
 * of keys, plus 2*rows*kp*8 bytes when k > 8192 (kp = k rounded up to a
 * multiple of 8192).  The work: for k <= 2048 the workgroup that finishes a
 * row orders it itself (one launch; the split kernel from the keys it
 * records in that scratch); for larger k the selection kernel records the
 * key of every index it writes and a second launch orders them: the rank
 * kernel for few rows (rows * k^2 <= 2^25, k <= 4096), else one sort kernel
 * (k <= 8192) or a sort kernel and ceil(log2(kp/8192)) merge passes.
 */
int topk_select_sorted(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k,
                       int32_t* out_idx, float* out_val, topk_select_stream_t stream);

/*
 * topk_indexer_logits - the logits the selector is fed: the TopK article,
 * section 01, step 1 of DSA-style decoding (logits of the current query
 * against every historical token).  The article gives no formula; the one
 * computed (the reading taken) has H indexer heads sharing one key per token:
 *
 *   logits[r*n + t] = sum_h w[r*H + h] *
 *                     max(0, sum_i q[(r*H + h)*dim + i] * kc[r*kstride + t*dim + i])
 *
 * for t < L_r, and -INFINITY for L_r <= t < n (keys there are not read).
 *
 *   q        device, bf16 bit patterns, [rows, heads, dim], 16-byte aligned.
 *   kc       device, bf16 bit patterns: the keys of row r are the [n, dim]
 *            array at kc + r*kstride; 16-byte aligned.
 *   w        device, float [rows, heads].
 *   rows >= 0, n >= 1, 1 <= heads <= 64, dim one of 32, 64, 128.
 *   kstride  elements between the keys of consecutive rows: 0 (every row
 *            uses the same keys) or at least n*dim; a multiple of 8.
 *   lengths  device int32 [rows] or NULL: valid lengths, clamped to [0, n].
 *   logits   device, float [rows, n]; must not overlap the inputs.
 *
 * Products of bf16 values are exact in float; the sums run on the matrix
 * cores in float, in an unspecified order, so each logit lies within
 * (dim + heads + 2) * 2^-24 * sum_h |w| sum_i |q k| of the exact value.
 * Errors as for topk_select (INVALID_VALUE enqueues nothing).
 */
int topk_indexer_logits(const uint16_t* q, const uint16_t* kc, const float* w, int32_t rows, int32_t n,
                        int32_t heads, int32_t dim, int64_t kstride, const int32_t* lengths, float* logits,
                        topk_select_stream_t stream);

/*
 * topk_indexer_select - topk_indexer_logits, then topk_select on those
 * logits with the same lengths: the indexer and the selector of the
 * article's section 01, steps 1 and 2.  out_idx as for topk_select.
 *   out_logits  device, float [rows, n], receives the logits; or NULL, and
 *               they go to a scratch area of the (device, stream) of
 *               rows*n*4 bytes (grown with hipMalloc when needed).
 * Two kernels are enqueued (the logits, then the selection).
 */
int topk_indexer_select(const uint16_t* q, const uint16_t* kc, const float* w, int32_t rows, int32_t n,
                        int32_t heads, int32_t dim, int64_t kstride, const int32_t* lengths, int32_t k,
                        int32_t* out_idx, float* out_logits, topk_select_stream_t stream);

/*
 * topk_indexer_select_fused - the same result as topk_indexer_select (the
 * same index set; the order within a row is fixed, by the values and the
 * launch shape, but may differ from topk_indexer_select's), with the
 * selection's pass over the row moved into the logits kernel (the article's
 * section 01: step 1 producing step 2's input), so that the selection
 * afterwards reads candidates only:
 *   1. one kernel computes the logits (written to out_logits or scratch, as
 *      above); WGs holding every F-th group of 64 tokens (F a power of two,
 *      at most 64 groups per row) publish their keys and the row's bound,
 *      the sample's element of rank m + 4 sqrt(m) + 6, m = k * S / L for S
 *      sampled valid tokens; the other WGs wait for it and write their
 *      logits at or above it to per-WG regions;
 *   2. one WG per row gathers those candidates and selects the k largest
 *      on chip; when fewer than k or too many came out (the sample misled)
 *      it selects by passes over the logits row.
 * Taken when the candidates fit the finishing WG (about
 * k + 4 sqrt(k F) + 6 F + 256 <= 7168) and a row needs at most 512 WGs;
 * else this is topk_indexer_select.  Measured on MI355X it is slower than
 * topk_indexer_select (the bound exists only once the logits pass is done,
 * and the chain after it outlasts the selection on fresh logits); it is the
 * fused form of the producer, kept for comparison.
 * Scratch of the (device, stream), grown with hipMalloc: 4160 + 32768 bytes
 * per row (zeroed when allocated) and 8 bytes per logit of the row's
 * regions.  Waits are bounded as in topk_select (flag 1); a WG that gives
 * up makes its row be selected by passes over the logits, so the output
 * stays exact.  Errors as for topk_indexer_select.
 */
int topk_indexer_select_fused(const uint16_t* q, const uint16_t* kc, const float* w, int32_t rows, int32_t n,
                              int32_t heads, int32_t dim, int64_t kstride, const int32_t* lengths, int32_t k,
                              int32_t* out_idx, float* out_logits, topk_select_stream_t stream);

/*
 * topk_sparse_attention - attention over the selected positions: the TopK
 * article, section 01, step 3 of DSA-style decoding (attention computed only
 * on the keys and values of the k selected positions).  The article gives
 * no formula; computed (the reading taken) is plain scaled dot-product
 * attention of each query head over the slots of idx[r] that hold a
 * position, keys and values shared by the heads:
 *
 *   s_j = scale * q[r][h] . K[r][idx[r][j]],   p_j = exp(s_j) / sum_j' exp(s_j')
 *   out[(r*heads + h)*dim + c] = sum_j p_j * V[r][idx[r][j]][c]
 *
 *   q        device, bf16 bit patterns, [rows, heads, dim], 16-byte aligned.
 *   kc, vc   device, bf16: the keys / values of row r are the [n, dim]
 *            arrays at kc + r*kvstride / vc + r*kvstride; 16-byte aligned.
 *   idx      device, int32 [rows, k]: positions, e.g. topk_select's output;
 *            -1 or any value outside [0, n) holds no position.
 *   scale    finite score scale (commonly 1/sqrt(dim)).
 *   out      device, float [rows, heads, dim]; a row whose slots hold no
 *            position gets zeros.  Must not overlap the inputs.
 *   rows >= 0, n >= 1, 1 <= heads <= 64, dim one of 32, 64, 128, k >= 1,
 *   kvstride 0 (shared keys and values) or at least n*dim, a multiple of 8.
 *
 * Precision: bf16 products are exact in float and the scores are summed in
 * float; each softmax weight p is split into two bf16 terms, hi = bf16(p)
 * and lo = bf16(p - hi) (|p - hi - lo| <= 2^-16 p), for two P.V products on
 * the matrix cores summed in float.  Each output lies within
 *   (2 (dim + 2) 2^-24 smax + 2^-16 + (k + 64) 2^-24 + 2^-20) * sum_j p_j |V[idx_j][c]|
 * of the exact value, smax = max_j scale * sum_i |q_i K[idx_j]_i|.
 * Two kernels are enqueued (per chunk of C slots, then the combination): C
 * is 256 when that still makes at least 512 chunks in all, else 128 when
 * that does, else 64.  Scratch of rows * ceil(k/C) * heads * (dim + 2) * 4
 * bytes per (device, stream), grown with hipMalloc when needed.  Errors as
 * for topk_select.
 */
int topk_sparse_attention(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const int32_t* idx,
                          int32_t rows, int32_t n, int32_t heads, int32_t dim, int64_t kvstride, int32_t k,
                          float scale, float* out, topk_select_stream_t stream);

/*
 * Launch-shape description, filled by topk_select_plan and accepted by
 * topk_select_ex.  Performance only: every plan yields the same selected sets.
 *   variant       kernel variant id (0 .. topk_select_num_variants()-1)
 *   wgs_per_row   workgroups cooperating on one row (>= 1)
 *   block         threads per workgroup of the variant (output only)
 *   items         logits per thread per tile of the variant (output only)
 *   resident      1 when each workgroup keeps its whole slice on chip across
 *                 rounds, 0 when it re-reads its slice every round (output only)
 *   first_bits    width in bits of the first radix digit (8 or 12) (output only)
 */
typedef struct {
    int32_t variant;
    int32_t wgs_per_row;
    int32_t block;
    int32_t items;
    int32_t resident;
    int32_t first_bits;
} topk_select_plan_t;

/* The launch shape topk_select would use for (rows, n, k) on the current
 * device.  Returns INVALID_VALUE for arguments topk_select would reject. */
int topk_select_plan(int32_t rows, int32_t n, int32_t k, topk_select_plan_t* plan);

/* topk_select with an explicit launch shape (plan->variant, plan->wgs_per_row).
 * Used by tests to drive every kernel path and by tuning sweeps.  Returns
 * INVALID_VALUE when the shape cannot cover n or cannot be co-resident. */
int topk_select_ex(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k,
                   int32_t* out_idx, topk_select_stream_t stream, const topk_select_plan_t* plan);

/* topk_select_sorted with an explicit selection launch shape (as for
 * topk_select_ex; the sort that follows does not depend on it). */
int topk_select_sorted_ex(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k,
                          int32_t* out_idx, float* out_val, topk_select_stream_t stream,
                          const topk_select_plan_t* plan);

/* Number of kernel variants compiled into the library; fills the shape of
 * variant v (block, items, resident) into plan when v is in range. */
int topk_select_num_variants(void);
int topk_select_variant_info(int32_t v, topk_select_plan_t* plan);

/*
 * Waits for `stream`, then reads and clears the device-side error flags of
 * the workspace of (current device, stream) and stores them in *flags (0 when
 * none were raised or no workspace exists).  Flags: 1 = a wait for another
 * workgroup exceeded its time bound (2 s; the waiting workgroup then
 * finished its rows by itself, and its output is still exact), 2 = an
 * internal capacity check failed.  After flag 1 the workspace may hold
 * counts or candidates written after their row was finished; this call
 * clears the whole workspace then, and a later call on the stream is exact
 * only after it.  Returns DEVICE_FLAG when any flag was set, SUCCESS
 * otherwise.  The flags of topk_select_no_alloc calls on the current device
 * are read and cleared as well (wait for those calls first when they ran on
 * other streams).
 */
int topk_select_device_status(topk_select_stream_t stream, int32_t* flags);

/* Frees every cached workspace (all devices and streams).  The caller must
 * make sure no enqueued selection is still running. */
int topk_select_release_workspace(void);

/* Static, human-readable description of a status code. */
const char* topk_select_error_string(int status);

/* TOPK_SELECT_VERSION of the built library. */
int topk_select_version(void);

/*
 * topk_stream_read - the yardstick for the selection's memory traffic (the
 * article's roofline view: the selection is bound by reading the logits
 * once): reads `bytes` of device memory at `p` once with 16-byte loads
 * spread over every CU, and nothing else, so its rate is the read bandwidth
 * the HBM achieves for a plain stream.
 *
 *   p       device, 16-byte aligned, `bytes` readable.  Read only.
 *   bytes   a positive multiple of 16.
 *   sink    device, uint32_t[1]: written only in the (practically never
 *           taken) case that keeps the loads live; its value means nothing.
 *   stream  stream the launch is enqueued on (returns without waiting).
 *
 * Returns INVALID_VALUE (nothing enqueued) for a null or misaligned pointer
 * or a size that is zero or not a multiple of 16.
 */
int topk_stream_read(const void* p, size_t bytes, uint32_t* sink, topk_select_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TOPK_SELECT_H_ */
