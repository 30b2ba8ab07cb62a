/*
 * atopk.h -- C ABI of libatopk.so: exact and bucketed top-k selection and
 * top-K sparse-attention decode on AMD Instinct MI355X (gfx950).
 *
 * What is computed (pages cited by title and section):
 *  - "Approximate Top-k for Increased Parallelism" (Pith review page),
 *    "The reading" and "What carries the argument": the exact top-k of a row,
 *    and the two-stage approximation of it -- positions dealt round-robin
 *    into b buckets, the k_b best of each bucket kept, and the best k of
 *    those b*k_b survivors taken when there are more than k of them.  The
 *    benchmark protocol in the reference list works on an (m, n) matrix x.
 *  - "Recall Before You Rank: Similarity-Guided Top-K Reuse ..." (fugumt
 *    page), Abstract: the decode step of Top-K sparse attention -- every
 *    cached key is scored against the new query, the K best are kept, and
 *    the softmax-weighted sum of values runs over those K keys alone.
 *  - STARC (Pith review page), Figure 3 caption: per head the query is one
 *    row of d_h values, the keys and values L such rows.
 *
 * Conventions shared by every entry point
 *  - Order: value descending, ties to the LOWER index.  -0.0 equals +0.0.
 *    NaN inputs are a precondition violation (result unspecified, no fault).
 *  - Bucket of element i is i mod b (interleaved).  Bucket r holds
 *    ceil((n - r) / b) elements; every bucket must hold at least k_b of them.
 *  - Returned values are bit copies of the selected input elements.
 *  - Indices are int32 positions inside the row (0 <= idx < n).
 *  - All pointers except `stream` are DEVICE pointers owned by the caller.
 *    The library never allocates, frees or synchronises: it enqueues kernels
 *    on `stream` (a hipStream_t; NULL = the default stream) and returns.  A
 *    caller-provided workspace (`ws`, at least the size the matching
 *    *_workspace query returns, 256-byte aligned) holds intermediate results.
 *    The workspace and outputs must not be in use by other work on other
 *    streams until the enqueued work completes.
 *  - Every call validates all arguments on the host before any launch and
 *    returns a status; on error nothing is written.  No C++ exception leaves
 *    the library.  Device faults surface at the caller's next synchronisation.
 *  - The library runs only on gfx950; any other device gives
 *    ATOPK_ERR_UNSUPPORTED.  It is thread safe (the only state is a one-time
 *    per-device property cache).
 */
#ifndef ATOPK_H
#define ATOPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types of x / out_vals */
typedef enum atopk_dtype { ATOPK_F32 = 0, ATOPK_BF16 = 1 } atopk_dtype;

/* status codes */
enum {
  ATOPK_OK = 0,
  ATOPK_ERR_NULL = 1,        /* a required pointer is NULL                        */
  ATOPK_ERR_SHAPE = 2,       /* m < 0, n < 1, ldx < n, k < 1, k > n, ctx < 1, ...  */
  ATOPK_ERR_PARAM = 3,       /* b < 1, kb < 1, b*kb < k, kb > floor(n / b),
                                element pointers not aligned to their size, ...   */
  ATOPK_ERR_UNSUPPORTED = 4, /* dtype, d != 128, kb > 16, k > 8192, n >= 2^31, arch */
  ATOPK_ERR_WORKSPACE = 5,   /* ws NULL or smaller than the query says, misaligned */
  ATOPK_ERR_HIP = 6          /* the HIP runtime refused a launch or a query        */
};

#define ATOPK_MAX_K 8192
#define ATOPK_MAX_KB 16

/* Static, human-readable text for a status code. */
const char* atopk_status_str(int status);

/* Library version as 10000*major + 100*minor + patch. */
int atopk_version(void);

/*
 * Measurement aid for benchmarks and profilers (not needed to use the
 * library).  After atopk_stage_events(events, count), the calling thread's
 * following entry-point calls record events[j] (caller-created hipEvent_t
 * handles, cast to void*) on their stream right after enqueuing their j-th
 * kernel, counting from 0 across calls until the next atopk_stage_events;
 * marks beyond `count` are counted but record nothing.  With an event
 * recorded by the caller before the call, the differences of consecutive
 * events give each kernel's duration (the stages of the path: scoring and
 * stage 1, stage 2, softmax-V).  count == 0 (events may be NULL) turns it
 * off.  atopk_stage_count() returns the number of marks since the last
 * atopk_stage_events on this thread.  The array must stay valid while on.
 * Recording events between kernels adds a little time to a call; the
 * library's results do not change.  ATOPK_ERR_PARAM for count < 0 or a
 * NULL array with count > 0.
 */
int atopk_stage_events(void* const* events, int count);
int atopk_stage_count(void);

/*
 * Exact top-k of every row of x.
 *   x         [m, ldx] row-major, dtype `dtype`; row r is x[r*ldx .. r*ldx+n).
 *   out_vals  [m, k] same dtype as x; out_idx [m, k] int32.  Row r lists the
 *             k greatest values of row r, value descending then index ascending.
 * Limits: 1 <= k <= min(n, 8192), n < 2^31.  m == 0 is a no-op.  x and
 * out_vals must be aligned to the element size, out_idx to 4 bytes
 * (ATOPK_ERR_PARAM otherwise); rows need no further alignment.
 */
int atopk_exact_workspace(int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, size_t* ws_bytes);
int atopk_exact(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k,
                void* out_vals, int32_t* out_idx, void* ws, size_t ws_bytes, void* stream);

/*
 * Two-stage bucketed top-k (stage 1: exact top-kb of each of b interleaved
 * buckets; stage 2 when final_exact != 0: exact top-k of the b*kb candidates).
 *   final_exact != 0: out_* are [m, k], sorted like atopk_exact.
 *   final_exact == 0: out_* are [m, b*kb], bucket-major: slot r*kb + j is the
 *                     j-th best element of bucket r.
 * Requires 1 <= b <= n, 1 <= kb <= floor(n / b), k <= b*kb (the invariant
 * b*k_b >= k), kb <= 16, k <= 8192, b*kb <= 2^20.  (b, kb) = (1, k) runs the
 * exact path (same result).
 */
int atopk_bucketed_workspace(int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, int64_t b,
                             int64_t kb, int final_exact, size_t* ws_bytes);
int atopk_bucketed(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, int64_t b,
                   int64_t kb, int final_exact, void* out_vals, int32_t* out_idx, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * atopk_bucketed for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops, harnesses that forbid allocation): the
 * same arguments and results without the workspace, which comes from a
 * device array inside the library of ATOPK_NOALLOC_SCRATCH_BYTES per GPU,
 * held from the library's first use on that GPU until the process ends.
 * Shapes whose workspace (atopk_bucketed_workspace) exceeds that size give
 * ATOPK_ERR_WORKSPACE before anything runs.  The call allocates nothing and
 * calls no allocating routine.  All calls on one GPU share the array, so two
 * such calls that may run at the same time on one GPU (different streams or
 * unordered threads) race: order them on one stream.
 */
#define ATOPK_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int atopk_bucketed_noalloc(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, int64_t b,
                           int64_t kb, int final_exact, void* out_vals, int32_t* out_idx, void* stream);

/* bucket assignments for atopk_bucketed_ex */
typedef enum atopk_assignment {
  ATOPK_INTERLEAVED = 0, /* bucket of i = i mod b (what atopk_bucketed uses)    */
  ATOPK_CONTIGUOUS = 1   /* bucket of i = floor(i * b / n): runs of consecutive */
} atopk_assignment;

/*
 * atopk_bucketed with a choice of bucket assignment.  "Approximate Top-k for
 * Increased Parallelism" (Pith review page), Figures 6 and 8 captions,
 * compares interleaved buckets with contiguous ones (recall on correlated
 * inputs, runtime); the page gives no formula for the contiguous buckets, and
 * the reading taken here is b runs of consecutive positions, bucket(i) =
 * floor(i * b / n) (sizes differ by at most one).  Arguments, outputs and
 * limits as atopk_bucketed; ATOPK_CONTIGUOUS with final_exact additionally
 * needs b*kb <= 8192 and uses no workspace.  An unknown assignment gives
 * ATOPK_ERR_PARAM.
 */
int atopk_bucketed_ex_workspace(int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, int64_t b,
                                int64_t kb, int final_exact, int assignment, size_t* ws_bytes);
int atopk_bucketed_ex(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, int64_t b,
                      int64_t kb, int final_exact, int assignment, void* out_vals, int32_t* out_idx,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * Top-K sparse-attention decode for one layer, one new token per sequence.
 *   q      [batch, hq, d] bf16 (contiguous)
 *   K, V   [batch, hkv, ctx_stride, d] bf16; key j of (batch i, KV head h) is
 *          K[((i*hkv + h)*ctx_stride + j)*d ...]; the first ctx rows are used.
 *   scale  score multiplier (usually 1/sqrt(d)); s_j = scale * <q, K_j>,
 *          accumulated in fp32 and scaled in fp32.
 *   Selection per QUERY head h (KV head h / (hq/hkv)): (b, kb) = (1, k_sel)
 *   is the exact Top-K; otherwise bucketed with b interleaved buckets of the
 *   ctx keys, k_b per bucket, and an exact final Top-K when b*kb > k_sel.
 *   out      [batch, hq, d] bf16 = softmax over the selected scores (maximum
 *            subtracted, fp32) times the selected V rows, rounded to nearest.
 *   sel_idx  [batch, hq, k_sel] int32, nullable: selected keys, score desc.
 *   scores   [batch, hq, ctx] fp32, nullable: every score (debug dump, costs
 *            bandwidth).
 * Requires d == 128, hq % hkv == 0, hq/hkv <= 8, ctx_stride >= ctx >= 1,
 * 1 <= k_sel <= min(ctx, 8192), b*kb >= k_sel, kb <= floor(ctx / b).
 */
int atopk_sparse_attn_decode_workspace(int64_t batch, int64_t hq, int64_t hkv, int64_t ctx,
                                       int64_t d, int64_t k_sel, int64_t b, int64_t kb,
                                       size_t* ws_bytes);
int atopk_sparse_attn_decode(const void* q, const void* K, const void* V, int64_t batch, int64_t hq,
                             int64_t hkv, int64_t ctx, int64_t ctx_stride, int64_t d, float scale,
                             int64_t k_sel, int64_t b, int64_t kb, void* out, int32_t* sel_idx,
                             float* scores, void* ws, size_t ws_bytes, void* stream);

/*
 * Candidate-set rerank decode ("Recall Before You Rank: Similarity-Guided
 * Top-K Reuse ..." (fugumt page), Abstract: the supports of the most similar
 * cached queries are united with a recent window and only that compact
 * candidate set is reranked with exact current-query scores).  This is the
 * rerank step; the cache of query / support pairs and the fallback policy
 * are the caller's.
 *   q, K, V, scale, ctx, ctx_stride, d, out   as atopk_sparse_attn_decode.
 *   cand    [batch, hq, cand_stride] int32 DEVICE array, row (i, h) holding
 *           ncand candidate key indices of query head h (entries outside
 *           [0, ctx) are skipped; repeats count once); NULL when ncand == 0.
 *   window  the last `window` keys [ctx - window, ctx) are candidates too.
 *   Per query head: the exact Top-k_sel of the candidate set by score (ties
 *   to the lower index) -- the whole set when it holds fewer keys -- then
 *   softmax and value aggregation over it.
 *   sel_idx [batch, hq, k_sel] int32, nullable: selected keys, score desc,
 *           padded with -1 when the set holds fewer than k_sel keys.
 *   scores  [batch, hq, ctx] fp32, nullable: the score of every candidate
 *           key written at its position (other positions are not written;
 *           a debug dump, as in atopk_sparse_attn_decode).
 * Requires d == 128, hq % hkv == 0, 1 <= ctx <= 262144, ctx_stride >= ctx,
 * 1 <= window <= ctx, 0 <= ncand <= cand_stride, ncand + window <= 8192,
 * 1 <= k_sel <= 8192, 16-byte aligned q, K, V.  The workspace (size from
 * atopk_sparse_attn_rerank_workspace, 256-byte aligned) holds the scored
 * candidate keys between the scoring and the selection kernels.
 */
int atopk_sparse_attn_rerank_workspace(int64_t batch, int64_t hq, int64_t hkv, int64_t ctx, int64_t ncand,
                                       int64_t window, size_t* ws_bytes);
int atopk_sparse_attn_rerank(const void* q, const void* K, const void* V, int64_t batch, int64_t hq, int64_t hkv,
                             int64_t ctx, int64_t ctx_stride, int64_t d, float scale, const int32_t* cand,
                             int64_t ncand, int64_t cand_stride, int64_t window, int64_t k_sel, void* out,
                             int32_t* sel_idx, float* scores, void* ws, size_t ws_bytes, void* stream);

/*
 * Expected recall of the bucketed top-k ("Approximate Top-k for Increased
 * Parallelism" (Pith review page), "What carries the argument", Eq. (1)) in
 * its finite-n form: the expected share of the true top-k kept by stage 1
 * for an iid row of n distinct values in b interleaved buckets (buckets of
 * ceil(n/b) or floor(n/b) elements).  Host only.  Needs 1 <= k <= n,
 * 1 <= b <= n, 1 <= kb <= floor(n / b), b*kb >= k (ATOPK_ERR_SHAPE /
 * ATOPK_ERR_PARAM otherwise).
 */
int atopk_expected_recall(int64_t n, int64_t k, int64_t b, int64_t kb, double* recall);

/*
 * Measured (b, kb) chooser (same page: "Core claim" and "If this is right" --
 * the recall model picks (b, kb) for a target accuracy without rerunning the
 * task; more buckets with kb = 1 when k is small against n, a small kb > 1
 * with b*kb near k when k is a large fraction of n).  For each kb in
 * {1, 2, 4, 8, 16} the smallest power-of-two b whose expected recall
 * (atopk_expected_recall) is >= min_recall, and the next larger b, are
 * timed on the caller's rows x together with the exact top-k (recall 1);
 * candidates keep b*kb <= 8192.  The fastest is returned in *b, *kb (the
 * exact top-k as b = 1, kb = k), its expected recall in *recall and its
 * measured time per call in *us (both nullable), and out_vals / out_idx
 * ([m, k], as atopk_bucketed with final_exact) hold its result.
 * Arguments and limits as atopk_exact, plus 0 <= min_recall <= 1; the
 * workspace is the largest any candidate needs (atopk_choose_workspace).
 * BLOCKS the calling thread until the timing launches on `stream` finish
 * (HIP events), so it cannot be captured into a graph; the caller keeps the
 * answer for later calls of the same shape.
 */
int atopk_choose_workspace(int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, double min_recall,
                           size_t* ws_bytes);
int atopk_choose(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, double min_recall,
                 void* out_vals, int32_t* out_idx, void* ws, size_t ws_bytes, void* stream, int64_t* b,
                 int64_t* kb, double* recall, float* us);

#ifdef __cplusplus
}
#endif

#endif /* ATOPK_H */
