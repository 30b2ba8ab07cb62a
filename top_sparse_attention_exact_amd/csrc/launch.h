// Internal launchers: the host API (api.cpp) validates arguments and sizes
// the workspace, then calls these to enqueue kernels on a stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace atopk {

// Measurement aid behind atopk_stage_events: records the calling thread's
// next stage event (if any) on the stream after a kernel launch.
void stage_mark(hipStream_t s);

// Every kernel launch of the library goes through this: the launch, then the
// stage mark.
#define ATOPK_LAUNCH(kernel, grid, block, shmem, stream, ...)                 \
  do {                                                                       \
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);     \
    ::atopk::stage_mark(stream);                                             \
  } while (0)

// Element types (match atopk_dtype) plus pre-built 64-bit keys.
enum InKind { IN_F32 = 0, IN_BF16 = 1, IN_KEY64 = 2 };

// ---- bucketed stage 1 ------------------------------------------------------

// Fast stage 1: register queues over 16-byte loads.  Grid rows x splits.
// Writes `lists_per_row` sorted k_b-lists per bucket to `lists`
// ([m][lists_per_row][b][kb] keys).
struct BucketPlan {
  int threads;        // workgroup size
  int splits;         // workgroups per row
  int64_t chunk;      // elements per workgroup (multiple of threads * vec)
  int lists_per_row;  // k_b-lists per bucket and row written by stage 1
  bool fast;          // register-queue kernel (else one thread per bucket)
};
BucketPlan plan_bucketed(int dtype, int64_t m, int64_t n, int64_t b, int64_t kb, bool aligned);

// With direct_done non-null, stage 1 may write the result itself (one split
// per row, lists merged in LDS: the bucket-major candidates, or the sorted
// top-k when b * kb <= 64); *direct_done then tells the caller to skip the
// finish.
hipError_t launch_bucket_stage1(const BucketPlan& p, const void* x, int dtype, int64_t m, int64_t n,
                                int64_t ldx, int64_t b, int64_t kb, uint64_t* lists, hipStream_t s, int64_t k = 0,
                                int final_exact = 0, void* out_vals = nullptr, int32_t* out_idx = nullptr,
                                bool* direct_done = nullptr);

// Merge the lists of every bucket; then either write the bucket-major
// candidates (final_exact == 0), or select and sort the final top-k
// (b * kb <= kFinishMaxCand), or write merged candidates to `cand_out`
// ([m][b*kb] keys) for the exact path to finish.  final_exact ==
// kFinishCertified: the exact top-k of the whole row, from the candidates
// plus a rescan of the buckets that may hide more of it (b*kb <= 8192).
constexpr int kFinishMaxCand = 8192;
constexpr int kFinishCertified = 3;
hipError_t launch_bucket_finish(const uint64_t* lists, int lists_per_row, int64_t m, int64_t n, int64_t b,
                                int64_t kb, int64_t k, int final_exact, const void* x, int dtype, int64_t ldx,
                                void* out_vals, int32_t* out_idx, uint64_t* cand_out, hipStream_t s);

// ---- exact top-k ------------------------------------------------------------

struct ExactPlan {
  int splits;       // workgroups per row in the first pass
  int64_t chunk;    // elements per workgroup
  int cap;          // LDS candidate capacity (keys)
};
ExactPlan plan_exact(int in_kind, int64_t m, int64_t n, int64_t k);

// Exact top-k over rows of `x` (values or 64-bit keys).  With splits > 1
// every workgroup writes its chunk's top-k keys to `part` ([m][splits][k]);
// otherwise sorted results go to out_vals / out_idx, the values being
// gathered from `src` (dtype src_dtype, row stride src_ld elements).
hipError_t launch_exact(const ExactPlan& p, const void* x, int in_kind, int64_t m, int64_t n, int64_t ld,
                        int64_t k, uint64_t* part, const void* src, int src_dtype, int64_t src_ld,
                        void* out_vals, int32_t* out_idx, hipStream_t s);

// ---- one workgroup per row (single launch, no workspace) -------------------

bool row_bucket_ok(int dtype, int64_t m, int64_t n, int64_t b, int64_t kb, bool aligned);
bool row_exact_ok(int dtype, int64_t m, int64_t n, int64_t k, bool aligned);
// Rows of at most 8192 elements, any alignment and any k: the whole row is
// ranked in LDS by one workgroup.
bool row_small_exact_ok(int dtype, int64_t m, int64_t n, int64_t k);
hipError_t launch_row_small_exact(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k,
                                  void* out_vals, int32_t* out_idx, hipStream_t s);
hipError_t launch_row_bucket(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, int64_t b,
                             int64_t kb, int final_exact, void* out_vals, int32_t* out_idx, hipStream_t s);
hipError_t launch_row_exact(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, void* out_vals,
                            int32_t* out_idx, hipStream_t s);

// Contiguous bucket assignment (bucket of i = floor(i * b / n)), one
// workgroup per row, no workspace.
bool row_contig_ok(int64_t n, int64_t b, int64_t kb, int final_exact);
hipError_t launch_row_contig(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, int64_t b,
                             int64_t kb, int final_exact, bool aligned, void* out_vals, int32_t* out_idx,
                             hipStream_t s);

// ---- wide fp32 rows: two streaming passes (values, then collect) -----------

struct WidePlan {
  bool ok;               // the shape fits this path
  int64_t b, kb;         // bucketing used (exact mode: a fixed one)
  int kbn;               // width of the value network (8 or 16)
  int64_t groups;        // 64-bucket groups per row
  int nchunks;           // waves per streaming workgroup (chunks of sweeps)
  int sweeps_per_chunk;
  int64_t blocks;        // streaming workgroups: rows * groups
  size_t vals_bytes, bucket_bytes, cand_bytes, row_bytes;
  // exact mode, one read: a sampled threshold, then a contiguous collect
  bool sampled;
  int sample_r;          // rank of the threshold among the row's samples
  int row_chunks;        // collect workgroups per row
  int steps_per_chunk;   // collect steps per workgroup
  int final_parts;       // final workgroups per row (they split the sort by value)
};
struct WideBuffers {
  float* vals;         // exact: top values per bucket
  float* thr;          // bucketed: T_r per (row, bucket)
  int* need;           // bucketed: ties each bucket takes
  uint64_t* cand;      // bucketed with final stage: the b * kb candidates
  float* rowthr;       // exact: lower bound of the k-th value per row
  int* row_cnt;        // exact: keys collected per row
  uint64_t* row_keys;  // exact: collected keys
};
WidePlan plan_wide(int dtype, int64_t m, int64_t n, int64_t k, int64_t b, int64_t kb, bool exact, bool final_exact);
hipError_t launch_wide(const WidePlan& p, const float* x, int64_t m, int64_t n, int64_t ldx, int64_t k, bool exact,
                       bool final_exact, const WideBuffers& w, void* out_vals, int32_t* out_idx, hipStream_t s);

// ---- decode -------------------------------------------------------------------

// scores[(i*hq + h)*ctx + j] = scale * <q[i, h], K[i, h / g, j]> (fp32).
hipError_t launch_decode_scores(const uint16_t* q, const uint16_t* K, int64_t batch, int64_t hq, int64_t hkv,
                                int64_t ctx, int64_t ctx_stride, float scale, float* scores, hipStream_t s);

// Fused decode: scoring + bucketed stage 1 per (batch, KV head, chunk), then
// merge + final Top-K + softmax-V per query head.
struct DecodePlan {
  bool fused;            // false: scores, selection and softmax-V as separate passes
  bool mfma;             // query-head groups: scores on the matrix cores
  int ppt;               // (head, bucket) pairs per thread in the scoring kernel
  int64_t chunk;         // keys per scoring workgroup (context-chunk mode)
  int nchunks;           // k_b-lists per (head, bucket) the finish merges
  int lgR;               // >= 0: bucket-range mode, 2^lgR buckets per scoring workgroup
  int tpp;               // bucket-range mode: threads folding one (head, bucket) pair
  int nsplit;            // scoring workgroups per (batch, KV head)
  size_t partial_bytes;  // k_b-lists in the workspace
};
DecodePlan plan_decode(int64_t batch, int64_t hq, int64_t hkv, int64_t ctx, int64_t k_sel, int64_t b, int64_t kb);
// certify != 0: (b, kb) is a certified plan for the exact Top-K and
// cert_buf a [B*Hq, ctx] fp32 buffer, scratch for the finish's rare
// full-row fallback.  The finish recomputes the scores of the buckets it
// rescans with kernel 1's arithmetic: certify == 1 for query-head groups
// (matrix cores), certify == 2 with one query head per KV head (packed dot
// products); any other pairing is rejected.  scores (nullable): every
// score, when the caller asks for them.
hipError_t launch_decode_fused(const DecodePlan& p, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                               int64_t batch, int64_t hq, int64_t hkv, int64_t ctx, int64_t ctx_stride, float scale,
                               int64_t k_sel, int64_t b, int64_t kb, uint64_t* partial, uint16_t* out,
                               int32_t* sel_idx, float* scores, int certify, float* cert_buf, hipStream_t s);

// Candidate-set rerank decode: per query head the given indices united with
// the last `window` keys, exact scores, Top-K, softmax-V.
constexpr int kRerankMaxCand = 8192;   // ncand + window
constexpr int kRerankMaxCtx = 262144;  // context covered by the LDS bitmap
size_t rerank_ws_bytes(int64_t batch, int64_t hq, int64_t ncand, int64_t window);
hipError_t launch_rerank(const uint16_t* q, const uint16_t* K, const uint16_t* V, int64_t batch, int64_t hq,
                         int64_t hkv, int64_t ctx, int64_t ctx_stride, float scale, const int32_t* cand, int64_t ncand,
                         int64_t cand_stride, int64_t window, int64_t k_sel, uint16_t* out, int32_t* sel_idx,
                         float* scores, void* ws, hipStream_t s);

// out[r] = softmax(sel_vals[r]) @ V[sel_idx[r]] for r = i*hq + h.
hipError_t launch_sparse_softmax_v(const float* sel_vals, const int32_t* sel_idx, const uint16_t* V,
                                   int64_t batch, int64_t hq, int64_t hkv, int64_t ctx_stride, int64_t k_sel,
                                   uint16_t* out, hipStream_t s);

}  // namespace atopk
