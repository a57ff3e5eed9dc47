/*
 * libqsa - query-aware sparse paged decode for AMD MI355X (gfx950).
 *
 * Single-token decode attention over a paged KV cache with query-aware page
 * selection, as stated on the TinyServe page ("KV缓存优化的核心挑战与TinyServe
 * 解决方案"): per-page min/max key metadata (§2.1), an upper-bound page score
 * (§2.2), top-K page selection and attention over only the selected pages
 * (§2.3); plus a shared-prefix cascade merged by log-sum-exp (Quail page,
 * join attention). The page table follows PagedAttention (CS336 lecture 10
 * page, §9.2) and Vortex's (b, p, I) paged-layout view (Vortex digest page,
 * vTensor).
 *
 * Conventions for every call:
 *  - Ownership: the caller owns every buffer. The library never allocates or
 *    frees device memory and keeps no state between calls; scratch space is a
 *    caller-provided workspace of the size the *_workspace_size query returns.
 *    Calls that share a workspace must not run concurrently.
 *  - Ordering: work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream) and the call returns without synchronising. Outputs are valid
 *    once the stream reaches that point.
 *  - Pointers are device pointers unless named *_host.
 *  - Errors: every call returns a qsa_status; on failure nothing has been
 *    enqueued (argument errors) or the launch failed (QSA_ERR_DEVICE), and
 *    qsa_last_error() returns a message for the calling thread. Nothing
 *    throws across this interface.
 *  - Supported shapes: page_size 16; (dtype, head_dim) = (QSA_BF16, 128) or
 *    (QSA_F32, 64) - both make one (page, KV head) tile 4 KiB; group size
 *    g = Hq / Hkv in {1, 2, 4, 8}. Other shapes return QSA_ERR_UNSUPPORTED.
 *  - Robustness: a logical page index outside [0, n_b), a physical page id
 *    outside [0, num_phys_pages) or a sel_count outside [1, min(k, n_b)] is
 *    never dereferenced or followed: the page is skipped (treated as holding
 *    no tokens; a count is clamped). By default this is silent. In checked
 *    mode (qsa_set_checked below) every kernel that skips such an entry
 *    records it in a device error word, and the call then returns
 *    QSA_ERR_DEVICE naming what was out of range (its outputs are those of
 *    the skipping run).
 */
#ifndef QSA_H_
#define QSA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qsa_status {
  QSA_OK = 0,
  QSA_ERR_INVALID_ARG = 1, /* NULL pointer, inconsistent sizes, k < 1, ...   */
  QSA_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim/dtype/group size */
  QSA_ERR_WORKSPACE = 3,   /* workspace smaller than the size query returns */
  QSA_ERR_DEVICE = 4       /* a HIP launch or runtime call failed            */
} qsa_status;

typedef enum qsa_dtype { QSA_F32 = 0, QSA_BF16 = 1 } qsa_dtype;

/* Problem sizes. B = num_seqs, Hq = num_q_heads, Hkv = num_kv_heads
 * (Hq % Hkv == 0; query head hq belongs to KV head hq / (Hq/Hkv)),
 * D = head_dim, page_size = tokens per page (16). dtype is the element type
 * of q, both pools and the page metadata. B is at most 65535 (a launch grid
 * dimension); QSA_ERR_UNSUPPORTED otherwise. */
typedef struct qsa_dims {
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t dtype; /* qsa_dtype */
} qsa_dims;

/* A paged KV cache seen through a block table (CS336 page §9.2; Vortex's
 * (b, p, I)). Logical page j of sequence b lives at physical slot
 * page_indices[page_indptr[b] + j], for j < n_b = ceil(seq_lens[b] / 16);
 * the last page holds seq_lens[b] - 16 (n_b - 1) valid tokens. Table entries
 * beyond n_b are ignored. Physical slots may be shared between sequences
 * (prefix sharing) and are visited once per referencing sequence. */
typedef struct qsa_paged_kv {
  const void* k_pool;            /* [num_phys_pages, Hkv, page_size, D]  */
  const void* v_pool;            /* same shape as k_pool                  */
  int32_t num_phys_pages;
  const int32_t* page_indptr;    /* [B + 1], non-decreasing               */
  const int32_t* page_indices;   /* [page_indptr[B]] physical slots       */
  const int32_t* seq_lens;       /* [B] tokens per sequence, each >= 1    */
  const int32_t* seq_lens_host;  /* [B] host copy of seq_lens (planning)  */
} qsa_paged_kv;

/* Step 1 - per-page bounding-box metadata (TinyServe §2.1; refreshed every
 * decode step per §5.3). For each sequence b, logical page j < n_b and KV
 * head h, read through the page table: meta[b][h][j][0][i] = min and
 * meta[b][h][j][1][i] = max over the page's valid tokens of K[p][h][t][i]
 * (p the physical slot), under IEEE total order (-0 < +0), so the values are
 * exact copies of key elements (bit-exact). meta: [B, Hkv, stride, 2, D] in
 * dims->dtype, stored in logical page order so that scoring streams each
 * (b, h) row; stride >= max_b n_b. Entries j >= n_b, and pages whose physical
 * slot is out of range, are not written. tail_pages = 0 rebuilds every page;
 * tail_pages = n > 0 rebuilds only the last n pages of each sequence (the
 * per-step update after a token is appended). Reads kv->k_pool only. */
qsa_status qsa_build_page_meta(const qsa_dims* dims, const qsa_paged_kv* kv,
                               int32_t tail_pages, void* meta, int32_t stride,
                               hipStream_t stream);

/* Step 2 - upper-bound page score (TinyServe §2.2):
 *   s[b][hq][j] = sum_i q[b][hq][i] * (q[b][hq][i] > 0 ? M_j[i] : m_j[i])
 * with (m_j, M_j) the metadata of logical page j of sequence b for KV head
 * hq / g, accumulated in fp32 (no softmax scale: the ranking does not
 * depend on it). group_scores[b][h][j] = max over the g query heads of KV
 * head h (this keeps the bound: it is >= every group head's largest q.k in
 * the page). Layouts: q [B, Hq, D] in dtype; meta [B, Hkv, stride, 2, D] as
 * written by qsa_build_page_meta with the same stride; group_scores
 * [B, Hkv, stride] fp32; head_scores [B, Hq, stride] fp32 or NULL. Entries
 * n_b <= j < stride are written as -inf. Requires stride >= max_b n_b.
 * refresh_tail = 1 first rebuilds each sequence's last page's metadata from
 * kv->k_pool exactly as qsa_build_page_meta(tail_pages = 1) would (writing
 * meta) and scores with it - the per-decode-step update of §5.3 fused into
 * this call; refresh_tail = 0 only reads meta. */
qsa_status qsa_score_pages(const qsa_dims* dims, const void* q,
                           const qsa_paged_kv* kv, void* meta,
                           float* group_scores, float* head_scores,
                           int32_t stride, int32_t refresh_tail,
                           hipStream_t stream);

/* Alternative page summary - the centroid (Vortex digest, cache phase: each
 * block's mean key, the summary its Block Top-K indexer scores). For each
 * sequence b, logical page j (physical slot read through the page table) and
 * KV head h: cent[b][h][j][:] = the mean of the page's valid keys, element
 * by element, rounded once to dims->dtype (bf16: nearest, ties to even; the
 * sum of a page's keys is exact in the fp64 the kernel sums in unless their
 * magnitudes span more than ~2^41, and means below 2^-126 in magnitude are
 * not supported). Layout [B, Hkv, stride, D] in dims->dtype, logical page
 * order (one 256-byte row per page). tail_pages and stride as in
 * qsa_build_page_meta. Reads kv->k_pool only. */
qsa_status qsa_build_page_centroids(const qsa_dims* dims, const qsa_paged_kv* kv,
                                    int32_t tail_pages, void* cent, int32_t stride,
                                    hipStream_t stream);

/* Centroid page score (Vortex digest, indexer phase of Block Top-K):
 * s[b][hq][j] = q[b][hq] . cent[b][hq / g][j], fp32 accumulation;
 * group_scores[b][h][j] = max over the g query heads of KV head h (the same
 * combination as qsa_score_pages; the centroid score is not an upper bound
 * of the page's logits, it is their mean up to the centroid's rounding).
 * Outputs, -inf padding, stride and refresh_tail (which rebuilds the tail
 * page's centroid from kv->k_pool, as qsa_build_page_centroids(tail_pages =
 * 1) would) as in qsa_score_pages. The result feeds qsa_topk_pages and
 * qsa_paged_decode unchanged. */
qsa_status qsa_score_pages_centroid(const qsa_dims* dims, const void* q,
                                    const qsa_paged_kv* kv, void* cent,
                                    float* group_scores, float* head_scores,
                                    int32_t stride, int32_t refresh_tail,
                                    hipStream_t stream);

/* Step 3 - top-K page selection per (sequence, KV head) (TinyServe §2.3; the
 * radix select of the Vortex digest, optimisations). For each (b, h):
 * the K_eff = min(k, n_b) logical pages with the largest group score, ties
 * (equal fp32 values, -0 == +0) broken towards the smaller page index.
 * Outputs: sel [B, Hkv, k] int32, ascending page order, padded with -1;
 * sel_count [B, Hkv] = K_eff; sel_phys [B, Hkv, k] (or NULL) = the physical
 * slots of sel, -1 padded. Rows of up to 16384 pages (stride <= 16384, i.e.
 * 256K tokens); longer rows return QSA_ERR_UNSUPPORTED. Workspace:
 * qsa_topk_workspace_size bytes (may be 0; ws may then be NULL). */
qsa_status qsa_topk_pages(const qsa_dims* dims, const qsa_paged_kv* kv,
                          const float* group_scores, int32_t stride, int32_t k,
                          int32_t* sel, int32_t* sel_count, int32_t* sel_phys,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* Step 3, approximate - the randomised radix top-K of the Vortex digest
 * (optimisations; efficiency analysis): the radix select stops once it holds
 * enough confident pages and draws the rest at random from the threshold
 * bin. Per (b, h) row, on the order-preserving keys of the fp32 scores (-0
 * taken as +0), most significant digit first, starting at the highest bit
 * where the row's keys differ, digit_bits (4..13) bits per pass:
 *   - each pass keeps the bin holding the K_eff-th largest key; the pages in
 *     higher bins are confident (certainly among the top K_eff);
 *   - the passes stop when the confident pages number >= min_confident,
 *     when the kept bin holds exactly the pages still needed, or when no
 *     bit is left;
 *   - the r pages still needed are drawn from the kept bin's c pages, taken
 *     in page order with ranks i = 0..c-1, by systematic sampling with a
 *     random start st = floor(row_rand[b][h] * c / 2^32): rank i is drawn
 *     when (i*r + st) mod c >= c - r (each bin page has probability r/c).
 * min_confident >= k never stops on confidence, so the result is the exact
 * top-K except that equal scores at the threshold are drawn at random.
 * row_rand: [B, Hkv] uint32 random words, device (the caller draws them).
 * Outputs as in qsa_topk_pages (ascending page order, -1 padding,
 * sel_phys nullable); passes (nullable) [B, Hkv] int32 = radix passes run
 * (0 when K_eff = n_b or all scores are equal). Rows of up to 16384 pages.
 * No workspace. Errors: QSA_ERR_INVALID_ARG for NULL inputs, k < 1,
 * digit_bits outside 4..13, min_confident < 0 or stride < max n_b;
 * QSA_ERR_UNSUPPORTED for stride > 16384. */
qsa_status qsa_topk_pages_approx(const qsa_dims* dims, const qsa_paged_kv* kv,
                                 const float* group_scores, int32_t stride,
                                 int32_t k, int32_t digit_bits,
                                 int32_t min_confident, const uint32_t* row_rand,
                                 int32_t* sel, int32_t* sel_count,
                                 int32_t* sel_phys, int32_t* passes,
                                 hipStream_t stream);

/* Step 4 - split-K flash-decode over the selected pages (TinyServe §2.3
 * stages 3-4; flash decoding per the CS336 page §9.2 and the Quail page).
 * For each (b, hq) with h = hq / g: attention of q[b][hq] over the valid
 * tokens of the pages sel[b][h][0 .. sel_count[b][h]) of sequence b, read in
 * place through the page table; sel == NULL means every page (dense paged
 * decode - the same kernels, so selecting every page gives bit-identical
 * results). z_t = sm_scale * q.k_t; out = sum_t e^{z_t} v_t / sum_t e^{z_t}
 * (fp32 [B, Hq, D]); lse = ln sum_t e^{z_t} (fp32 [B, Hq], or NULL).
 * sel: [B, Hkv, k] logical page indices; sel_count [B, Hkv] (each in
 * [1, min(k, n_b)]); k is the row stride of sel. Pages are split into work units that
 * run in parallel and are merged by log-sum-exp. Workspace:
 * qsa_decode_workspace_size(dims, seq_lens_host, sel ? k : 0). */
qsa_status qsa_paged_decode(const qsa_dims* dims, const void* q,
                            const qsa_paged_kv* kv, const int32_t* sel,
                            const int32_t* sel_count, int32_t k, float sm_scale,
                            float* out, float* lse, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* Step 5 - shared-prefix cascade decode (Quail page, join attention: all
 * queries attend the shared anchor once, each sequence attends its own
 * suffix, the two partial results merge by LSE rescaling). The prefix is
 * prefix_len tokens stored once at physical slots prefix_pages[0 ..
 * ceil(prefix_len/16)) of kv->k_pool / kv->v_pool; it is attended whole by
 * every sequence, as a dense [B*g, D] x [D, prefix_len] contraction per KV
 * head on the matrix cores. The suffix is kv's per-sequence table, attended
 * as in qsa_paged_decode (all pages when sel == NULL, else the selection).
 * out/lse as in qsa_paged_decode, over prefix ∪ suffix. Requires bf16,
 * head_dim 128. Workspace: qsa_cascade_workspace_size(...). */
qsa_status qsa_cascade_decode(const qsa_dims* dims, const void* q,
                              const int32_t* prefix_pages, int32_t prefix_len,
                              const qsa_paged_kv* kv, const int32_t* sel,
                              const int32_t* sel_count, int32_t k,
                              float sm_scale, float* out, float* lse, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/* qsa_paged_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, contract, plan and kernels as
 * qsa_paged_decode (so the results are bit-identical to it), minus the
 * workspace. The split-K partials go to a static device array of
 * QSA_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until the
 * process ends; the call allocates nothing. A batch whose partials need more
 * (qsa_decode_workspace_size above the limit) returns QSA_ERR_WORKSPACE
 * before any device work. Every call on one GPU shares that GPU's array and
 * leaves its contents behind (nothing needs clearing: every partial a call
 * reads is written earlier in the same call); calls that overlap on one GPU
 * (other streams, other threads) race on it and must be serialised by the
 * caller. */
#define QSA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
qsa_status qsa_paged_decode_noalloc(const qsa_dims* dims, const void* q,
                                    const qsa_paged_kv* kv, const int32_t* sel,
                                    const int32_t* sel_count, int32_t k,
                                    float sm_scale, float* out, float* lse,
                                    hipStream_t stream);

/* Steps 2-4 as one call: one decode step of the sparse path (TinyServe §3.2
 * fuses page scoring, top-K selection and the sparse attention into one
 * kernel, with the scores kept on chip). Computes exactly what
 * qsa_score_pages(refresh_tail) -> qsa_topk_pages(k) -> qsa_paged_decode(sel)
 * compute: the same group scores (equal values; a -0 score may be returned
 * as +0), the same selection, and
 * out / lse within fp32 rounding of qsa_paged_decode on that selection.
 * meta / stride / refresh_tail as in qsa_score_pages (meta is written only
 * when refresh_tail = 1); k, out, lse as in qsa_topk_pages / qsa_paged_decode.
 * Optional outputs (each may be NULL): group_scores [B, Hkv, stride] fp32,
 * sel [B, Hkv, k] int32 (ascending, -1 padded), sel_count [B, Hkv] int32.
 * path selects the kernels:
 *   QSA_PATH_FUSED - one launch: one workgroup per (b, h) row scores,
 *     selects, attends and merges in LDS; rows of at most 4096 pages
 *     (max_b n_b <= 4096) with min(k, max_b n_b) <= 512, else
 *     QSA_ERR_UNSUPPORTED. With at most half as many rows as the GPU has
 *     CUs, two workgroups share each row, each attending over half of the selected
 *     pages, and the second to finish merges the two partial results
 *     through the workspace (the result does not depend on which one that
 *     is). Rows of at most 64 pages with bf16 groups of 4 or 8 heads and the
 *     bound scorer take one wave per row instead;
 *   QSA_PATH_SPLIT - the separate score, top-K and split-K decode kernels,
 *     which spread one row over many workgroups (long rows, few rows);
 *   QSA_PATH_AUTO - FUSED when supported and B * Hkv >= 64, else SPLIT.
 * Workspace: qsa_sparse_decode_workspace_size(...) with the same path, 16-byte
 * aligned; too small returns QSA_ERR_WORKSPACE. For the fused path it is 0
 * (ws may be NULL) unless rows are shared: then its first B * Hkv * 4 bytes
 * are per-row arrival counters, which must be zero before the workspace's
 * first use with this path; every fused call leaves them zero, but any other
 * call given the same workspace may overwrite them (zero them again before
 * the next fused call; checked mode reports counters that are not). A
 * workspace serves one call at a time (calls that overlap on one GPU need
 * their own). */
typedef enum qsa_path {
  QSA_PATH_AUTO = 0,
  QSA_PATH_FUSED = 1,
  QSA_PATH_SPLIT = 2
} qsa_path;

qsa_status qsa_sparse_decode(const qsa_dims* dims, const void* q,
                             const qsa_paged_kv* kv, void* meta, int32_t stride,
                             int32_t refresh_tail, int32_t k, float sm_scale,
                             float* out, float* lse, float* group_scores,
                             int32_t* sel, int32_t* sel_count, int32_t path /* qsa_path */,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* qsa_sparse_decode with the centroid scorer (Vortex digest, Block Top-K's
 * mean-key summary): cent holds the centroid rows written by
 * qsa_build_page_centroids ([B, Hkv, stride, D] in dims->dtype); computes
 * exactly what qsa_score_pages_centroid(refresh_tail) -> qsa_topk_pages(k) ->
 * qsa_paged_decode(sel) compute (refresh_tail rebuilds the tail page's
 * centroid). Paths, limits, optional outputs and workspace as for
 * qsa_sparse_decode (the same qsa_sparse_decode_path and workspace size). */
qsa_status qsa_sparse_decode_centroid(const qsa_dims* dims, const void* q,
                                      const qsa_paged_kv* kv, void* cent,
                                      int32_t stride, int32_t refresh_tail,
                                      int32_t k, float sm_scale, float* out,
                                      float* lse, float* group_scores,
                                      int32_t* sel, int32_t* sel_count,
                                      int32_t path /* qsa_path */, void* ws, size_t ws_bytes,
                                      hipStream_t stream);

/* One decode step of the selective cascade (Quail page, join attention; the
 * suffix selection of TinyServe §2.2-§2.3): computes exactly what
 * qsa_score_pages(refresh_tail) -> qsa_topk_pages(k) on the suffix pages ->
 * qsa_cascade_decode(sel) compute - the same group scores (a -0 score may
 * come back as +0), the same selection, and out / lse within fp32 rounding
 * of qsa_cascade_decode on that selection. The prefix (prefix_pages,
 * prefix_len) is attended whole by every sequence on the matrix cores; kv,
 * meta, stride, refresh_tail, k and the optional outputs (group_scores, sel,
 * sel_count: each may be NULL) are those of qsa_sparse_decode for the
 * suffix tables. Suffix rows of at most 64 pages with bf16 groups of 4 or 8
 * heads run in two launches: one grid that interleaves the prefix's
 * workgroups (1024-token splits on the matrix cores) with the suffix rows'
 * (one wave per (sequence, KV head) row that scores, selects and attends),
 * so that a CU runs one of each at once, then the log-sum-exp merge of the
 * prefix and suffix partials. Other shapes run the prefix kernel and the
 * separate score, top-K and split-K kernels with the prefix partials folded
 * into the merge. Requires bf16, head_dim 128.
 * Workspace: qsa_cascade_sparse_decode_workspace_size(...). */
qsa_status qsa_cascade_sparse_decode(const qsa_dims* dims, const void* q,
                                     const int32_t* prefix_pages, int32_t prefix_len,
                                     const qsa_paged_kv* kv, void* meta, int32_t stride,
                                     int32_t refresh_tail, int32_t k, float sm_scale,
                                     float* out, float* lse, float* group_scores,
                                     int32_t* sel, int32_t* sel_count, void* ws,
                                     size_t ws_bytes, hipStream_t stream);
size_t qsa_cascade_sparse_decode_workspace_size(const qsa_dims* dims, int32_t prefix_len,
                                                const int32_t* suffix_lens_host,
                                                int32_t stride, int32_t k);

/* The kernels qsa_sparse_decode will run for these arguments (QSA_PATH_FUSED
 * or QSA_PATH_SPLIT), in *chosen. */
qsa_status qsa_sparse_decode_path(const qsa_dims* dims, const int32_t* seq_lens_host,
                                  int32_t stride, int32_t k, int32_t path /* qsa_path */,
                                  qsa_path* chosen);

/* Workspace sizes in bytes (0 on invalid arguments). k <= 0 means dense. */
size_t qsa_topk_workspace_size(const qsa_dims* dims, int32_t max_pages, int32_t k);
size_t qsa_decode_workspace_size(const qsa_dims* dims, const int32_t* seq_lens_host, int32_t k);
size_t qsa_cascade_workspace_size(const qsa_dims* dims, int32_t prefix_len,
                                  const int32_t* suffix_lens_host, int32_t k);
size_t qsa_sparse_decode_workspace_size(const qsa_dims* dims, const int32_t* seq_lens_host,
                                        int32_t stride, int32_t k, int32_t path /* qsa_path */);

/* The decode work split the library will use. bf16 groups of 4 or more
 * query heads with at most 1024 sequences take the stream split: every wave
 * gets an equal share of all rows' pages; *chunk_pages is that share (rounded
 * up) and *max_units the most partial results one (b, h) row can have.
 * Otherwise rows are cut into work units: *chunk_pages pages per unit and
 * *max_units the most units of one row. *stream (may be NULL) is 1 for the
 * stream split, else 0. Returns QSA_ERR_INVALID_ARG on bad arguments,
 * QSA_ERR_UNSUPPORTED when a row would need more than 65535 units. */
qsa_status qsa_decode_plan(const qsa_dims* dims, const int32_t* seq_lens_host,
                           int32_t k, int32_t* chunk_pages, int32_t* max_units,
                           int32_t* stream);

/* Checked mode (process-wide; off unless the environment holds QSA_CHECKED
 * set to anything but "" or "0", or qsa_set_checked(1) is called). The
 * range checks that keep a corrupted page table, selection or count from
 * being dereferenced run in every call (see Robustness above); checked mode
 * adds their report: each compute call clears a per-device error word on
 * its stream, passes it to its kernels, then waits for the stream and
 * returns QSA_ERR_DEVICE if any kernel skipped an out-of-range entry, or if
 * a fused-path row counter in the workspace was neither 0 nor 1 (a workspace
 * not zeroed before its first use; that call's outputs are not valid). The
 * wait makes checked calls synchronous, so they are meant for debugging and
 * tests, not for graph capture; concurrent checked calls on one device share
 * the word, so a report may name another call's entry. The top-K calls read
 * no pool and report nothing. (The CS336 lecture 10 page, §9.2: the block
 * table is the indirection these checks guard.) */
void qsa_set_checked(int32_t on);
int32_t qsa_get_checked(void);

/* floor(budget_tokens / page_size): a token budget in whole pages (>= 0). */
int32_t qsa_budget_pages(int32_t budget_tokens, int32_t page_size);

/* status: a qsa_status value (others give "unknown status"). Enumerated
 * arguments (status, path, dims->dtype) are passed as int32_t, so a value
 * outside the enumeration is an argument error rather than undefined
 * behaviour of the library. */
const char* qsa_status_string(int32_t status);
const char* qsa_last_error(void);
int32_t qsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H_ */
