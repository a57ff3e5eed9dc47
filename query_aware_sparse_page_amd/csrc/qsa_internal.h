// Internal (host-side) interface between the C ABI layer and the kernel
// translation units of libqsa. Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// Shapes and table pointers every launcher needs, validated by the ABI layer.
struct LaunchCommon {
  int B = 0, Hq = 0, Hkv = 0, D = 0, G = 0;
  bool bf16 = true;
  const void* k_pool = nullptr;
  const void* v_pool = nullptr;
  int num_phys = 0;
  const int* page_indptr = nullptr;
  const int* page_indices = nullptr;
  const int* seq_lens = nullptr;
  // Device error word (checked mode) or NULL: kernels that skip a page
  // because a table or selection entry is out of range OR one of the
  // kErr* bits into it (see report_bad below).
  unsigned int* err = nullptr;
};

// Bits of the device error word.
constexpr unsigned int kErrPhys = 1u;   // a physical page id outside [0, num_phys_pages)
constexpr unsigned int kErrSel = 2u;    // a selected logical page outside [0, n_b)
constexpr unsigned int kErrCount = 4u;  // a sel_count entry outside [1, k]
constexpr unsigned int kErrExchange = 8u;  // a fused row's arrival counter was neither 0 nor 1

// Records a skipped out-of-range entry in the error word (one lane per call
// site is enough; every lane may call it). A vector atomic to global memory.
__device__ __forceinline__ void report_bad(unsigned int* err, unsigned int bit) {
  if (err != nullptr) __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Split-K decode work split: `chunk` pages per work unit (a multiple of 4,
// one quarter per wave), `max_units` units for the longest (b, h) row.
struct DecodePlan {
  int chunk = 4;       // units: pages per unit; stream: pages per wave (rounded up)
  int max_units = 0;   // units: most units of one row; stream: most partial slots of one row
  bool stream = false; // the stream split (decode_stream_kernel)
  int waves = 0;       // stream: waves in the launch (a multiple of 4)
};

// Sequences whose per-sequence tables the stream split keeps in LDS.
constexpr int kStreamMaxB = 1024;

// Per-unit partial results: part_o [units, G, D] (unnormalised, relative to
// the unit's running max), part_ml [units, G, 2] = (max in log2 units, sum).
struct Partials {
  float* o = nullptr;
  float* ml = nullptr;
  int* row_slots = nullptr;  // stream split: [rows][2] first and last wave of each row
};

hipError_t launch_build_meta(const LaunchCommon& c, int max_pages, int tail_pages, void* meta,
                             int stride, hipStream_t stream);

hipError_t launch_build_centroids(const LaunchCommon& c, int max_pages, int tail_pages, void* cent,
                                  int stride, hipStream_t stream);

hipError_t launch_score(const LaunchCommon& c, const void* q, void* meta, int refresh_tail,
                        float* group_scores, float* head_scores, int stride, hipStream_t stream);

// Centroid scores q . c_j (records of one 256-byte row), same outputs.
hipError_t launch_score_centroid(const LaunchCommon& c, const void* q, void* cent,
                                 int refresh_tail, float* group_scores, float* head_scores,
                                 int stride, hipStream_t stream);

// Longest row the top-K kernel handles (pages): 1024 threads x 16 keys.
constexpr int kTopkMaxPages = 16384;

hipError_t launch_topk(const LaunchCommon& c, const float* group_scores, int stride, int k,
                       int* sel, int* sel_count, int* sel_phys, hipStream_t stream);

// Approximate top-K (digit_bits-wide digits, early stop at min_confident
// confident pages, random fill from the threshold bin driven by row_rand).
// passes (nullable) receives each row's number of radix passes.
hipError_t launch_topk_approx(const LaunchCommon& c, const float* group_scores, int stride, int k,
                              int digit_bits, int min_confident, const uint32_t* row_rand,
                              int* sel, int* sel_count, int* sel_phys, int* passes,
                              hipStream_t stream);

// Split-K decode (partials into `part`) followed by the log-sum-exp merge of
// each (b, hq) into out / lse, which also folds in n_prefix shared-prefix
// partials per query row laid out [Hkv][n_prefix][B*G] (cascade).
hipError_t launch_decode(const LaunchCommon& c, const void* q, const int* sel, const int* sel_count,
                         int k, float scale_log2, const DecodePlan& plan, Partials part,
                         Partials prefix, int n_prefix, float* out, float* lse,
                         hipStream_t stream);

// Fused per-row sparse decode step (score -> top-K -> attention -> merge in
// one workgroup per (b, h) row, or two workgroups per row that each attend
// over half of the selected pages and merge through a RowExchange). Rows of at most
// kRowMaxPages pages, at most kRowMaxSelect selected pages.
constexpr int kRowMaxPages = 4096;
constexpr int kRowMaxSelect = 512;

// centroid: meta holds centroid rows (256 bytes per page) scored as q . c
// instead of [m | M] records scored by the bound.
// The exchange of the fused kernel's two workgroups per row (both NULL: one
// workgroup per row): per-row arrival counters (zero before the first call,
// left zero by every call) and per (row, part) partial results of
// G * (D + 2) floats.
struct RowExchange {
  unsigned int* counters = nullptr;
  float* partials = nullptr;
};
hipError_t launch_sparse_row(const LaunchCommon& c, const void* q, void* meta, int stride,
                             int refresh_tail, int k, float scale_log2, const RowExchange& x,
                             bool centroid, float* out, float* lse, float* group_scores, int* sel,
                             int* sel_count, hipStream_t stream);

// Steps 2-4 for rows of at most kShortMaxPages pages, one wave per (b, h)
// row (bf16, D = 128, G = 4 or 8, the bound scorer): scores with the
// tail-page refresh, the top-k pages, attention over them, and the LSE merge
// with n_prefix prefix partials per query row ([Hkv][n_prefix][B*G], as the
// cascade prefix writes them; n_prefix = 0: none). Outputs as
// launch_sparse_row's.
constexpr int kShortMaxPages = 64;
hipError_t launch_short_rows(const LaunchCommon& c, const void* q, void* meta, int stride, int refresh_tail,
                             int k, float scale_log2, Partials prefix, int n_prefix, float* out, float* lse,
                             float* group_scores, int* sel, int* sel_count, hipStream_t stream);

// The log-sum-exp merge alone: per query row, the row's split-K partials
// (units of `chunk` pages over its seq_lens pages, at most max_units; the
// layout of launch_decode's) and n_prefix prefix partials, into out / lse
// (D = 128).
hipError_t launch_merge(const LaunchCommon& c, Partials part, int max_units, int chunk, Partials prefix,
                        int n_prefix, float* out, float* lse, hipStream_t stream);

// A selective cascade step's two halves in one launch, ahead of
// launch_merge: the cascade prefix's workgroups (4 waves each) interleaved
// with the short-row workgroups of the suffix rows, whose unmerged partials
// go to suffix (one unit per row: [rows][G][D] and [rows][G][2]). A CU holds
// two of these workgroups, so the prefix's products and the suffix rows'
// loads share it (cus_per_xcd: the device's CUs per XCD, which sets the
// interleave). bf16, D = 128, G = 4 or 8, suffix rows of at most
// kShortMaxPages pages.
hipError_t launch_cascade_overlap(const LaunchCommon& c, const void* q, const int* prefix_pages, int prefix_len,
                                  int n_splits, float scale_log2, Partials prefix, void* meta, int stride,
                                  int refresh_tail, int k, Partials suffix, float* group_scores, int* sel,
                                  int* sel_count, int cus_per_xcd, hipStream_t stream);

// Cascade prefix on the matrix cores (bf16, D = 128): partials per
// (KV head, split, query row).
hipError_t launch_cascade_prefix(const LaunchCommon& c, const void* q, const int* prefix_pages,
                                 int prefix_len, int n_splits, float scale_log2, Partials prefix,
                                 hipStream_t stream);

}  // namespace qsa
