// The two halves of a selective cascade step in one launch (Quail page, join
// attention: the shared anchor attended once, merged with each sequence's
// suffix by log-sum-exp; the suffix is a sparse decode step of the TinyServe
// page, §2.2-§3.2): the prefix workgroups of cascade_prefix.h and the suffix
// rows' workgroups of short_row.h in one grid, followed by the merge.
//
// Alone, the prefix kernel keeps each CU's SIMDs busy with products and
// softmax while HBM idles, and the short-row kernel waits on HBM while the
// SIMDs idle. Both roles here use 4-wave workgroups, two of which fit a CU,
// and the grid alternates between the roles every 8 workgroups (one per
// XCD), so a CU usually holds one of each: the suffix rows' loads are in
// flight while the prefix's products run. The suffix rows leave their
// unmerged partials (one unit per row) for launch_merge, which also folds in
// the prefix partials.
#include <algorithm>

#include "cascade_prefix.h"
#include "short_row.h"

namespace qsa {
namespace {

constexpr int kOvWaves = 4;  // waves per workgroup, both roles
static_assert(shortrow::kShortWaves == kOvWaves, "the roles share the workgroup size");

template <int G>
union OverlapShared {
  cascade::CascadeShared p;
  shortrow::ShortShared<G> s;
};

// Block -> (role, index within the role). Blocks go round-robin over the 8
// XCDs (block mod 8), and an XCD's blocks fill its CUs in turn (its k-th
// block on CU k mod C, C = `chunk` CUs per XCD), so groups of 8 consecutive
// blocks are dealt out in chunks of C groups that alternate between the
// roles while both have groups left: an XCD's first C blocks are prefix
// workgroups and its next C suffix workgroups, one of each per CU. The index
// keeps the block's position within its group, so the prefix workgroups keep
// their XCD (index mod 8), as in the prefix kernel. Returns false for blocks
// past their role's count.
__device__ __forceinline__ bool place(int block, int n_pre_blocks, int n_suf_blocks, int chunk, bool* pre,
                                      int* idx) {
  const int gp = (n_pre_blocks + 7) / 8, gs = (n_suf_blocks + 7) / 8;
  const int cp = (gp + chunk - 1) / chunk, cs = (gs + chunk - 1) / chunk;
  const int both = min(cp, cs);
  const int g = block >> 3;
  const int ci = g / chunk, o = g - ci * chunk;
  int rc;
  if (ci < 2 * both) {
    *pre = (ci & 1) == 0;
    rc = ci >> 1;
  } else {
    *pre = cp > cs;
    rc = both + (ci - 2 * both);
  }
  const int rg = rc * chunk + o;  // the group within the role
  *idx = rg * 8 + (block & 7);
  return *idx < (*pre ? n_pre_blocks : n_suf_blocks);
}

template <int G>
__global__ void __launch_bounds__(64 * kOvWaves) __attribute__((amdgpu_waves_per_eu(2)))
cascade_overlap_kernel(const bf16s* __restrict__ q, const bf16s* __restrict__ k_pool,
                       const bf16s* __restrict__ v_pool, int num_phys, int B, int Hkv,
                       const int* __restrict__ prefix_pages, int prefix_len, int split_tokens, int n_splits,
                       float scale_log2, float* __restrict__ pre_o, float* __restrict__ pre_ml, int n_pre_blocks,
                       bf16s* __restrict__ meta, int stride, const int* __restrict__ page_indptr,
                       const int* __restrict__ page_indices, const int* __restrict__ seq_lens, int refresh_tail,
                       int k, float* __restrict__ suf_o, float* __restrict__ suf_ml, int n_suf_blocks,
                       int chunk, float* __restrict__ group_scores, int* __restrict__ sel, int* __restrict__ sel_count,
                       unsigned int* __restrict__ err) {
  __shared__ OverlapShared<G> sh;
  bool pre;
  int idx;
  if (!place(blockIdx.x, n_pre_blocks, n_suf_blocks, chunk, &pre, &idx)) return;  // (whole workgroup)
  if (pre) {
    cascade::prefix_block<kOvWaves>(sh.p, idx, threadIdx.x, reinterpret_cast<const uint16_t*>(q),
                                    reinterpret_cast<const uint16_t*>(k_pool),
                                    reinterpret_cast<const uint16_t*>(v_pool), num_phys, B, Hkv, G, prefix_pages,
                                    prefix_len, split_tokens, n_splits, scale_log2, pre_o, pre_ml, err);
  } else {
    shortrow::short_row_block<G>(sh.s, idx, threadIdx.x, q, meta, stride, k_pool, v_pool, num_phys, B, Hkv,
                                 page_indptr, page_indices, seq_lens, refresh_tail, k, scale_log2, nullptr,
                                 nullptr, 0, nullptr, nullptr, group_scores, sel, sel_count, err, suf_o, suf_ml);
  }
}

}  // namespace

hipError_t launch_cascade_overlap(const LaunchCommon& c, const void* q, const int* prefix_pages, int prefix_len,
                                  int n_splits, float scale_log2, Partials prefix, void* meta, int stride,
                                  int refresh_tail, int k, Partials suffix, float* group_scores, int* sel,
                                  int* sel_count, int cus_per_xcd, hipStream_t stream) {
  using namespace cascade;
  if (!c.bf16 || c.D != kCD || (c.G != 4 && c.G != 8)) return hipErrorInvalidValue;
  int split_tokens = (prefix_len + n_splits - 1) / n_splits;
  split_tokens = (split_tokens + kKeyBlock - 1) / kKeyBlock * kKeyBlock;
  if (split_tokens / kPage + 1 > kMaxSplitPages) return hipErrorInvalidValue;
  constexpr int kRows = PrefixCfg<kOvWaves>::kRowsPerWG;
  const int R = c.B * c.G;
  const int n_pre = (R + kRows - 1) / kRows * c.Hkv * n_splits;
  const int n_suf = (c.B * c.Hkv + kOvWaves - 1) / kOvWaves;
  const int chunk = std::max(1, cus_per_xcd);
  const int gp = (n_pre + 7) / 8, gs = (n_suf + 7) / 8;
  const int blocks = 8 * chunk * ((gp + chunk - 1) / chunk + (gs + chunk - 1) / chunk);
#define QSA_OVERLAP_CASE(GG)                                                                             \
  case GG:                                                                                               \
    hipLaunchKernelGGL((cascade_overlap_kernel<GG>), dim3(blocks), dim3(64 * kOvWaves), 0, stream,       \
                       static_cast<const bf16s*>(q), static_cast<const bf16s*>(c.k_pool),                \
                       static_cast<const bf16s*>(c.v_pool), c.num_phys, c.B, c.Hkv, prefix_pages, prefix_len, \
                       split_tokens, n_splits, scale_log2, prefix.o, prefix.ml, n_pre,                   \
                       static_cast<bf16s*>(meta), stride, c.page_indptr, c.page_indices, c.seq_lens,     \
                       refresh_tail, k, suffix.o, suffix.ml, n_suf, chunk, group_scores, sel, sel_count,  \
                       c.err);                                                                           \
    break;
  switch (c.G) {
    QSA_OVERLAP_CASE(4)
    QSA_OVERLAP_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef QSA_OVERLAP_CASE
  return hipGetLastError();
}

}  // namespace qsa
