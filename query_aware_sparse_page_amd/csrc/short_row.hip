// Steps 2-4 of one decode step for rows of at most 64 pages, one wave per
// (sequence, KV head) row, with an optional log-sum-exp merge of
// shared-prefix partials: the kernel around short_row.h's workgroup body.
#include "short_row.h"

namespace qsa {
namespace {

using shortrow::kShortWaves;
using shortrow::ShortShared;

template <int G>
__global__ void __launch_bounds__(64 * kShortWaves) __attribute__((amdgpu_waves_per_eu(2)))
short_row_kernel(const bf16s* __restrict__ q, bf16s* __restrict__ meta, int stride,
                 const bf16s* __restrict__ k_pool, const bf16s* __restrict__ v_pool, int num_phys, int B,
                 int Hkv, const int* __restrict__ page_indptr, const int* __restrict__ page_indices,
                 const int* __restrict__ seq_lens, int refresh_tail, int k, float scale_log2,
                 const float* __restrict__ pre_o, const float* __restrict__ pre_ml, int n_pre,
                 float* __restrict__ out, float* __restrict__ lse, float* __restrict__ group_scores,
                 int* __restrict__ sel, int* __restrict__ sel_count, unsigned int* __restrict__ err) {
  __shared__ ShortShared<G> sh;
  shortrow::short_row_block<G>(sh, blockIdx.x, threadIdx.x, q, meta, stride, k_pool, v_pool, num_phys, B, Hkv,
                               page_indptr, page_indices, seq_lens, refresh_tail, k, scale_log2, pre_o, pre_ml,
                               n_pre, out, lse, group_scores, sel, sel_count, err, nullptr, nullptr);
}

}  // namespace

hipError_t launch_short_rows(const LaunchCommon& c, const void* q, void* meta, int stride, int refresh_tail,
                             int k, float scale_log2, Partials prefix, int n_prefix, float* out, float* lse,
                             float* group_scores, int* sel, int* sel_count, hipStream_t stream) {
  if (!c.bf16 || c.D != 128) return hipErrorInvalidValue;
  const int rows = c.B * c.Hkv;
  const dim3 grid((rows + kShortWaves - 1) / kShortWaves);
#define QSA_SHORT_CASE(GG)                                                                            \
  case GG:                                                                                            \
    hipLaunchKernelGGL((short_row_kernel<GG>), grid, dim3(64 * kShortWaves), 0, stream,               \
                       static_cast<const bf16s*>(q), static_cast<bf16s*>(meta), stride,               \
                       static_cast<const bf16s*>(c.k_pool), static_cast<const bf16s*>(c.v_pool),      \
                       c.num_phys, c.B, c.Hkv, c.page_indptr, c.page_indices, c.seq_lens, refresh_tail, \
                       k, scale_log2, prefix.o, prefix.ml, n_prefix, out, lse, group_scores, sel,     \
                       sel_count, c.err);                                                             \
    break;
  switch (c.G) {
    QSA_SHORT_CASE(4)
    QSA_SHORT_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef QSA_SHORT_CASE
  return hipGetLastError();
}

}  // namespace qsa
