// Step 5 (prefix half): the shared prefix of a cascade (Quail page, join
// attention: every suffix query attends the shared anchor once; the partial
// result is merged with the suffix's by log-sum-exp rescaling).
//
// With B sequences sharing the prefix, the queries of one KV head form a
// dense [R = B*g, D] block and the prefix a [D, prefix_len] block: a real
// contraction, so it runs on the matrix cores (v_mfma_f32_16x16x32_bf16,
// fp32 accumulate). Flash-attention style: a workgroup owns 256 query rows
// (8 waves, two 16-column tiles each, so every K and V read from LDS serves
// 32 queries) and one split of the prefix keys; it walks the split in blocks
// of 32 keys (two pages), keeping an online softmax per query.
//
// Orientation: the wave computes S^T = K . Q^T (rows = keys, cols = queries),
// so the probabilities come out of the MFMA already in the layout of the B
// operand of O^T = V^T . P^T and never leave registers. K and V blocks are
// staged row-major in LDS (16-byte stores into padded rows), double-buffered,
// with the global loads of the next kDepth blocks in flight in registers
// while a block is computed; the A operand V^T is read with
// ds_read_b64_tr_b16, which transposes 4 keys x 16 dims on the way (a 16-lane
// group's lane s reads key row key0 + s/4, dims d0 + 4 (s%4) .. +3, and lane
// s receives V[key0 .. key0+3][d0 + s]).
//
// MFMA operand layout (v_mfma_f32_16x16x32_bf16, lane l, g = l/16):
//   A[i][k]: i = l%16, k = 8g .. 8g+7     B[k][j]: j = l%16, k = 8g .. 8g+7
//   C[i][j]: j = l%16, i = 4g .. 4g+3
// S^T (over the head dim) leaves lane l the logits of keys 4g .. 4g+3 of each
// 16-key tile. O^T += V^T . P^T takes the block's 32 keys in one product with
// its k-slots 8g .. 8g+7 holding keys 4g .. 4g+3 of tile 0 and then of tile 1
// (any order works as long as A and B agree): the B operand is the lane's own
// eight weights, and the A operand two transposing reads, one per tile. The
// weights enter as bf16 high and low parts, one product each, so the output
// carries no bf16 rounding of them.
#include "cascade_prefix.h"

namespace qsa {
namespace {

using cascade::PrefixCfg;
constexpr int kPrefixWaves = 8;

__global__ void __launch_bounds__(64 * kPrefixWaves) __attribute__((amdgpu_waves_per_eu(1)))
cascade_prefix_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, int num_phys, int B, int Hkv, int G,
    const int* __restrict__ prefix_pages, int prefix_len, int split_tokens, int n_splits,
    float scale_log2, float* __restrict__ pre_o, float* __restrict__ pre_ml,
    unsigned int* __restrict__ err) {
  __shared__ cascade::CascadeShared sh;
  cascade::prefix_block<kPrefixWaves>(sh, blockIdx.x, threadIdx.x, q, k_pool, v_pool, num_phys, B, Hkv, G,
                                      prefix_pages, prefix_len, split_tokens, n_splits, scale_log2, pre_o, pre_ml,
                                      err);
}

}  // namespace

hipError_t launch_cascade_prefix(const LaunchCommon& c, const void* q, const int* prefix_pages,
                                 int prefix_len, int n_splits, float scale_log2, Partials prefix,
                                 hipStream_t stream) {
  using namespace cascade;
  if (!c.bf16 || c.D != kCD) return hipErrorInvalidValue;
  const int R = c.B * c.G;
  int split_tokens = (prefix_len + n_splits - 1) / n_splits;
  split_tokens = (split_tokens + kKeyBlock - 1) / kKeyBlock * kKeyBlock;
  if (split_tokens / kPage + 1 > kMaxSplitPages) return hipErrorInvalidValue;
  constexpr int kRows = PrefixCfg<kPrefixWaves>::kRowsPerWG;
  const int row_tiles = (R + kRows - 1) / kRows;
  hipLaunchKernelGGL(cascade_prefix_kernel, dim3(row_tiles * c.Hkv * n_splits), dim3(64 * kPrefixWaves), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(c.k_pool),
                     static_cast<const uint16_t*>(c.v_pool), c.num_phys, c.B, c.Hkv, c.G,
                     prefix_pages, prefix_len, split_tokens, n_splits, scale_log2, prefix.o,
                     prefix.ml, c.err);
  return hipGetLastError();
}

}  // namespace qsa
