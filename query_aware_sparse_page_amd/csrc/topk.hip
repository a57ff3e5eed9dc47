// Step 3: per-(sequence, KV head) top-K page selection (TinyServe page, §2.3:
// the K highest-scoring pages; the Vortex digest names radix top-K as the
// indexer's bottleneck).
//
// Scores map to order-preserving uint32 keys (-0 folded onto +0), held in
// registers. Rows of up to 1024 pages take one wave each (8-bit digits, no
// workgroup barriers); longer rows one workgroup of 1024 threads each (up to
// 16384 pages), each thread a contiguous run of pages. (The approximate
// select below runs as a 256-thread workgroup for rows of up to 1024 pages.)
// An MSB-first radix select finds the bin holding the K_eff-th largest key,
// and how many of its keys are still needed (krem): it starts below the bits
// that every key shares (from the row's min and max) and takes 8 bits per
// pass (wave kernel) or about log2(n) + 2 bits (block kernel: at most 13, an
// 8192-bin LDS histogram, so typical fp32 scores resolve in two passes); the
// block kernel also stops once the bin holds exactly the keys still needed. A compaction in page order then keeps every
// page above the bin and the first krem pages in it - ties go to the smaller
// page index and the output is in ascending page order; each kept page's
// position comes from one block-wide scan of (above, in-bin) counts.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) { return wave_min_u32(v); }
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) { return wave_max_u32(v); }

// Rows of up to 1024 pages: one wave per row (4 rows per workgroup), no
// workgroup barriers. Lane l owns pages l*kKeys .. l*kKeys + kKeys - 1; the
// radix select uses 8-bit digits with a per-wave LDS histogram.
template <int kKeys>
__global__ void __launch_bounds__(256) topk_wave_kernel(
    const float* __restrict__ group_scores, int stride, int Hkv, int rows,
    const int* __restrict__ seq_lens, const int* __restrict__ page_indptr,
    const int* __restrict__ page_indices, int k, int* __restrict__ sel,
    int* __restrict__ sel_count, int* __restrict__ sel_phys) {
  __shared__ uint32_t hist[4][256];
  __shared__ uint32_t pick[4][2];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row_i = blockIdx.x * 4 + wave;
  if (row_i >= rows) return;
  const size_t row = (size_t)row_i;
  const int b = row_i / Hkv;
  const float* sc = group_scores + row * stride;
  int* out = sel + row * k;
  int* outp = sel_phys ? sel_phys + row * k : nullptr;
  // scores first (every j < stride is in bounds), then the row length
  const int j0 = lane * kKeys;
  float raw[kKeys];
#pragma unroll
  for (int i = 0; i < kKeys; ++i) raw[i] = (j0 + i < stride) ? sc[j0 + i] : 0.0f;
  const int L = seq_lens[b];
  int n = L > 0 ? (L + kPage - 1) / kPage : 0;
  n = n < stride ? n : stride;
  n = n < 64 * kKeys ? n : 64 * kKeys;
  const int keff = k < n ? k : n;
  const int* table = page_indices + page_indptr[b];
  uint32_t* h = hist[wave];

  if (keff == n) {
    for (int i = lane; i < k; i += 64) {
      out[i] = i < n ? i : -1;
      if (outp) outp[i] = i < n ? table[i] : -1;
    }
    if (lane == 0) sel_count[row] = keff;
    return;
  }

  uint32_t keys[kKeys];
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < kKeys; ++i) {
    const int j = j0 + i;
    keys[i] = j < n ? score_key(raw[i]) : 0u;
    if (j < n) {
      kmin = min(kmin, keys[i]);
      kmax = max(kmax, keys[i]);
    }
  }
  kmin = wave_min_u(kmin);
  kmax = wave_max_u(kmax);

  uint32_t krem = (uint32_t)keff;
  uint32_t T = kmin;
  const uint32_t diff = kmin ^ kmax;
  if (diff != 0u) {
    int shift = 32 - __builtin_clz(diff);
    uint32_t prefix = (uint32_t)((uint64_t)kmin >> shift);
    while (shift > 0) {
      const int nb = shift < 8 ? shift : 8;
      const int lo = shift - nb;
      const uint32_t nbins = 1u << nb;
#pragma unroll
      for (int i = 0; i < 4; ++i) h[lane * 4 + i] = 0u;
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < kKeys; ++i) {
        if (j0 + i < n && (uint32_t)((uint64_t)keys[i] >> shift) == prefix)
          atomicAdd(&h[(keys[i] >> lo) & (nbins - 1u)], 1u);
      }
      wave_lds_sync();
      // lane l scans digits nbins-1 - (4l .. 4l+3), i.e. descending
      uint32_t cnt[4];
      uint32_t local = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = lane * 4 + i;
        cnt[i] = pos < (int)nbins ? h[nbins - 1 - pos] : 0u;
        local += cnt[i];
      }
      uint32_t above = wave_scan_incl(local) - local;
      if (above < krem && above + local >= krem) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (above < krem && above + cnt[i] >= krem) {
            pick[wave][0] = nbins - 1u - (uint32_t)(lane * 4 + i);
            pick[wave][1] = krem - above;
          }
          above += cnt[i];
        }
      }
      wave_lds_sync();
      prefix = (prefix << nb) | pick[wave][0];
      krem = pick[wave][1];
      shift = lo;
      wave_lds_sync();
    }
    T = prefix;
  }

  uint32_t gt_n = 0, eq_n = 0;
#pragma unroll
  for (int i = 0; i < kKeys; ++i) {
    if (j0 + i < n) {
      gt_n += keys[i] > T ? 1u : 0u;
      eq_n += keys[i] == T ? 1u : 0u;
    }
  }
  const uint32_t packed = gt_n | (eq_n << 16);
  const uint32_t excl = wave_scan_incl(packed) - packed;
  uint32_t gt_before = excl & 0xFFFFu;
  uint32_t eq_before = excl >> 16;
#pragma unroll
  for (int i = 0; i < kKeys; ++i) {
    const int j = j0 + i;
    if (j >= n) break;
    const bool gt = keys[i] > T;
    const bool eq = keys[i] == T;
    if (gt || (eq && eq_before < krem)) {
      const uint32_t pos = gt_before + (eq_before < krem ? eq_before : krem);
      if (pos < (uint32_t)keff) {
        out[pos] = j;
        if (outp) outp[pos] = table[j];
      }
    }
    gt_before += gt ? 1u : 0u;
    eq_before += eq ? 1u : 0u;
  }
  for (int i = keff + lane; i < k; i += 64) {
    out[i] = -1;
    if (outp) outp[i] = -1;
  }
  if (lane == 0) sel_count[row] = keff;
}

// As block_excl_scan, without the closing barrier: wsum must not be written
// again until every thread has passed another workgroup barrier.
template <int kWaves>
__device__ __forceinline__ uint32_t block_excl_scan_once(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t incl = wave_scan_incl(v);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t t = wsum[w];
    before += (w < wave) ? t : 0u;
    tot += t;
  }
  *total = tot;
  return before + incl - v;
}

// Block kernel (one workgroup per row). kApprox = false is the exact select;
// kApprox = true is the approximate select of the Vortex digest
// (optimisations: radix top-K that terminates early once it holds enough
// confident pages and fills the rest at random from the threshold bin):
//   * digits are digit_bits wide (the exact select sizes them from n);
//   * after each pass the pages in bins above the kept bin are confident;
//     the passes stop once they number at least min_confident;
//   * the r pages still needed come from the c pages of the kept bin, in
//     page order (rank i), by systematic sampling with a random start
//     st = floor(row_rand * c / 2^32): rank i is taken when
//     (i*r + st) mod c >= c - r, so floor((i*r + st) / c) bin pages of lower
//     rank are taken before it, and every bin page has probability r/c.
// Both stop as soon as the kept bin is exactly the pages still needed (the
// result is then the same as running to the last bit).
template <int kThreads, int kKeys, bool kApprox>
__global__ void __launch_bounds__(kThreads) topk_kernel(
    const float* __restrict__ group_scores, int stride, int Hkv, const int* __restrict__ seq_lens,
    const int* __restrict__ page_indptr, const int* __restrict__ page_indices, int k,
    int digit_bits, int min_confident, const uint32_t* __restrict__ row_rand,
    int* __restrict__ sel, int* __restrict__ sel_count, int* __restrict__ sel_phys,
    int* __restrict__ passes_out) {
  constexpr int kWaves = kThreads / 64;
  constexpr int kRadixBits = 13;  // widest digit (the approximate select's digit_bits <= 13)
  constexpr int kExactBits = 10;  // widest digit of the exact select
  constexpr int kBins = 1 << kRadixBits;
  constexpr int kBinsPerThread = kBins / kThreads;
  // Histograms, scan sums and the picked digit alternate between two
  // buffers by pass, so a pass needs two workgroup barriers: the next
  // pass's histogram is cleared while this one is filled, and nothing is
  // rewritten before every thread has passed the next barrier.
  __shared__ uint32_t hist[2][kBins];
  __shared__ uint32_t wsum[2][kWaves];
  __shared__ uint32_t wmin[kWaves], wmax[kWaves];
  __shared__ uint32_t s_pick[2][3];  // digit, pages still needed, pages in the digit's bin

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const size_t row = (size_t)b * Hkv + h;
  const float* sc = group_scores + row * stride;
  int* out = sel + row * k;
  int* outp = sel_phys ? sel_phys + row * k : nullptr;
  const int j0 = tid * kKeys;
  float raw[kKeys];
#pragma unroll
  for (int i = 0; i < kKeys; ++i) raw[i] = (j0 + i < stride) ? sc[j0 + i] : 0.0f;
  const int L = seq_lens[b];
  int n = L > 0 ? (L + kPage - 1) / kPage : 0;
  n = n < stride ? n : stride;
  n = n < kThreads * kKeys ? n : kThreads * kKeys;
  const int keff = k < n ? k : n;
  const int* table = page_indices + page_indptr[b];

  if (keff == n) {
    // Budget covers the sequence: every page, in order.
    for (int i = tid; i < k; i += kThreads) {
      out[i] = i < n ? i : -1;
      if (outp) outp[i] = i < n ? table[i] : -1;
    }
    if (tid == 0) {
      sel_count[row] = keff;
      if (passes_out) passes_out[row] = 0;
    }
    return;
  }

  // Keys stay in registers; thread t owns the contiguous pages t*kKeys + i.
  uint32_t keys[kKeys];
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < kKeys; ++i) {
    const int j = j0 + i;
    keys[i] = j < n ? score_key(raw[i]) : 0u;
    if (j < n) {
      kmin = min(kmin, keys[i]);
      kmax = max(kmax, keys[i]);
    }
  }
  // exact: digit width about log2(n) + 2 bits, so the histogram stays small
  // for short rows, at most kExactBits: a pass over 1024 bins (one per
  // thread) is cheaper than one over 8192, which more than pays for a third
  // pass on rows of 8192 pages (13.5 against 14.4 us per launch for 10 and
  // 13 bits)
  const int width = kApprox ? digit_bits : min(kExactBits, max(4, 34 - __builtin_clz((uint32_t)n)));
  // the first pass's histogram (at most 2^width bins) is cleared before the
  // min / max barrier
  for (int i = tid; i < (1 << width); i += kThreads) hist[0][i] = 0u;
  kmin = wave_min_u(kmin);
  kmax = wave_max_u(kmax);
  if (lane == 0) {
    wmin[wave] = kmin;
    wmax[wave] = kmax;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    kmin = min(kmin, wmin[w]);
    kmax = max(kmax, wmax[w]);
  }

  // Radix select, MSB first, starting below the bits every key shares. After
  // the loop the kept bin is {keys with key >> shift == prefix}; krem of its
  // pages are still needed.
  uint32_t krem = (uint32_t)keff;
  uint32_t prefix = kmin;
  int shift = 0;
  int passes = 0;
  const uint32_t diff = kmin ^ kmax;
  int pb = 0;  // this pass's buffers
  if (diff != 0u) {
    shift = 32 - __builtin_clz(diff);               // bits below `shift` still open
    prefix = (uint32_t)((uint64_t)kmin >> shift);
    while (shift > 0) {
      const int nb = shift < width ? shift : width;
      const int lo = shift - nb;
      const uint32_t nbins = 1u << nb;
      uint32_t* hcur = hist[pb];
#pragma unroll
      for (int i = 0; i < kKeys; ++i) {
        if (j0 + i < n && (uint32_t)((uint64_t)keys[i] >> shift) == prefix)
          atomicAdd(&hcur[(keys[i] >> lo) & (nbins - 1u)], 1u);
      }
      if (lo > 0) {  // the next pass's histogram
        const int nb_next = lo < width ? lo : width;
        for (int i = tid; i < (1 << nb_next); i += kThreads) hist[pb ^ 1][i] = 0u;
      }
      __syncthreads();
      // thread t scans digits nbins-1 - (t*B .. t*B+B-1), i.e. descending
      uint32_t cnt[kBinsPerThread];
      uint32_t local = 0;
#pragma unroll
      for (int i = 0; i < kBinsPerThread; ++i) {
        const int pos = tid * kBinsPerThread + i;
        cnt[i] = pos < (int)nbins ? hcur[nbins - 1 - pos] : 0u;
        local += cnt[i];
      }
      uint32_t total;
      uint32_t above = block_excl_scan_once<kWaves>(local, wsum[pb], &total);
      if (above < krem && above + local >= krem) {
#pragma unroll
        for (int i = 0; i < kBinsPerThread; ++i) {
          if (above < krem && above + cnt[i] >= krem) {
            s_pick[pb][0] = nbins - 1u - (uint32_t)(tid * kBinsPerThread + i);
            s_pick[pb][1] = krem - above;
            s_pick[pb][2] = cnt[i];
          }
          above += cnt[i];
        }
      }
      __syncthreads();
      prefix = (prefix << nb) | s_pick[pb][0];
      krem = s_pick[pb][1];
      const uint32_t bin = s_pick[pb][2];
      shift = lo;
      ++passes;
      pb ^= 1;
      if (bin == krem) break;                          // the whole bin is taken
      if (kApprox && (uint32_t)keff - krem >= (uint32_t)min_confident) break;
    }
  }

  // Compaction in page order: one block scan of (above the bin, in the bin)
  // counts gives each kept page its output position.
  uint32_t gt_n = 0, eq_n = 0;
#pragma unroll
  for (int i = 0; i < kKeys; ++i) {
    if (j0 + i < n) {
      const uint32_t hi = (uint32_t)((uint64_t)keys[i] >> shift);
      gt_n += hi > prefix ? 1u : 0u;
      eq_n += hi == prefix ? 1u : 0u;
    }
  }
  uint32_t total;
  const uint32_t excl = block_excl_scan_once<kWaves>(gt_n | (eq_n << 16), wsum[pb], &total);
  uint32_t gt_before = excl & 0xFFFFu;
  uint32_t eq_before = excl >> 16;
  const uint32_t c = total >> 16;                     // pages in the kept bin
  uint32_t st = 0;
  if (kApprox) st = (uint32_t)(((uint64_t)row_rand[row] * c) >> 32);
  // bin pages of rank < i that are taken
  auto taken_before = [&](uint32_t i) -> uint32_t {
    if (kApprox) return (i * krem + st) / c;
    return i < krem ? i : krem;
  };
#pragma unroll
  for (int i = 0; i < kKeys; ++i) {
    const int j = j0 + i;
    if (j >= n) break;
    const uint32_t hi = (uint32_t)((uint64_t)keys[i] >> shift);
    const bool gt = hi > prefix;
    const bool eq = hi == prefix;
    bool take = gt;
    if (eq) take = kApprox ? (eq_before * krem + st) % c >= c - krem : eq_before < krem;
    if (take) {
      const uint32_t pos = gt_before + taken_before(eq_before);
      if (pos < (uint32_t)keff) {
        out[pos] = j;
        if (outp) outp[pos] = table[j];
      }
    }
    gt_before += gt ? 1u : 0u;
    eq_before += eq ? 1u : 0u;
  }
  for (int i = keff + tid; i < k; i += kThreads) {
    out[i] = -1;
    if (outp) outp[i] = -1;
  }
  if (tid == 0) {
    sel_count[row] = keff;
    if (passes_out) passes_out[row] = passes;
  }
}

}  // namespace

hipError_t launch_topk(const LaunchCommon& c, const float* group_scores, int stride, int k,
                       int* sel, int* sel_count, int* sel_phys, hipStream_t stream) {
  dim3 grid(c.Hkv, c.B);
  const int rows = c.B * c.Hkv;
  if (stride <= 64 * 4) {
    hipLaunchKernelGGL((topk_wave_kernel<4>), dim3((rows + 3) / 4), dim3(256), 0, stream,
                       group_scores, stride, c.Hkv, rows, c.seq_lens, c.page_indptr, c.page_indices,
                       k, sel, sel_count, sel_phys);
  } else if (stride <= 64 * 16) {
    hipLaunchKernelGGL((topk_wave_kernel<16>), dim3((rows + 3) / 4), dim3(256), 0, stream,
                       group_scores, stride, c.Hkv, rows, c.seq_lens, c.page_indptr, c.page_indices,
                       k, sel, sel_count, sel_phys);
  } else if (stride <= 1024 * 8) {
    hipLaunchKernelGGL((topk_kernel<1024, 8, false>), grid, dim3(1024), 0, stream, group_scores,
                       stride, c.Hkv, c.seq_lens, c.page_indptr, c.page_indices, k, 0, 0, nullptr,
                       sel, sel_count, sel_phys, nullptr);
  } else if (stride <= kTopkMaxPages) {
    hipLaunchKernelGGL((topk_kernel<1024, 16, false>), grid, dim3(1024), 0, stream, group_scores,
                       stride, c.Hkv, c.seq_lens, c.page_indptr, c.page_indices, k, 0, 0, nullptr,
                       sel, sel_count, sel_phys, nullptr);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_topk_approx(const LaunchCommon& c, const float* group_scores, int stride, int k,
                              int digit_bits, int min_confident, const uint32_t* row_rand,
                              int* sel, int* sel_count, int* sel_phys, int* passes,
                              hipStream_t stream) {
  dim3 grid(c.Hkv, c.B);
  if (stride <= 256 * 4) {
    hipLaunchKernelGGL((topk_kernel<256, 4, true>), grid, dim3(256), 0, stream, group_scores,
                       stride, c.Hkv, c.seq_lens, c.page_indptr, c.page_indices, k, digit_bits,
                       min_confident, row_rand, sel, sel_count, sel_phys, passes);
  } else if (stride <= 1024 * 8) {
    hipLaunchKernelGGL((topk_kernel<1024, 8, true>), grid, dim3(1024), 0, stream, group_scores,
                       stride, c.Hkv, c.seq_lens, c.page_indptr, c.page_indices, k, digit_bits,
                       min_confident, row_rand, sel, sel_count, sel_phys, passes);
  } else if (stride <= kTopkMaxPages) {
    hipLaunchKernelGGL((topk_kernel<1024, 16, true>), grid, dim3(1024), 0, stream, group_scores,
                       stride, c.Hkv, c.seq_lens, c.page_indptr, c.page_indices, k, digit_bits,
                       min_confident, row_rand, sel, sel_count, sel_phys, passes);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qsa
