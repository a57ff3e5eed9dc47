// Step 3: per-(sequence, KV head) top-K page selection (TinyServe page, §2.3:
// the K highest-scoring pages; the Vortex digest names radix top-K as the
// indexer's bottleneck).
//
// One workgroup per row. Scores map to order-preserving uint32 keys (-0 folded
// onto +0). An MSB-first radix select (4 passes of 8 bits, histograms in LDS)
// finds the K_eff-th largest key T exactly, and how many keys equal to T are
// still needed (krem). A compaction pass in page order then keeps every page
// with key > T and the first krem pages with key == T - so ties go to the
// smaller page index and the output comes out in ascending page order, with
// the position of a kept page given by two block-wide prefix counts. Keys stay
// in registers for the whole select (up to 16 per thread, so rows of up to
// 16384 pages); each wave counts into its own LDS histogram.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

// Inclusive prefix sum over a wave (ds_bpermute steps of 1..32 lanes).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = __lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t t = (uint32_t)__builtin_amdgcn_ds_bpermute((lane - d) << 2, (int)v);
    if (lane >= d) v += t;
  }
  return v;
}

template <int kThreads, int kKeys>
__global__ void __launch_bounds__(kThreads) topk_kernel(
    const float* __restrict__ group_scores, int stride, int Hkv, const int* __restrict__ seq_lens,
    const int* __restrict__ page_indptr, const int* __restrict__ page_indices, int k,
    int* __restrict__ sel, int* __restrict__ sel_count, int* __restrict__ sel_phys) {
  constexpr int kWaves = kThreads / 64;
  constexpr int kBinsPad = 257;  // per-wave histogram; the pad spreads the waves over LDS banks
  __shared__ uint32_t hist[kWaves * kBinsPad];
  __shared__ uint32_t wtot[kWaves];
  __shared__ uint32_t s_digit, s_krem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const size_t row = (size_t)b * Hkv + h;
  const float* sc = group_scores + row * stride;
  int* out = sel + row * k;
  int* outp = sel_phys ? sel_phys + row * k : nullptr;
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
    if (tid == 0) sel_count[row] = keff;
    return;
  }

  // Keys stay in registers: slot i holds page j = tid + i * kThreads.
  uint32_t keys[kKeys];
#pragma unroll
  for (int i = 0; i < kKeys; ++i) {
    const int j = tid + i * kThreads;
    keys[i] = j < n ? score_key(sc[j]) : 0u;
  }

  uint32_t prefix = 0, mask = 0, krem = (uint32_t)keff;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kWaves * kBinsPad; i += kThreads) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kKeys; ++i) {
      const int j = tid + i * kThreads;
      if (j < n && (keys[i] & mask) == prefix)
        atomicAdd(&hist[wave * kBinsPad + ((keys[i] >> shift) & 0xFFu)], 1u);
    }
    __syncthreads();
    // Thread t < 256 owns digit 255 - t, so an inclusive scan over t counts
    // the keys whose digit is >= that digit.
    uint32_t v = 0, incl = 0;
    if (tid < 256) {
      const int d = 255 - tid;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += hist[w * kBinsPad + d];
      incl = wave_incl_scan(v);
      if (lane == 63) wtot[wave] = incl;
    }
    __syncthreads();
    if (tid < 256) {
      for (int w = 0; w < wave; ++w) incl += wtot[w];
      const uint32_t above = incl - v;  // keys with a larger digit
      if (above < krem && incl >= krem) {
        s_digit = 255u - (uint32_t)tid;
        s_krem = krem - above;
      }
    }
    __syncthreads();
    prefix |= s_digit << shift;
    mask |= 0xFFu << shift;
    krem = s_krem;
    __syncthreads();
  }
  const uint32_t T = prefix;

  // Compaction in page order: round i covers pages i*kThreads .. +kThreads.
  uint32_t gt_base = 0, eq_base = 0;
#pragma unroll
  for (int i = 0; i < kKeys; ++i) {
    if (i * kThreads >= n) break;
    const int j = tid + i * kThreads;
    const uint32_t key = keys[i];
    const uint32_t gt = (j < n && key > T) ? 1u : 0u;
    const uint32_t eq = (j < n && key == T) ? 1u : 0u;
    const uint32_t packed = gt | (eq << 16);
    uint32_t incl = wave_incl_scan(packed);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    uint32_t before = 0, total = 0;
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t t = wtot[w];
      if (w < wave) before += t;
      total += t;
    }
    const uint32_t excl = before + incl - packed;
    const uint32_t gt_before = gt_base + (excl & 0xFFFFu);
    const uint32_t eq_before = eq_base + (excl >> 16);
    if (gt || (eq && eq_before < krem)) {
      const uint32_t pos = gt_before + (eq_before < krem ? eq_before : krem);
      if (pos < (uint32_t)keff) {
        out[pos] = j;
        if (outp) outp[pos] = table[j];
      }
    }
    gt_base += total & 0xFFFFu;
    eq_base += total >> 16;
    __syncthreads();
  }
  for (int i = keff + tid; i < k; i += kThreads) {
    out[i] = -1;
    if (outp) outp[i] = -1;
  }
  if (tid == 0) sel_count[row] = keff;
}

}  // namespace

hipError_t launch_topk(const LaunchCommon& c, const float* group_scores, int stride, int k,
                       int* sel, int* sel_count, int* sel_phys, hipStream_t stream) {
  dim3 grid(c.Hkv, c.B);
  if (stride <= 256 * 4) {
    hipLaunchKernelGGL((topk_kernel<256, 4>), grid, dim3(256), 0, stream, group_scores, stride,
                       c.Hkv, c.seq_lens, c.page_indptr, c.page_indices, k, sel, sel_count, sel_phys);
  } else if (stride <= 1024 * 8) {
    hipLaunchKernelGGL((topk_kernel<1024, 8>), grid, dim3(1024), 0, stream, group_scores, stride,
                       c.Hkv, c.seq_lens, c.page_indptr, c.page_indices, k, sel, sel_count, sel_phys);
  } else if (stride <= kTopkMaxPages) {
    hipLaunchKernelGGL((topk_kernel<1024, 16>), grid, dim3(1024), 0, stream, group_scores, stride,
                       c.Hkv, c.seq_lens, c.page_indptr, c.page_indices, k, sel, sel_count, sel_phys);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qsa
