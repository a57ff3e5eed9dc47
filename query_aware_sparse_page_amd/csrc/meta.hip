// Step 1: per-page bounding-box metadata (TinyServe page, §2.1).
//
// meta[b][h][j][0][:] = element-wise min, meta[b][h][j][1][:] = element-wise
// max of the valid keys of logical page j of sequence b, KV head h (read
// through the page table). The metadata is stored in logical page order so
// that scoring streams each (sequence, KV head) row contiguously. The
// comparison is an unsigned compare of order-preserving keys (IEEE total
// order, -0 < +0), so the result is exact and independent of reduction order.
//
// One wave per (page, KV head) tile (tile_minmax), read with the non-temporal
// hint (ld16_stream).
//
// The centroid summary (build_centroid_kernel) is the alternative page
// summary of the Vortex digest's cache phase, laid out the same way with one
// 256-byte row per page.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

template <typename T>
__global__ void __launch_bounds__(256) build_meta_kernel(
    const T* __restrict__ k_pool, int num_phys, int Hkv, const int* __restrict__ page_indptr,
    const int* __restrict__ page_indices, const int* __restrict__ seq_lens, int tail_pages,
    T* __restrict__ meta, int stride, unsigned int* __restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int L = seq_lens[b];
  if (L <= 0) return;
  const int n = min((L + kPage - 1) / kPage, stride);
  const int first = tail_pages > 0 ? (n > tail_pages ? n - tail_pages : 0) : 0;
  const int tile = blockIdx.x * 4 + wave;  // (page, head) tile of this wave
  const int j = first + tile / Hkv;
  const int h = tile - (tile / Hkv) * Hkv;
  if (j >= n) return;
  const int p = page_indices[page_indptr[b] + j];
  if (p < 0 || p >= num_phys) {
    report_bad(err, kErrPhys);
    return;
  }
  const int valid = min(kPage, L - kPage * j);
  const int chunk = lane & 15;
  const char* src = reinterpret_cast<const char*>(k_pool) + ((size_t)p * Hkv + h) * kTileBytes;

  uint4 vmn, vmx;
  tile_minmax<T, true>(src, valid, lane, vmn, vmx);
  // lanes 0..15 write the min row, lanes 16..31 the max row of this
  // sequence's logical page j
  if (lane < 32) {
    char* dst = reinterpret_cast<char*>(meta) + (((size_t)b * Hkv + h) * stride + j) * 512;
    st16(dst + (lane >> 4) * 256 + chunk * 16, lane < 16 ? vmn : vmx);
  }
}

// Centroid summary (Vortex digest, cache phase: each block's mean key):
// cent[b][h][j][:] = mean of the valid keys of logical page j, rounded once to
// the key type (tile_mean). Same launch geometry as the min/max build; lanes
// 0..15 write the 256-byte row.
template <typename T>
__global__ void __launch_bounds__(256) build_centroid_kernel(
    const T* __restrict__ k_pool, int num_phys, int Hkv, const int* __restrict__ page_indptr,
    const int* __restrict__ page_indices, const int* __restrict__ seq_lens, int tail_pages,
    T* __restrict__ cent, int stride, unsigned int* __restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int L = seq_lens[b];
  if (L <= 0) return;
  const int n = min((L + kPage - 1) / kPage, stride);
  const int first = tail_pages > 0 ? (n > tail_pages ? n - tail_pages : 0) : 0;
  const int tile = blockIdx.x * 4 + wave;
  const int j = first + tile / Hkv;
  const int h = tile - (tile / Hkv) * Hkv;
  if (j >= n) return;
  const int p = page_indices[page_indptr[b] + j];
  if (p < 0 || p >= num_phys) {
    report_bad(err, kErrPhys);
    return;
  }
  const int valid = min(kPage, L - kPage * j);
  const char* src = reinterpret_cast<const char*>(k_pool) + ((size_t)p * Hkv + h) * kTileBytes;
  const uint4 mean = tile_mean<T, true>(src, valid, lane);
  if (lane < 16) {
    char* dst = reinterpret_cast<char*>(cent) + (((size_t)b * Hkv + h) * stride + j) * kRowBytes;
    st16(dst + lane * 16, mean);
  }
}

}  // namespace

hipError_t launch_build_centroids(const LaunchCommon& c, int max_pages, int tail_pages, void* cent,
                                  int stride, hipStream_t stream) {
  const int pages = tail_pages > 0 ? (tail_pages < max_pages ? tail_pages : max_pages) : max_pages;
  dim3 grid((pages * c.Hkv + 3) / 4, c.B);
  if (c.bf16) {
    hipLaunchKernelGGL(build_centroid_kernel<bf16s>, grid, dim3(256), 0, stream,
                       static_cast<const bf16s*>(c.k_pool), c.num_phys, c.Hkv, c.page_indptr,
                       c.page_indices, c.seq_lens, tail_pages, static_cast<bf16s*>(cent), stride, c.err);
  } else {
    hipLaunchKernelGGL(build_centroid_kernel<float>, grid, dim3(256), 0, stream,
                       static_cast<const float*>(c.k_pool), c.num_phys, c.Hkv, c.page_indptr,
                       c.page_indices, c.seq_lens, tail_pages, static_cast<float*>(cent), stride, c.err);
  }
  return hipGetLastError();
}

hipError_t launch_build_meta(const LaunchCommon& c, int max_pages, int tail_pages, void* meta,
                             int stride, hipStream_t stream) {
  const int pages = tail_pages > 0 ? (tail_pages < max_pages ? tail_pages : max_pages) : max_pages;
  dim3 grid((pages * c.Hkv + 3) / 4, c.B);
  if (c.bf16) {
    hipLaunchKernelGGL(build_meta_kernel<bf16s>, grid, dim3(256), 0, stream,
                       static_cast<const bf16s*>(c.k_pool), c.num_phys, c.Hkv, c.page_indptr,
                       c.page_indices, c.seq_lens, tail_pages, static_cast<bf16s*>(meta), stride, c.err);
  } else {
    hipLaunchKernelGGL(build_meta_kernel<float>, grid, dim3(256), 0, stream,
                       static_cast<const float*>(c.k_pool), c.num_phys, c.Hkv, c.page_indptr,
                       c.page_indices, c.seq_lens, tail_pages, static_cast<float*>(meta), stride, c.err);
  }
  return hipGetLastError();
}

}  // namespace qsa
