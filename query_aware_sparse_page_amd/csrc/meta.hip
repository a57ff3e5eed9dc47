// Step 1: per-page bounding-box metadata (TinyServe page, §2.1).
//
// meta[b][h][j][0][:] = element-wise min, meta[b][h][j][1][:] = element-wise
// max of the valid keys of logical page j of sequence b, KV head h (read
// through the page table). The metadata is stored in logical page order so
// that scoring streams each (sequence, KV head) row contiguously. The
// comparison is an unsigned compare of order-preserving keys (IEEE total
// order, -0 < +0), so the result is exact and independent of reduction order.
//
// One wave per (page, KV head) tile. A tile is 16 rows x 256 B; each load
// instruction reads 1 KiB contiguous (lane l: bytes r*1024 + l*16, i.e. row
// 4r + l/16, chunk l%16), so a lane holds chunk l%16 of rows {l/16, 4 + l/16,
// 8 + l/16, 12 + l/16}. After an in-lane reduction over its 4 rows the lanes
// l, l^16, l^32, l^48 combine.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

template <typename T>
struct MetaOps;

template <>
struct MetaOps<bf16s> {
  // Keys of 8 bf16 values (4 dwords), min/max identities for masked rows.
  static __device__ __forceinline__ uint32_t key(uint32_t x) { return bf2_to_key(x); }
  static __device__ __forceinline__ uint32_t unkey(uint32_t k) { return key_to_bf2(k); }
  static __device__ __forceinline__ uint32_t vmin(uint32_t a, uint32_t b) { return umin2x16(a, b); }
  static __device__ __forceinline__ uint32_t vmax(uint32_t a, uint32_t b) { return umax2x16(a, b); }
};
template <>
struct MetaOps<float> {
  static __device__ __forceinline__ uint32_t key(uint32_t x) { return f32_to_key(x); }
  static __device__ __forceinline__ uint32_t unkey(uint32_t k) { return key_to_f32(k); }
  static __device__ __forceinline__ uint32_t vmin(uint32_t a, uint32_t b) { return a < b ? a : b; }
  static __device__ __forceinline__ uint32_t vmax(uint32_t a, uint32_t b) { return a > b ? a : b; }
};

template <typename T>
__global__ void __launch_bounds__(256) build_meta_kernel(
    const T* __restrict__ k_pool, int num_phys, int Hkv, const int* __restrict__ page_indptr,
    const int* __restrict__ page_indices, const int* __restrict__ seq_lens, int tail_pages,
    T* __restrict__ meta, int stride) {
  using Ops = MetaOps<T>;
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
  if (p < 0 || p >= num_phys) return;
  const int valid = min(kPage, L - kPage * j);
  const int row0 = lane >> 4;
  const int chunk = lane & 15;
  const char* src = reinterpret_cast<const char*>(k_pool) + ((size_t)p * Hkv + h) * kTileBytes;

  uint4 rows[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) rows[r] = ld16(src + r * 1024 + lane * 16);
  uint32_t mn[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  uint32_t mx[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (4 * r + row0 < valid) {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(&rows[r]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kk = Ops::key(w[e]);
        mn[e] = Ops::vmin(mn[e], kk);
        mx[e] = Ops::vmax(mx[e], kk);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    mn[e] = Ops::vmin(mn[e], xshfl_u(mn[e], 16));
    mx[e] = Ops::vmax(mx[e], xshfl_u(mx[e], 16));
    mn[e] = Ops::vmin(mn[e], xshfl_u(mn[e], 32));
    mx[e] = Ops::vmax(mx[e], xshfl_u(mx[e], 32));
  }
  // lanes 0..15 write the min row, lanes 16..31 the max row of this
  // sequence's logical page j
  if (lane < 32) {
    const uint32_t* srcv = lane < 16 ? mn : mx;
    uint4 out;
    out.x = Ops::unkey(srcv[0]);
    out.y = Ops::unkey(srcv[1]);
    out.z = Ops::unkey(srcv[2]);
    out.w = Ops::unkey(srcv[3]);
    char* dst = reinterpret_cast<char*>(meta) + (((size_t)b * Hkv + h) * stride + j) * 512;
    st16(dst + (lane >> 4) * 256 + chunk * 16, out);
  }
}

}  // namespace

hipError_t launch_build_meta(const LaunchCommon& c, int max_pages, int tail_pages, void* meta,
                             int stride, hipStream_t stream) {
  const int pages = tail_pages > 0 ? (tail_pages < max_pages ? tail_pages : max_pages) : max_pages;
  dim3 grid((pages * c.Hkv + 3) / 4, c.B);
  if (c.bf16) {
    hipLaunchKernelGGL(build_meta_kernel<bf16s>, grid, dim3(256), 0, stream,
                       static_cast<const bf16s*>(c.k_pool), c.num_phys, c.Hkv, c.page_indptr,
                       c.page_indices, c.seq_lens, tail_pages, static_cast<bf16s*>(meta), stride);
  } else {
    hipLaunchKernelGGL(build_meta_kernel<float>, grid, dim3(256), 0, stream,
                       static_cast<const float*>(c.k_pool), c.num_phys, c.Hkv, c.page_indptr,
                       c.page_indices, c.seq_lens, tail_pages, static_cast<float*>(meta), stride);
  }
  return hipGetLastError();
}

}  // namespace qsa
