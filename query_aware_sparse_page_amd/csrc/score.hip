// Step 2: upper-bound page score (TinyServe page, §2.2) and the group max.
//
// score_j = sum_i q_i * (q_i > 0 ? M_j[i] : m_j[i]) is evaluated as
// q_neg . m_j + q_pos . M_j with q split by sign (q_neg keeps the negative
// elements, q_pos the others), which turns it into one dot product of length
// 2D between the split query and the page's 512-byte [m | M] metadata row.
// bf16 products are exact in fp32; they accumulate with v_dot2_f32_bf16.
//
// With refresh_tail set, the wave that holds a row's last page first rebuilds
// that page's min/max from the keys (the per-step update after a token is
// appended) and writes it back, so a decode step needs no separate metadata
// launch.
//
// Layout: the metadata is in logical page order, so a (sequence, KV head) row
// is one contiguous stream of 512-byte [m | M] records. 16 lanes (one DPP
// row) per page; lane c of the row holds chunk c of m and chunk c of M (16
// bytes each). A wave covers 4 consecutive pages per step (2 KiB contiguous),
// a workgroup (4 waves) 64 pages. Lane partials are summed
// over the row with DPP; the group max over the g query heads is in-lane.
//
// kCentroid = true scores the centroid summary instead (Vortex digest: a
// block's score is the query's dot product with its mean key): 256-byte
// records [c], q unsplit, score = q . c_j, the same group max; the tail-page
// refresh rebuilds the centroid (tile_mean).
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kScorePagesPerBlock = 64;

template <typename T, int G, bool kCentroid>
__global__ void __launch_bounds__(256) score_kernel(
    const T* __restrict__ q, T* __restrict__ meta, int Hkv, const int* __restrict__ seq_lens,
    const int* __restrict__ page_indptr, const int* __restrict__ page_indices,
    const T* __restrict__ k_pool, int num_phys, int refresh_tail,
    float* __restrict__ group_scores, float* __restrict__ head_scores, int stride,
    unsigned int* __restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int c = lane & 15;      // chunk within a metadata row
  const int slot = lane >> 4;   // which of the wave's 4 pages
  const int base_j = blockIdx.x * kScorePagesPerBlock;
  constexpr int kRec = kCentroid ? kRowBytes : 2 * kRowBytes;  // bytes per page record
  char* mrow_base = reinterpret_cast<char*>(meta) + ((size_t)b * Hkv + h) * stride * kRec;

  // Metadata loads first (any j < stride is in bounds; each record is read
  // once, with the non-temporal hint), then the row length.
  constexpr int kSteps = kScorePagesPerBlock / 16;
  uint4 mrow[kSteps], Mrow[kSteps];
  int jj[kSteps];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    jj[s] = base_j + s * 16 + wave * 4 + slot;
    if (jj[s] < stride) {
      const char* rec = mrow_base + (size_t)jj[s] * kRec;
      mrow[s] = ld16_stream(rec + c * 16);
      if (!kCentroid) Mrow[s] = ld16_stream(rec + 256 + c * 16);
    }
  }
  // Query chunks of the group's heads (split by sign for the bound).
  uint4 qn[G], qp[G];
  const int Hq = Hkv * G;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const char* qrow = reinterpret_cast<const char*>(q) + ((size_t)b * Hq + h * G + hh) * kRowBytes;
    uint4 qc = ld16(qrow + c * 16);
    if (kCentroid)
      qn[hh] = qc;
    else
      chunk_sign_split(qc, qn[hh], qp[hh], T{});
  }
  const int L = seq_lens[b];
  const int n = L > 0 ? min((L + kPage - 1) / kPage, stride) : 0;

  // Optional refresh of the tail page's record (the page a decode step
  // appends to), by the wave whose slots hold it: min/max (or mean) of its
  // valid keys, written back and used for this score.
  if (refresh_tail && n > 0) {
    const int jt = n - 1;
    const int off = jt - base_j;
    if (off >= 0 && off < kScorePagesPerBlock && ((off & 15) >> 2) == wave) {
      const int p = page_indices[page_indptr[b] + jt];
      if (p < 0 || p >= num_phys) report_bad(err, kErrPhys);  // the stored record is scored
      if (p >= 0 && p < num_phys) {
        const int valid = min(kPage, L - kPage * jt);
        const char* src = reinterpret_cast<const char*>(k_pool) + ((size_t)p * Hkv + h) * kTileBytes;
        uint4 vmn, vmx;
        if (kCentroid) {
          vmn = tile_mean<T>(src, valid, lane);
          if (lane < 16) st16(mrow_base + (size_t)jt * kRec + c * 16, vmn);
        } else {
          tile_minmax<T>(src, valid, lane, vmn, vmx);
          if (lane < 32) st16(mrow_base + (size_t)jt * kRec + (lane >> 4) * 256 + c * 16, lane < 16 ? vmn : vmx);
        }
        const int st = off >> 4;
        if (slot == (off & 3)) {
#pragma unroll
          for (int s = 0; s < kSteps; ++s)
            if (s == st) {
              mrow[s] = vmn;
              if (!kCentroid) Mrow[s] = vmx;
            }
        }
      }
    }
  }

#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int j = jj[s];
    if (j >= stride) continue;
    const bool ok = j < n;
    float hs[G];
    float gmax = -__builtin_inff();
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float acc = 0.0f;
      if (ok) {
        acc = chunk_dot(qn[hh], mrow[s], acc, T{});
        if (!kCentroid) acc = chunk_dot(qp[hh], Mrow[s], acc, T{});
      }
      acc = sum16(acc);
      hs[hh] = ok ? acc : -__builtin_inff();
      gmax = fmaxf(gmax, hs[hh]);
    }
    if (c == 0) group_scores[((size_t)b * Hkv + h) * stride + j] = gmax;
    if (head_scores != nullptr && c < G) {
      float v = hs[0];
#pragma unroll
      for (int hh = 1; hh < G; ++hh) v = (c == hh) ? hs[hh] : v;
      head_scores[((size_t)b * Hq + h * G + c) * stride + j] = v;
    }
  }
}

template <typename T, bool kCentroid>
hipError_t launch_score_t(const LaunchCommon& c, const void* q, void* meta, int refresh_tail,
                          float* gs, float* hs, int stride, hipStream_t stream) {
  dim3 grid((stride + kScorePagesPerBlock - 1) / kScorePagesPerBlock, c.Hkv, c.B);
  const T* qq = static_cast<const T*>(q);
  T* mm = static_cast<T*>(meta);
  const T* kp = static_cast<const T*>(c.k_pool);
#define QSA_SCORE_CASE(GG)                                                                       \
  case GG:                                                                                       \
    hipLaunchKernelGGL((score_kernel<T, GG, kCentroid>), grid, dim3(256), 0, stream, qq, mm,    \
                       c.Hkv, c.seq_lens, c.page_indptr, c.page_indices, kp, c.num_phys,        \
                       refresh_tail, gs, hs, stride, c.err);                                     \
    break;
  switch (c.G) {
    QSA_SCORE_CASE(1)
    QSA_SCORE_CASE(2)
    QSA_SCORE_CASE(4)
    QSA_SCORE_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef QSA_SCORE_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const LaunchCommon& c, const void* q, void* meta, int refresh_tail,
                        float* group_scores, float* head_scores, int stride, hipStream_t stream) {
  return c.bf16 ? launch_score_t<bf16s, false>(c, q, meta, refresh_tail, group_scores, head_scores,
                                               stride, stream)
                : launch_score_t<float, false>(c, q, meta, refresh_tail, group_scores, head_scores,
                                               stride, stream);
}

hipError_t launch_score_centroid(const LaunchCommon& c, const void* q, void* cent,
                                 int refresh_tail, float* group_scores, float* head_scores,
                                 int stride, hipStream_t stream) {
  return c.bf16 ? launch_score_t<bf16s, true>(c, q, cent, refresh_tail, group_scores, head_scores,
                                              stride, stream)
                : launch_score_t<float, true>(c, q, cent, refresh_tail, group_scores, head_scores,
                                              stride, stream);
}

}  // namespace qsa
