// Step 4: split-K flash-decode over the selected pages (TinyServe page, §2.3
// stages 3-4: load only the selected pages' K/V, attention fused with the
// load; flash decoding's split + log-sum-exp merge per the CS336 page §9.2
// and the Quail page's join attention).
//
// Work unit = (sequence b, KV head h, a chunk of `chunk` consecutive entries
// of the row's page list), block (h, b, chunk). The unit's workgroup has 4 waves; wave w takes
// entries w, w+4, ... of the chunk and runs them through the per-wave
// attention: on the matrix cores (decode_mfma.h) for bf16 groups of 4 or
// more heads, else on the vector ALU (decode_wave.h). Unit results (o unnormalised, max, sum) go to
// the workspace and are merged per (b, hq) by merge_kernel. (Merging inside
// the last-arriving unit would need device-scope release fences in every
// unit; on this chip those write back the XCD's L2 and cost far more than the
// separate launch.)
#include "decode_mfma.h"
#include "decode_wave.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

// bf16 groups of 4 or more query heads attend on the matrix cores
// (decode_mfma.h); fp32 pools and smaller groups on the vector ALU
// (decode_wave.h), where the products are too narrow to gain.
template <typename T>
struct IsBf16 {
  static constexpr bool value = false;
};
template <>
struct IsBf16<bf16s> {
  static constexpr bool value = true;
};
template <typename T, int G>
constexpr bool use_mfma() {
  return IsBf16<T>::value && G >= 4;
}

template <typename T, int G, bool kMfma = use_mfma<T, G>()>
struct DecodeShared {
  static constexpr int D = WaveAttn<T, G>::D;
  float p[4][WaveAttn<T, G>::kPBufFloats];  // per wave, double-buffered page probabilities
  float o[4][G][D];                         // per-wave results for the workgroup combine
  float ml[4][G][2];
  uint4 q[WaveAttn<T, G>::kQInLds ? G * kRowBytes / 16 : 1];  // the group's query rows
};
template <typename T, int G>
struct DecodeShared<T, G, true> {
  static constexpr int D = WaveAttnMfma<G>::D;
  alignas(16) char v[4][WaveAttnMfma<G>::kLdsBytes];  // per wave, the staged V tiles
  alignas(16) float o[4][G][D];
  float ml[4][G][2];
};

template <typename T, int G>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ k_pool, const T* __restrict__ v_pool,
    int num_phys, int Hkv, const int* __restrict__ page_indptr,
    const int* __restrict__ page_indices, const int* __restrict__ seq_lens,
    const int* __restrict__ sel, const int* __restrict__ sel_count, int k_stride,
    float scale_log2, int chunk, int max_units, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  using WA = WaveAttn<T, G>;
  constexpr int EPC = WA::EPC;
  constexpr int D = WA::D;
  constexpr bool kMfma = use_mfma<T, G>();
  __shared__ DecodeShared<T, G> sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int u = blockIdx.z;
  const int Hq = Hkv * G;
  const size_t row = (size_t)b * Hkv + h;
  const int ubeg = u * chunk;
  // First level of loads, all independent: row length, selection count,
  // table base and (speculatively) this wave's selection entries.
  const int L = seq_lens[b];
  const int cnt_sel = sel != nullptr ? sel_count[row] : 0;
  const int tbase = page_indptr[b];
  const int idx = ubeg + wave + 4 * lane;
  int jsel = idx;
  if (sel != nullptr && lane < (chunk >> 2) && idx < k_stride) jsel = sel[row * k_stride + idx];
  const int n = L > 0 ? (L + kPage - 1) / kPage : 0;
  int count = n;
  if (sel != nullptr) {
    count = cnt_sel < k_stride ? cnt_sel : k_stride;
    count = count < n ? count : n;  // a row selects distinct pages of the sequence
    count = count > 0 ? count : 0;
  }
  int units = (count + chunk - 1) / chunk;
  units = units < 1 ? 1 : (units < max_units ? units : max_units);
  if (u >= units) return;  // whole workgroup: nothing in this unit
  const int uend = min(ubeg + chunk, count);
  const int npw = (uend - ubeg > wave) ? (uend - ubeg - wave + 3) / 4 : 0;

  // This wave's pages: physical slot and valid-token count, one per lane.
  int my_p = 0, my_valid = 0;
  if (lane < npw) {
    const int j = jsel;
    if (j >= 0 && j < n) {
      const int p = page_indices[tbase + j];
      if (p >= 0 && p < num_phys) {
        my_p = p;
        my_valid = min(kPage, L - kPage * j);
      }
    }
  }

  const char* qrows = reinterpret_cast<const char*>(q) + ((size_t)b * Hq + h * G) * kRowBytes;
  LanePages src{my_p, my_valid, npw};
  const char* kbase = reinterpret_cast<const char*>(k_pool) + (size_t)h * kTileBytes;
  const char* vbase = reinterpret_cast<const char*>(v_pool) + (size_t)h * kTileBytes;
  const size_t page_stride = (size_t)Hkv * kTileBytes;
  if constexpr (kMfma) {
    WaveAttnMfma<G> wa;
    wa.init(qrows, lane);
    wa.run(src, kbase, vbase, page_stride, scale_log2, sh.v[wave], lane);
    wa.store(&sh.o[wave][0][0], &sh.ml[wave][0][0], lane);
  } else {
    if constexpr (WA::kQInLds) {
      if (tid < G * kRowBytes / 16) sh.q[tid] = ld16(qrows + tid * 16);
      __syncthreads();
      qrows = reinterpret_cast<const char*>(sh.q);
    }
    WA wa;
    wa.init(qrows, lane);
    wa.run(src, kbase, vbase, page_stride, scale_log2, sh.p[wave], lane);
    // ---- wave epilogue
    float mw, lw;
    wa.reduce(&mw, &lw);
    if (lane < 16) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < EPC; ++e) sh.o[wave][hh][lane * EPC + e] = wa.o[hh][e];
    }
    if (lane < G) {
      sh.ml[wave][lane][0] = mw;
      sh.ml[wave][lane][1] = lw;
    }
  }
  // ---- the workgroup combine of the 4 waves -> one partial per (unit, head)
  __syncthreads();

  const size_t unit = row * (size_t)max_units + u;
  for (int idx2 = tid; idx2 < G * D; idx2 += 256) {
    const int hh = idx2 / D;
    const int d = idx2 - hh * D;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sh.ml[w][hh][0]);
    float acc = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw2 = sh.ml[w][hh][0];
      const float sc = (mw2 == -__builtin_inff()) ? 0.0f : fast_exp2(mw2 - M);
      acc += sh.o[w][hh][d] * sc;
      lsum += sh.ml[w][hh][1] * sc;
    }
    part_o[(unit * G + hh) * D + d] = acc;
    if (d == 0) {
      part_ml[(unit * G + hh) * 2 + 0] = M;
      part_ml[(unit * G + hh) * 2 + 1] = lsum;
    }
  }
}

// One wave per (b, hq): log-sum-exp merge of the unit partials (and of the
// shared-prefix partials for the cascade), then normalisation. The partials
// are loaded without waiting for the row's unit count (every slot the row can
// own is in bounds), so the merge costs one round of dependent loads.
template <int D>
__global__ void __launch_bounds__(256) merge_kernel(
    int B, int Hkv, int G, const int* __restrict__ seq_lens, const int* __restrict__ sel_count,
    int k_stride, int chunk, int max_units, const float* __restrict__ part_o,
    const float* __restrict__ part_ml, const float* __restrict__ pre_o,
    const float* __restrict__ pre_ml, int n_pre, float* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int PER = D / 64;
  constexpr int kBatch = 16;  // partial slots loaded per round (a cascade row has 8 prefix splits + suffix units)
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Hq = Hkv * G;
  if (gw >= B * Hq) return;
  const int b = gw / Hq;
  const int hq = gw - b * Hq;
  const int h = hq / G;
  const int hh = hq - h * G;
  const size_t row = (size_t)b * Hkv + h;
  const size_t pre_row = (size_t)b * G + hh;
  const int L = seq_lens[b];
  const int cnt_sel = sel_count != nullptr ? sel_count[row] : 0;
  const int slots = max_units + n_pre;

  float M = -__builtin_inff(), lsum = 0.0f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
  int units = -1;
  for (int base = 0; base < slots; base += kBatch) {
    float m[kBatch], l[kBatch], v[kBatch][PER];
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      const int i = min(base + t, slots - 1);
      const float* po;
      const float* pml;
      if (i < max_units) {
        const size_t un = row * max_units + i;
        po = part_o + (un * G + hh) * D;
        pml = part_ml + (un * G + hh) * 2;
      } else {
        const size_t pr = ((size_t)h * n_pre + (i - max_units)) * ((size_t)B * G) + pre_row;
        po = pre_o + pr * D;
        pml = pre_ml + pr * 2;
      }
      m[t] = pml[0];
      l[t] = pml[1];
#pragma unroll
      for (int e = 0; e < PER; ++e) v[t][e] = po[lane + 64 * e];
    }
    if (units < 0) {
      const int n = L > 0 ? (L + kPage - 1) / kPage : 0;
      int count = n;
      if (sel_count != nullptr) {
        count = cnt_sel < k_stride ? cnt_sel : k_stride;
        count = count < n ? count : n;
        count = count > 0 ? count : 0;
      }
      units = (count + chunk - 1) / chunk;
      units = units < max_units ? units : max_units;
    }
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      const int i = base + t;
      // slots past the row's units (and past the list) hold stale values
      const bool use = i < slots && (i < units || i >= max_units);
      if (!use || m[t] == -__builtin_inff()) continue;
      if (m[t] > M) {
        const float a = (M == -__builtin_inff()) ? 0.0f : fast_exp2(M - m[t]);
        lsum *= a;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] *= a;
        M = m[t];
      }
      const float w = fast_exp2(m[t] - M);
      lsum = __builtin_fmaf(w, l[t], lsum);
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = __builtin_fmaf(w, v[t][e], acc[e]);
    }
  }
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[(size_t)gw * D + lane + 64 * e] = acc[e] * inv;
  if (lse != nullptr && lane == 0) {
    lse[gw] = lsum > 0.0f ? (M + __log2f(lsum)) * 0.69314718055994530942f : -__builtin_inff();
  }
}

template <typename T>
hipError_t launch_decode_t(const LaunchCommon& c, const void* q, const int* sel,
                           const int* sel_count, int k, float scale_log2, const DecodePlan& plan,
                           Partials part, Partials prefix, int n_prefix, float* out, float* lse,
                           hipStream_t stream) {
  // The KV head is the fastest grid dimension and the unit the slowest.
  // Workgroups go round-robin over the 8 XCDs by linear id, so with 8 KV
  // heads every XCD serves one head of every row (equal work); with the unit
  // fastest instead, XCD x would get units x and x + 8 of every row, and
  // only long rows have the high units.
  dim3 grid(c.Hkv, c.B, plan.max_units);
  const T* qq = static_cast<const T*>(q);
  const T* kk = static_cast<const T*>(c.k_pool);
  const T* vv = static_cast<const T*>(c.v_pool);
#define QSA_DECODE_CASE(GG)                                                                     \
  case GG:                                                                                      \
    hipLaunchKernelGGL((decode_split_kernel<T, GG>), grid, dim3(256), 0, stream, qq, kk, vv,    \
                       c.num_phys, c.Hkv, c.page_indptr, c.page_indices, c.seq_lens, sel,       \
                       sel_count, k, scale_log2, plan.chunk, plan.max_units, part.o, part.ml); \
    break;
  switch (c.G) {
    QSA_DECODE_CASE(1)
    QSA_DECODE_CASE(2)
    QSA_DECODE_CASE(4)
    QSA_DECODE_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef QSA_DECODE_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 mgrid((c.B * c.Hq + 3) / 4);
  const int* sc = sel != nullptr ? sel_count : nullptr;
  if (c.D == 128) {
    hipLaunchKernelGGL(merge_kernel<128>, mgrid, dim3(256), 0, stream, c.B, c.Hkv, c.G, c.seq_lens,
                       sc, k, plan.chunk, plan.max_units, part.o, part.ml, prefix.o, prefix.ml,
                       n_prefix, out, lse);
  } else {
    hipLaunchKernelGGL(merge_kernel<64>, mgrid, dim3(256), 0, stream, c.B, c.Hkv, c.G, c.seq_lens,
                       sc, k, plan.chunk, plan.max_units, part.o, part.ml, prefix.o, prefix.ml,
                       n_prefix, out, lse);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const LaunchCommon& c, const void* q, const int* sel, const int* sel_count,
                         int k, float scale_log2, const DecodePlan& plan, Partials part,
                         Partials prefix, int n_prefix, float* out, float* lse,
                         hipStream_t stream) {
  if (plan.max_units <= 0) return hipSuccess;
  return c.bf16 ? launch_decode_t<bf16s>(c, q, sel, sel_count, k, scale_log2, plan, part, prefix,
                                         n_prefix, out, lse, stream)
                : launch_decode_t<float>(c, q, sel, sel_count, k, scale_log2, plan, part, prefix,
                                         n_prefix, out, lse, stream);
}

}  // namespace qsa
