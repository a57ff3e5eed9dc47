// Step 4: split-K flash-decode over the selected pages (TinyServe page, §2.3
// stages 3-4: load only the selected pages' K/V, attention fused with the
// load; flash decoding's split + log-sum-exp merge per the CS336 page §9.2
// and the Quail page's join attention).
//
// Work unit = (sequence b, KV head h, a chunk of `chunk` consecutive entries
// of the row's page list). The unit's workgroup has 4 waves; wave w takes
// entries w, w+4, ... of the chunk. Every query head of the GQA group is
// handled by the same wave, so each K/V tile is read from HBM once for g
// heads. Pages are read in place through the page table (no gather copy).
//
// Per page (tile of 16 rows x 256 B, read as 4+4 coalesced 16-byte loads per
// lane):
//  * QK with K in "8 lanes per row" layout: lane l holds chunks l%8 and l%8+8
//    of rows l/8 and l/8+8; q.k partials (v_dot2_f32_bf16 for bf16) are summed
//    over the 8 lanes with DPP, leaving every lane with the 2 x g logits of
//    its two rows.
//  * Online softmax with a lazily moved reference: each (row, head) pair is
//    owned by one lane; the wave's reference max m_h only moves (and the
//    accumulators are rescaled) when some logit exceeds m_h + 8 (log2
//    units), so probabilities stay <= 2^8 and the rescale is rare.
//  * PV with V in linear layout: lane l holds chunk l%16 of rows
//    {l/16, 4+l/16, 8+l/16, 12+l/16}; probabilities move from the QK layout
//    through 512 B of LDS per page; o[g][chunk] accumulates in fp32.
// Unit results (o unnormalised, max, sum) go to the workspace and are merged
// per (b, hq) by merge_kernel.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr float kLazyTau = 8.0f;  // log2 headroom before the reference max moves

template <typename T, int G>
struct DecodeShared {
  static constexpr int D = 16 * Elem<T>::kPerChunk;
  float p[4][2][kPage * G];  // per wave, double-buffered page probabilities
  float o[4][G][D];          // per-wave results for the workgroup combine
  float ml[4][G][2];
};

template <typename T, int G>
__global__ void __launch_bounds__(256) decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ k_pool, const T* __restrict__ v_pool,
    int num_phys, int Hkv, const int* __restrict__ page_indptr,
    const int* __restrict__ page_indices, const int* __restrict__ seq_lens,
    const int* __restrict__ sel, const int* __restrict__ sel_count, int k_stride,
    float scale_log2, int chunk, int max_units, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  constexpr int EPC = Elem<T>::kPerChunk;
  constexpr int D = 16 * EPC;
  constexpr int NP = (2 * G + 7) / 8;  // (row, head) pairs owned per lane
  __shared__ DecodeShared<T, G> sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int u = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int Hq = Hkv * G;
  const int L = seq_lens[b];
  if (L <= 0) return;
  const int n = (L + kPage - 1) / kPage;
  const size_t row = (size_t)b * Hkv + h;
  int count = n;
  if (sel != nullptr) {
    count = sel_count[row];
    count = count < k_stride ? count : k_stride;
    count = count < n ? count : n;  // a row selects distinct pages of the sequence
  }
  const int ubeg = u * chunk;
  if (ubeg >= count) return;  // whole workgroup: nothing in this unit
  const int uend = min(ubeg + chunk, count);
  const int npw = (uend - ubeg > wave) ? (uend - ubeg - wave + 3) / 4 : 0;

  // This wave's pages: physical slot and valid-token count, one per lane.
  // Two dependent loads (selection entry, then table entry).
  int my_p = 0, my_valid = 0;
  if (lane < npw) {
    const int idx = ubeg + wave + 4 * lane;
    const int j = sel != nullptr ? sel[row * k_stride + idx] : idx;
    if (j >= 0 && j < n) {
      const int p = page_indices[page_indptr[b] + j];
      if (p >= 0 && p < num_phys) {
        my_p = p;
        my_valid = min(kPage, L - kPage * j);
      }
    }
  }

  const int gi = lane >> 3;  // K layout: row pair (gi, gi + 8)
  const int qa = lane & 7;   // K layout: chunks qa, qa + 8
  const int hl = qa & (G - 1);  // the head whose logits this lane owns
  const int vr = lane >> 4;  // V layout: rows vr + 4r
  const int vc = lane & 15;  // V layout: chunk

  uint4 qk[G][2];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const char* qrow = reinterpret_cast<const char*>(q) + ((size_t)b * Hq + h * G + hh) * kRowBytes;
    qk[hh][0] = ld16(qrow + qa * 16);
    qk[hh][1] = ld16(qrow + (qa + 8) * 16);
  }

  float o[G][EPC];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < EPC; ++e) o[hh][e] = 0.0f;
  float m_lane = -__builtin_inff();
  float l_lane = 0.0f;

  const char* kbase = reinterpret_cast<const char*>(k_pool) + (size_t)h * kTileBytes;
  const char* vbase = reinterpret_cast<const char*>(v_pool) + (size_t)h * kTileBytes;
  const size_t page_stride = (size_t)Hkv * kTileBytes;

  // Issue the loads of page sp of this wave (K in the QK layout, V linear).
  auto issue = [&](int sp, uint4 (&kA)[2][2], uint4 (&vB)[4]) {
    const int p = __builtin_amdgcn_readlane(my_p, sp);
    const int valid = __builtin_amdgcn_readlane(my_valid, sp);
    if (valid == 0) return;
    const char* kt = kbase + (size_t)p * page_stride;
    const char* vt = vbase + (size_t)p * page_stride;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      kA[s2][0] = ld16(kt + (gi + 8 * s2) * kRowBytes + qa * 16);
      kA[s2][1] = ld16(kt + (gi + 8 * s2) * kRowBytes + (qa + 8) * 16);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) vB[r] = ld16(vt + r * 1024 + lane * 16);
  };

  // Attention over page sp, whose tiles are in kA / vB.
  auto process = [&](int sp, const uint4 (&kA)[2][2], const uint4 (&vB)[4]) {
    const int valid = __builtin_amdgcn_readlane(my_valid, sp);
    if (valid == 0) return;

    // ---- logits of rows gi, gi+8 for every head of the group
    float z[2][G];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float acc = chunk_dot(qk[hh][0], kA[s2][0], 0.0f, T{});
        acc = chunk_dot(qk[hh][1], kA[s2][1], acc, T{});
        z[s2][hh] = sum8(acc);
      }

    // ---- the lane's own (row, head) pairs
    float zl[NP];
    int tok[NP];
    bool act[NP];
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      const int pi = qa + 8 * e;
      act[e] = pi < 2 * G;
      const int s2 = pi / G;
      float zs = z[0][0];
#pragma unroll
      for (int sc = 0; sc < 2; ++sc)
#pragma unroll
        for (int hc = 0; hc < G; ++hc)
          if (sc == s2 && hc == hl) zs = z[sc][hc];
      tok[e] = gi + 8 * s2;
      zl[e] = (act[e] && tok[e] < valid) ? zs * scale_log2 : -__builtin_inff();
    }

    // ---- move the reference max if a logit outgrew it
    bool exceed = false;
#pragma unroll
    for (int e = 0; e < NP; ++e) exceed |= zl[e] > m_lane + kLazyTau;
    if (__builtin_amdgcn_ballot_w64(exceed) != 0) {
      float pm = zl[0];
#pragma unroll
      for (int e = 1; e < NP; ++e) pm = fmaxf(pm, zl[e]);
#pragma unroll
      for (int msk = G; msk < 64; msk <<= 1) pm = fmaxf(pm, xshfl(pm, msk));
      const float mn = fmaxf(m_lane, pm);
      const float alpha = (mn == -__builtin_inff()) ? 1.0f : fast_exp2(m_lane - mn);
      m_lane = mn;
      l_lane *= alpha;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float a = readlane_f(alpha, hh);
#pragma unroll
        for (int e = 0; e < EPC; ++e) o[hh][e] *= a;
      }
    }

    // ---- probabilities to LDS
    float* pb = sh.p[wave][sp & 1];
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      const float pv = act[e] ? fast_exp2(zl[e] - m_lane) : 0.0f;
      l_lane += pv;
      if (act[e]) pb[tok[e] * G + hl] = pv;
    }
    wave_lds_sync();

    // ---- o += p * v
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * r + vr;
      float pr[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) pr[hh] = pb[t * G + hh];
      float vf[EPC];
      chunk_unpack(vB[r], vf, T{});
      if (valid < kPage && t >= valid) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) vf[e] = 0.0f;  // rows past the end may hold anything
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < EPC; ++e) o[hh][e] = __builtin_fmaf(pr[hh], vf[e], o[hh][e]);
    }
    wave_lds_sync();
  };

  // Software pipeline: the next page's loads are in flight while the current
  // page is processed (two register buffers, unrolled so no copies).
  uint4 kA0[2][2], vB0[4], kA1[2][2], vB1[4];
  if (npw > 0) issue(0, kA0, vB0);
  for (int sp = 0; sp < npw; sp += 2) {
    if (sp + 1 < npw) issue(sp + 1, kA1, vB1);
    process(sp, kA0, vB0);
    if (sp + 1 >= npw) break;
    if (sp + 2 < npw) issue(sp + 2, kA0, vB0);
    process(sp + 1, kA1, vB1);
  }

  // ---- wave epilogue: sum l over the lanes of a head, o over the 4 row groups
  float lr = l_lane;
#pragma unroll
  for (int msk = G; msk < 64; msk <<= 1) lr += xshfl(lr, msk);
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      float v = o[hh][e];
      v += xshfl(v, 16);
      v += xshfl(v, 32);
      o[hh][e] = v;
    }
  if (lane < 16) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < EPC; ++e) sh.o[wave][hh][vc * EPC + e] = o[hh][e];
  }
  if (lane < G) {
    sh.ml[wave][lane][0] = m_lane;
    sh.ml[wave][lane][1] = lr;
  }
  __syncthreads();

  // ---- workgroup combine of the 4 waves -> one partial per (unit, head)
  const size_t unit = row * (size_t)max_units + u;
  for (int idx = tid; idx < G * D; idx += 256) {
    const int hh = idx / D;
    const int d = idx - hh * D;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sh.ml[w][hh][0]);
    float acc = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sh.ml[w][hh][0];
      const float sc = (mw == -__builtin_inff()) ? 0.0f : fast_exp2(mw - M);
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
// shared-prefix partials for the cascade), then normalisation. All partial
// maxima are loaded at once (one per lane), so the merge costs two dependent
// loads rather than one per unit.
template <int D>
__global__ void __launch_bounds__(256) merge_kernel(
    int B, int Hkv, int G, const int* __restrict__ seq_lens, const int* __restrict__ sel_count,
    int k_stride, int chunk, int max_units, const float* __restrict__ part_o,
    const float* __restrict__ part_ml, const float* __restrict__ pre_o,
    const float* __restrict__ pre_ml, int n_pre, float* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int Hq = Hkv * G;
  if (gw >= B * Hq) return;
  const int b = gw / Hq;
  const int hq = gw - b * Hq;
  const int h = hq / G;
  const int hh = hq - h * G;
  const size_t row = (size_t)b * Hkv + h;
  const int L = seq_lens[b];
  const int n = L > 0 ? (L + kPage - 1) / kPage : 0;
  int count = n;
  if (sel_count != nullptr) {
    count = sel_count[row];
    count = count < k_stride ? count : k_stride;
    count = count < n ? count : n;
  }
  int units = count > 0 ? (count + chunk - 1) / chunk : 0;
  units = units < max_units ? units : max_units;  // never beyond the planned workspace
  const int total = units + n_pre;

  // partial i: decode unit i (i < units) or prefix split i - units
  auto part = [&](int i, const float*& po, const float*& pml) {
    if (i < units) {
      const size_t unit = row * (size_t)max_units + i;
      po = part_o + (unit * G + hh) * D;
      pml = part_ml + (unit * G + hh) * 2;
    } else {
      const size_t pr = ((size_t)h * n_pre + (i - units)) * ((size_t)B * G) + (size_t)b * G + hh;
      po = pre_o + pr * D;
      pml = pre_ml + pr * 2;
    }
  };

  float M = -__builtin_inff();
  for (int base = 0; base < total; base += 64) {
    const int i = base + lane;
    if (i < total) {
      const float* po;
      const float* pml;
      part(i, po, pml);
      M = fmaxf(M, pml[0]);
    }
  }
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) M = fmaxf(M, xshfl(M, msk));

  float lsum = 0.0f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
  for (int base = 0; base < total; base += 64) {
    const int i = base + lane;
    float w = 0.0f;
    if (i < total) {
      const float* po;
      const float* pml;
      part(i, po, pml);
      const float m = pml[0];
      w = (m == -__builtin_inff()) ? 0.0f : fast_exp2(m - M);
      lsum += w * pml[1];
    }
    const int cnt = min(64, total - base);
    for (int t = 0; t < cnt; ++t) {
      const float wt = readlane_f(w, t);
      const float* po;
      const float* pml;
      part(base + t, po, pml);
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = __builtin_fmaf(wt, po[lane + 64 * e], acc[e]);
    }
  }
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) lsum += xshfl(lsum, msk);

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
                           Partials part, hipStream_t stream) {
  dim3 grid(plan.max_units, c.Hkv, c.B);
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
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_split(const LaunchCommon& c, const void* q, const int* sel,
                               const int* sel_count, int k, float scale_log2,
                               const DecodePlan& plan, Partials part, hipStream_t stream) {
  if (plan.max_units <= 0) return hipSuccess;
  return c.bf16 ? launch_decode_t<bf16s>(c, q, sel, sel_count, k, scale_log2, plan, part, stream)
                : launch_decode_t<float>(c, q, sel, sel_count, k, scale_log2, plan, part, stream);
}

hipError_t launch_merge(const LaunchCommon& c, const int* sel_count, int k, const DecodePlan& plan,
                        Partials part, Partials prefix, int n_prefix_splits, float* out,
                        float* lse, hipStream_t stream) {
  const int waves = c.B * c.Hq;
  dim3 grid((waves + 3) / 4);
  if (c.D == 128) {
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(256), 0, stream, c.B, c.Hkv, c.G, c.seq_lens,
                       sel_count, k, plan.chunk, plan.max_units, part.o, part.ml, prefix.o,
                       prefix.ml, n_prefix_splits, out, lse);
  } else {
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(256), 0, stream, c.B, c.Hkv, c.G, c.seq_lens,
                       sel_count, k, plan.chunk, plan.max_units, part.o, part.ml, prefix.o,
                       prefix.ml, n_prefix_splits, out, lse);
  }
  return hipGetLastError();
}

}  // namespace qsa
