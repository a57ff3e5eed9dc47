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
// per (b, hq) by merge_kernel. (Merging inside the last-arriving unit would
// need device-scope release fences in every unit; on this chip those write
// back the XCD's L2 and cost far more than the separate launch.)
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
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ k_pool, const T* __restrict__ v_pool,
    int num_phys, int Hkv, const int* __restrict__ page_indptr,
    const int* __restrict__ page_indices, const int* __restrict__ seq_lens,
    const int* __restrict__ sel, const int* __restrict__ sel_count, int k_stride,
    float scale_log2, int chunk, int max_units, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  constexpr int EPC = Elem<T>::kPerChunk;
  constexpr int D = 16 * EPC;
  constexpr int NP = (2 * G + 7) / 8;  // (row, head) pairs owned per lane
  constexpr int kStages = G >= 8 ? 2 : 3;  // pages in flight per wave (register budget)
  __shared__ DecodeShared<T, G> sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int u = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
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
  // Branch-free, so the compiler's wait counts stay exact and the next page's
  // loads overlap the current page's math; a skipped page (no valid tokens)
  // reads physical slot 0, which always exists.
  auto issue = [&](int sp, uint4 (&kA)[2][2], uint4 (&vB)[4]) {
    const int p = __builtin_amdgcn_readlane(my_p, sp);
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
      if (__builtin_expect(valid < kPage, 0)) {
        // rows past the end of a partial last page may hold anything
        if (t >= valid) {
#pragma unroll
          for (int e = 0; e < EPC; ++e) vf[e] = 0.0f;
        }
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < EPC; ++e) o[hh][e] = __builtin_fmaf(pr[hh], vf[e], o[hh][e]);
    }
    wave_lds_sync();
  };

  // Software pipeline: the loads of the next kStages-1 pages are in flight
  // while the current page is processed (HBM latency is several times the
  // math of one page). kStages register buffers, rotated by an unrolled loop
  // so no data is copied; past the wave's last page the prefetch re-reads
  // that page (an L2 hit, no extra HBM traffic).
  if (npw > 0) {
    uint4 kA0[2][2], vB0[4], kA1[2][2], vB1[4];
    issue(0, kA0, vB0);
    int sp = 0;
    if constexpr (kStages == 2) {
      while (true) {
        issue(min(sp + 1, npw - 1), kA1, vB1);
        process(sp, kA0, vB0);
        if (++sp >= npw) break;
        issue(min(sp + 1, npw - 1), kA0, vB0);
        process(sp, kA1, vB1);
        if (++sp >= npw) break;
      }
    } else {
      uint4 kA2[2][2], vB2[4];
      issue(min(1, npw - 1), kA1, vB1);
      while (true) {
        issue(min(sp + 2, npw - 1), kA2, vB2);
        process(sp, kA0, vB0);
        if (++sp >= npw) break;
        issue(min(sp + 2, npw - 1), kA0, vB0);
        process(sp, kA1, vB1);
        if (++sp >= npw) break;
        issue(min(sp + 2, npw - 1), kA1, vB1);
        process(sp, kA2, vB2);
        if (++sp >= npw) break;
      }
    }
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
  for (int idx2 = tid; idx2 < G * D; idx2 += 256) {
    const int hh = idx2 / D;
    const int d = idx2 - hh * D;
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
  constexpr int kBatch = 8;
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
