// Steps 2-4 of one decode step for rows of at most 64 pages, one wave per
// (sequence, KV head) row (TinyServe page, §3.2: score the pages, pick the
// top-K and attend over them in one kernel, nothing materialised between the
// steps; the score is §2.2, the selection §2.3), with an optional log-sum-exp
// merge of shared-prefix partials (Quail page, join attention) so that the
// suffix half of a selective cascade step is one launch.
//
// Short rows leave too little work for a workgroup per row (the suffix rows of
// a shared-prefix batch hold 32 pages and keep 9): one wave does everything,
// with no workgroup barrier, and four independent rows share a workgroup.
//  1. Score: the row's [m | M] records (logical page order, contiguous), 16
//     lanes per page and 4 pages per step with the score kernel's arithmetic
//     (q split by sign, v_dot2, DPP row sum, group max), so the group scores
//     are bit-identical to qsa_score_pages'. With refresh_tail the tail page's
//     record is rebuilt from its keys first, written back and scored. Page j's
//     order key ends in lane j.
//  2. Select: lane j's rank is the number of pages with a larger key, or an
//     equal key and a smaller index; the K_eff = min(k, n) pages of rank
//     below K_eff are selected (ties to the smaller page, as the radix
//     select), listed in ascending page order by their position among the
//     selected lanes.
//  3. Attend: the selected pages through the matrix-core page loop of
//     decode_mfma.h (lane i holds the i-th selected page).
//  4. Merge: the wave's (max, sum, o) per head with the n_pre prefix
//     partials of its query rows, normalised into out / lse.
#pragma once

#include "decode_mfma.h"
#include "qsa_internal.h"

namespace qsa {
namespace shortrow {

constexpr int kShortWaves = 4;  // rows per workgroup

// rows per launch block; the block's waves are independent
template <int G>
struct ShortShared {
  alignas(16) char v[kShortWaves][WaveAttnMfma<G>::kLdsBytes];  // staged V tiles
  alignas(16) float o[kShortWaves][G][128];                      // the wave's partial
  float ml[kShortWaves][G][2];
};

// The rows of workgroup `block` (kShortWaves of them, one per wave). With
// suf_o non-null each row's unmerged partial (o relative to its max, then
// (max, sum) per head, the layout of split-K partials with one unit per row)
// goes to suf_o / suf_ml instead of out / lse, and the prefix partials are
// not read.
template <int G>
__device__ __forceinline__ void short_row_block(ShortShared<G>& sh, int block, int tid, const bf16s* __restrict__ q, bf16s* __restrict__ meta, int stride,
                 const bf16s* __restrict__ k_pool, const bf16s* __restrict__ v_pool, int num_phys, int B,
                 int Hkv, const int* __restrict__ page_indptr, const int* __restrict__ page_indices,
                 const int* __restrict__ seq_lens, int refresh_tail, int k, float scale_log2,
                 const float* __restrict__ pre_o, const float* __restrict__ pre_ml, int n_pre,
                 float* __restrict__ out, float* __restrict__ lse, float* __restrict__ group_scores,
                 int* __restrict__ sel, int* __restrict__ sel_count, unsigned int* __restrict__ err,
    float* __restrict__ suf_o, float* __restrict__ suf_ml) {
  using WA = WaveAttnMfma<G>;
  constexpr int D = 128;
  constexpr int kRec = 2 * kRowBytes;  // [m | M] record
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row_i = block * kShortWaves + wave;
  if (row_i >= B * Hkv) return;  // whole wave; the waves share no barrier
  const int b = row_i / Hkv;
  const int h = row_i - b * Hkv;
  const int Hq = Hkv * G;
  const size_t row = (size_t)row_i;
  const int c = lane & 15;     // chunk within a record
  const int slot = lane >> 4;  // page of a 4-page step

  // ---- first loads: length, table base, the query chunks, the table entry
  // of page `lane` and the first records
  const int L = seq_lens[b];
  const int tbase = page_indptr[b];
  const int n = L > 0 ? min(min((L + kPage - 1) / kPage, stride), 64) : 0;  // the host keeps n <= 64
  const char* qrows = reinterpret_cast<const char*>(q) + ((size_t)b * Hq + h * G) * kRowBytes;
  uint4 qn[G], qp[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) qn[hh] = ld16(qrows + hh * kRowBytes + c * 16);
  const int pj = (n > 0) ? page_indices[tbase + min(lane, n - 1)] : 0;  // this lane's page's slot
  const char* mrow = reinterpret_cast<const char*>(meta) + row * stride * kRec;
  // records of 4-step chunk ch (16 pages); pages past the row read the
  // row's last stride slot (in bounds), their scores are masked
  constexpr int kSteps = 4;
  auto issue = [&](int ch, uint4 (&bm)[kSteps], uint4 (&bM)[kSteps]) {
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
      const int j = min(16 * ch + 4 * t + slot, stride - 1);
      bm[t] = ld16(mrow + (size_t)j * kRec + c * 16);
      bM[t] = ld16(mrow + (size_t)j * kRec + 256 + c * 16);
    }
  };
  const int nch = (n + 15) / 16;
  uint4 bm0[kSteps], bM0[kSteps], bm1[kSteps], bM1[kSteps];
  issue(0, bm0, bM0);
  issue(min(1, max(nch - 1, 0)), bm1, bM1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const uint4 qc = qn[hh];
    chunk_sign_split(qc, qn[hh], qp[hh], bf16s{});
  }
  auto score_page = [&](const uint4& m, const uint4& M) -> float {
    float gmax = -__builtin_inff();
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float acc = chunk_dot(qn[hh], m, 0.0f, bf16s{});
      acc = chunk_dot(qp[hh], M, acc, bf16s{});
      gmax = fmaxf(gmax, sum16(acc));
    }
    return gmax;
  };

  // ---- tail-page refresh (its record rebuilt from the keys, written back)
  const int jt = n - 1;
  bool tail_ok = false;
  float tail_score = 0.0f;
  if (refresh_tail && n > 0) {
    const int tp = __builtin_amdgcn_readlane(pj, jt);
    tail_ok = tp >= 0 && tp < num_phys;
    if (tail_ok) {
      uint4 tmn, tmx;
      const char* tile = reinterpret_cast<const char*>(k_pool) + ((size_t)tp * Hkv + h) * kTileBytes;
      tile_minmax<bf16s>(tile, min(kPage, L - kPage * jt), lane, tmn, tmx);
      char* trec = reinterpret_cast<char*>(meta) + (row * stride + jt) * kRec;
      if (lane < 32) st16(trec + (lane >> 4) * 256 + c * 16, lane < 16 ? tmn : tmx);
      tail_score = score_page(tmn, tmx);
    } else if (lane == 0) {
      report_bad(err, kErrPhys);  // the stored record is scored unchanged
    }
  }

  // ---- scores: page j's order key into lane j
  uint32_t mykey = 0u;
  auto score_chunk = [&](int ch, const uint4 (&bm)[kSteps], const uint4 (&bM)[kSteps]) {
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
      const float s = score_page(bm[t], bM[t]);
      // the 4 pages of the step sit in lanes 0, 16, 32, 48: gather them
      // into lanes 16 ch + 4 t .. + 3
      const uint32_t key = score_key(s);
      const uint32_t got = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * (lane & 3)) << 2, (int)key);
      if ((lane >> 2) == 4 * ch + t) mykey = got;
    }
  };
  score_chunk(0, bm0, bM0);
  if (nch > 1) {
    score_chunk(1, bm1, bM1);
    for (int ch = 2; ch < nch; ++ch) {  // rows of 33..64 pages
      issue(ch, bm0, bM0);
      score_chunk(ch, bm0, bM0);
    }
  }
  if (tail_ok && lane == jt) mykey = score_key(tail_score);
  if (group_scores != nullptr) {
    for (int j = lane; j < stride; j += 64)
      group_scores[row * stride + j] = j < n ? __uint_as_float(key_to_f32(mykey)) : -__builtin_inff();
  }

  // ---- select: rank of lane j among the row's pages (larger key first,
  // ties to the smaller page)
  const int keff = min(k, n);
  int rank = 0;
  for (int i = 0; i < n; ++i) {
    const uint32_t ki = (uint32_t)__builtin_amdgcn_readlane((int)mykey, i);
    rank += (ki > mykey || (ki == mykey && i < lane)) ? 1 : 0;
  }
  const bool chosen = lane < n && rank < keff;
  const unsigned long long mask = __builtin_amdgcn_ballot_w64(chosen);
  const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                            __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
  if (sel != nullptr) {
    if (chosen) sel[row * k + pos] = lane;
    for (int i = keff + lane; i < k; i += 64) sel[row * k + i] = -1;
    if (lane == 0) sel_count[row] = keff;
  }
  // the i-th selected page's slot and valid rows into lane i
  const bool pok = pj >= 0 && pj < num_phys;
  if (chosen && !pok) report_bad(err, kErrPhys);
  const int my_valid_j = (chosen && pok) ? min(kPage, L - kPage * lane) : 0;
  // destinations form a permutation of the 64 lanes: the chosen lanes go to
  // their list positions 0 .. keff-1 (exactly keff lanes are chosen: the
  // ranks are distinct), the others, in lane order, to keff .. 63
  const int dst = (chosen ? pos : keff + (lane - pos)) << 2;
  const int my_p = __builtin_amdgcn_ds_permute(dst, pok ? pj : 0);
  const int my_valid = __builtin_amdgcn_ds_permute(dst, my_valid_j);
  LanePages src{my_p, lane < keff ? my_valid : 0, keff};

  // ---- attention over the selected pages
  WA wa;
  wa.init(qrows, lane);
  wa.run(src, reinterpret_cast<const char*>(k_pool) + (size_t)h * kTileBytes,
         reinterpret_cast<const char*>(v_pool) + (size_t)h * kTileBytes, (size_t)Hkv * kTileBytes,
         scale_log2, sh.v[wave], lane);
  wa.store(&sh.o[wave][0][0], &sh.ml[wave][0][0], lane);
  wave_lds_sync();
  if (suf_o != nullptr) {  // the unmerged partial, for a merge launched later
    const size_t r0 = row * G;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      suf_o[(r0 + hh) * D + lane] = sh.o[wave][hh][lane];
      suf_o[(r0 + hh) * D + lane + 64] = sh.o[wave][hh][lane + 64];
    }
    if (lane < 2 * G) suf_ml[r0 * 2 + lane] = (&sh.ml[wave][0][0])[lane];
    return;
  }

  // ---- merge with the prefix partials (layout [Hkv][n_pre][B * G] rows)
  // and normalise; lane l covers dims l and l + 64 of every head. A round
  // issues the loads of kPB partials of every head before combining any.
  constexpr int kPB = 32 / G;
  float M[G], lsum[G], a0[G], a1[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    M[hh] = sh.ml[wave][hh][0];
    const bool any = M[hh] != -__builtin_inff();
    lsum[hh] = any ? sh.ml[wave][hh][1] : 0.0f;
    a0[hh] = any ? sh.o[wave][hh][lane] : 0.0f;
    a1[hh] = any ? sh.o[wave][hh][lane + 64] : 0.0f;
  }
  for (int base = 0; base < n_pre; base += kPB) {
    float pm[G][kPB], pl[G][kPB], p0[G][kPB], p1[G][kPB];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int t = 0; t < kPB; ++t) {
        const int si = min(base + t, n_pre - 1);
        const size_t pr = ((size_t)h * n_pre + si) * ((size_t)B * G) + (size_t)b * G + hh;
        pm[hh][t] = pre_ml[pr * 2 + 0];
        pl[hh][t] = pre_ml[pr * 2 + 1];
        p0[hh][t] = pre_o[pr * D + lane];
        p1[hh][t] = pre_o[pr * D + lane + 64];
      }
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int t = 0; t < kPB; ++t) {
        const float m2 = pm[hh][t];
        if (base + t >= n_pre || m2 == -__builtin_inff()) continue;
        if (m2 > M[hh]) {
          const float a = (M[hh] == -__builtin_inff()) ? 0.0f : fast_exp2(M[hh] - m2);
          lsum[hh] *= a;
          a0[hh] *= a;
          a1[hh] *= a;
          M[hh] = m2;
        }
        const float w = fast_exp2(m2 - M[hh]);
        lsum[hh] = __builtin_fmaf(w, pl[hh][t], lsum[hh]);
        a0[hh] = __builtin_fmaf(w, p0[hh][t], a0[hh]);
        a1[hh] = __builtin_fmaf(w, p1[hh][t], a1[hh]);
      }
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float inv = lsum[hh] > 0.0f ? 1.0f / lsum[hh] : 0.0f;
    const size_t qrow = (size_t)b * Hq + h * G + hh;
    out[qrow * D + lane] = a0[hh] * inv;
    out[qrow * D + lane + 64] = a1[hh] * inv;
    if (lse != nullptr && lane == 0)
      lse[qrow] = lsum[hh] > 0.0f ? (M[hh] + __log2f(lsum[hh])) * 0.69314718055994530942f : -__builtin_inff();
  }
}

}  // namespace shortrow
}  // namespace qsa
