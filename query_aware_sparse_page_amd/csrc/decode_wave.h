// One wave's share of paged decode attention (TinyServe page, §2.3 stages
// 3-4: only the chosen pages' K/V are loaded and attention runs on them as
// they arrive; the online softmax and its (max, sum, unnormalised output)
// partial state follow the CS336 page §9.2).
//
// A wave owns a list of pages (one per lane: physical slot and valid-token
// count) and every query head of one GQA group, so each K/V tile is read
// from HBM once for g heads. Pages are read in place through the page table.
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
#pragma once

#include "qsa_device.h"

namespace qsa {

constexpr float kLazyTau = 8.0f;  // log2 headroom before the reference max moves

// kStagesArg page buffers per wave (kStagesArg - 1 pages in flight while
// one is computed); the default is what the register file holds at two
// waves per SIMD: three at g <= 4, two at g = 8. At g = 8 the query rows
// (8 VGPRs per head) are read from LDS for every page instead of being held
// in registers (the caller stages them in LDS). kStreamArg: the K/V tile
// loads carry the non-temporal hint (ld16_stream).
template <typename T, int G, int kStagesArg = 2, bool kStreamArg = false>
struct WaveAttn {
  static constexpr int EPC = Elem<T>::kPerChunk;
  static constexpr int D = 16 * EPC;
  static constexpr int NP = (2 * G + 7) / 8;         // (row, head) pairs owned per lane
  static constexpr int kStages = kStagesArg;         // page buffers per wave
  static constexpr bool kStream = kStreamArg;
  static constexpr bool kQInLds = G >= 8;            // query rows read from LDS
  static constexpr int kPBufFloats = 2 * kPage * G;  // LDS per wave: double-buffered probabilities
  // s_waitcnt immediate (gfx9 layout: vmcnt in bits 3:0 and 15:14, expcnt
  // and lgkmcnt left at their maxima) that waits until at most the loads of
  // kStages-1 pages (8 vector loads each) are outstanding.
  static constexpr int kSkipVm = (kStages - 1) * 8;
  static constexpr int kSkipWait = (kSkipVm & 15) | ((kSkipVm >> 4) << 14) | 0x0F70;
  static_assert(kSkipVm < 64, "vmcnt holds at most 63");

  uint4 qk[G][2];     // the group's query rows, K layout (registers)
  const char* q_lds;  // or: the group's query rows in LDS (kQInLds)
  float o[G][EPC];
  float m_lane;    // reference max of head (lane & (G-1)), log2 units
  float l_lane;    // this lane's share of that head's sum

  // q_rows: the G consecutive query rows of the group (256 B each), in
  // LDS when kQInLds, else in global memory.
  __device__ __forceinline__ void init(const char* q_rows, int lane) {
    const int qa = lane & 7;
    if constexpr (kQInLds) {
      q_lds = q_rows;
    } else {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        qk[hh][0] = ld16(q_rows + hh * kRowBytes + qa * 16);
        qk[hh][1] = ld16(q_rows + hh * kRowBytes + (qa + 8) * 16);
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < EPC; ++e) o[hh][e] = 0.0f;
    m_lane = -__builtin_inff();
    l_lane = 0.0f;
  }

  // Attention over the pages a page source hands this wave, one at a time:
  // src.empty() says whether the wave gets any page; src.next(&p, &v) gives
  // the next page's physical slot p and valid-token count v (0: skip the
  // page; -1: no more pages, p then naming a page the wave has read).
  // kbase / vbase point at the KV head's tile of physical page 0; tiles of
  // consecutive physical pages are page_stride bytes apart. pbuf: this
  // wave's kPBufFloats of LDS.
  template <class Src>
  __device__ __forceinline__ void run(Src& src, const char* kbase, const char* vbase,
                                      size_t page_stride, float scale_log2, float* pbuf,
                                      int lane) {
    const int gi = lane >> 3;      // K layout: row pair (gi, gi + 8)
    const int qa = lane & 7;       // K layout: chunks qa, qa + 8
    const int hl = qa & (G - 1);   // the head whose logits this lane owns
    const int vr = lane >> 4;      // V layout: rows vr + 4r

    // Issue the loads of the next page of the source (K in the QK layout, V
    // linear) and return its valid-token count. Branch-free, so the
    // compiler's wait counts stay exact and the next pages' loads overlap the
    // current page's math; past the wave's last page it re-reads a page it
    // has read (an L2 hit, no extra HBM traffic).
    auto issue = [&](uint4 (&kA)[2][2], uint4 (&vB)[4]) -> int {
      int p, valid;
      src.next(&p, &valid);
      const char* kt = kbase + (size_t)p * page_stride;
      const char* vt = vbase + (size_t)p * page_stride;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        kA[s2][0] = ld16_as<kStream>(kt + (gi + 8 * s2) * kRowBytes + qa * 16);
        kA[s2][1] = ld16_as<kStream>(kt + (gi + 8 * s2) * kRowBytes + (qa + 8) * 16);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) vB[r] = ld16_as<kStream>(vt + r * 1024 + lane * 16);
      return valid;
    };

    // Attention over the page whose tiles are in kA / vB (`valid` rows).
    auto process = [&](int sp, int valid, const uint4 (&kA)[2][2], const uint4 (&vB)[4]) {
      // A skipped page (valid <= 0: skipped, or a slot past the wave's last
      // page) only retires its loads: the wait leaves the kStages-1 newer
      // pages' loads in flight, as the compute path would, so every path
      // through the loop carries the same loads and the loop head never
      // drains the memory queue.
      if (valid <= 0) {
        __builtin_amdgcn_s_waitcnt(kSkipWait);
        return;
      }

      // ---- logits of rows gi, gi+8 for every head of the group
      float z[2][G];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          uint4 q0, q1;
          if constexpr (kQInLds) {
            q0 = *reinterpret_cast<const uint4*>(q_lds + hh * kRowBytes + qa * 16);
            q1 = *reinterpret_cast<const uint4*>(q_lds + hh * kRowBytes + (qa + 8) * 16);
          } else {
            q0 = qk[hh][0];
            q1 = qk[hh][1];
          }
          float acc = chunk_dot(q0, kA[s2][0], 0.0f, T{});
          acc = chunk_dot(q1, kA[s2][1], acc, T{});
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
      float* pb = pbuf + (sp & 1) * (kPage * G);
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
    // math of one page). kStages register buffers, rotated by an unrolled
    // loop so no data is copied. The loop runs whole rotations and leaves at
    // the bottom once no buffer holds a page (a single exit).
    if (src.empty()) return;
    uint4 kA[kStages][2][2], vB[kStages][4];
    int vld[kStages];
    // (the scheduling barriers keep the pages' loads in issue order, which
    // the in-order memory counter needs for the waits below to be partial)
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) {
      vld[s] = issue(kA[s], vB[s]);
      __builtin_amdgcn_sched_barrier(0);
    }
    int sp = 0;
    while (true) {
#pragma unroll
      for (int r = 0; r < kStages; ++r) {
        vld[(r + kStages - 1) % kStages] =
            issue(kA[(r + kStages - 1) % kStages], vB[(r + kStages - 1) % kStages]);
        process(sp, vld[r], kA[r], vB[r]);
        ++sp;
      }
      bool more = false;
#pragma unroll
      for (int s = 0; s < kStages - 1; ++s) more |= vld[s] >= 0;
      if (!more) break;
    }
  }

  // Wave epilogue: afterwards lanes 0..15 hold o[hh][e] summed over the 4 row
  // groups for chunk lane (elements lane*EPC .. +EPC-1), and lanes 0..G-1
  // hold (m, l) of head `lane` in *m_out / *l_out.
  __device__ __forceinline__ void reduce(float* m_out, float* l_out) {
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
    *m_out = m_lane;
    *l_out = lr;
  }
};

// Page source: the wave's pages held one per lane (lane i: physical slot
// and valid-token count of the wave's i-th page), npw <= 64 of them.
struct LanePages {
  int my_p, my_valid, npw;
  int i = 0;
  __device__ __forceinline__ bool empty() const { return npw <= 0; }
  __device__ __forceinline__ void next(int* p, int* v) {
    *p = __builtin_amdgcn_readlane(my_p, min(i, npw - 1));
    *v = i < npw ? __builtin_amdgcn_readlane(my_valid, min(i, 63)) : -1;
    ++i;
  }
};

}  // namespace qsa
