// One wave's share of paged decode attention on the matrix cores (bf16 K/V,
// head_dim 128, the up to 16 query heads of one GQA group). Same contract as
// WaveAttn (decode_wave.h): the wave owns a list of pages and every head of
// its group, each K/V tile is read from HBM once for all g heads, and the
// online softmax keeps (max, sum, unnormalised output) per head (CS336 page
// §9.2). Per page the two products are small dense contractions - logits
// [16 keys x 128] x [128 x g] and output [128 x 16 keys] x [16 keys x g] -
// which v_mfma does in a few instructions where the vector ALU needs
// hundreds, so the wave's time goes to memory instead of arithmetic.
//
// MFMA operand layouts (lane l, grp = l/16, c16 = l%16):
//   16x16x32: A[i][k]: i = c16, k = 8 grp .. +7   B[k][j]: j = c16, k = 8 grp .. +7
//   16x16x16: A[i][k]: i = c16, k = 4 grp .. +3   B[k][j]: j = c16, k = 4 grp .. +3
//   both:     C[i][j]: j = c16, i = 4 grp .. +3
// Orientation: S^T = K . Q^T (rows = the page's 16 keys, columns = heads),
// so lane l ends with the logits of keys 4 grp .. +3 for head c16 - the
// k-slots of the B operand of O^T = V^T . P^T (16x16x16, one page per
// contraction): the probabilities never leave the lane. V^T comes from the
// V tile staged in LDS, read transposed with ds_read_b64_tr_b16 (a 16-lane
// group's lane s reads row key0 + s/4, columns d0 + 4 (s%4) .. +3, and lane
// s then holds V[key0 .. key0+3][d0 + s]).
//
// The probabilities are split into bf16 high and low parts (p = hi + lo to
// about 2^-17) and both go through the matrix cores, so the output carries
// no bf16 rounding of the weights; the softmax sum adds the fp32 p.
#pragma once

#include "decode_wave.h"

namespace qsa {

typedef __bf16 mf_bf16x8_t __attribute__((ext_vector_type(8)));
typedef short mf_i16x4_t __attribute__((ext_vector_type(4)));
typedef float mf_f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ mf_f32x4_t mfma_k32(const uint4& a, const uint4& b, mf_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mf_bf16x8_t, a),
                                                 __builtin_bit_cast(mf_bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ mf_f32x4_t mfma_k16(const uint2& a, const uint2& b, mf_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(mf_i16x4_t, a),
                                                   __builtin_bit_cast(mf_i16x4_t, b), c, 0, 0, 0);
}
typedef __bf16 mf_bf16x2_t __attribute__((ext_vector_type(2)));

// The default segment hook: a page list within one (b, h) row.
struct NoSegments {
  static constexpr bool kActive = false;
  template <class WA>
  __device__ __forceinline__ void operator()(WA&, int) const {}
};

// Two page buffers (one page in flight while one is computed) measured
// faster than three or four. kStreamArg: the K/V tile loads carry the
// non-temporal hint (ld16_stream).
template <int G, int kStagesArg = 2, bool kStreamArg = false>
struct WaveAttnMfma {
  static_assert(G >= 1 && G <= 16, "one 16-column tile of heads");
  static constexpr int D = 128;
  static constexpr int kStages = kStagesArg;     // page buffers per wave
  static constexpr bool kStream = kStreamArg;
  static constexpr int kVPitch = 144;            // LDS row of the V tile in bf16 (256 B + 32 B pad)
  static constexpr int kVTileBytes = kPage * kVPitch * 2;
  static constexpr int kLdsBytes = 2 * kVTileBytes;  // per wave: double-buffered V tile
  // s_waitcnt immediate (gfx9 layout) that leaves the loads of kStages-1
  // pages (8 vector loads each) outstanding (see WaveAttn).
  static constexpr int kSkipVm = (kStages - 1) * 8;
  static constexpr int kSkipWait = (kSkipVm & 15) | ((kSkipVm >> 4) << 14) | 0x0F70;
  static_assert(kSkipVm < 64, "vmcnt holds at most 63");

  uint4 qb[4];           // B operand of S^T: Q^T[dims 8 grp + 32 ks ..][head c16] (zero past G)
  mf_f32x4_t oacc[8];    // O^T tiles: dims 16 dt + 4 grp + i, head c16
  float m_run;           // head c16: reference max, log2 units
  float l_run;           // this lane's share of head c16's sum

  // q_rows: the group's G query rows (256 B each) in global memory.
  __device__ __forceinline__ void init(const char* q_rows, int lane) {
    const int c16 = lane & 15;
    const int grp = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qb[ks] = c16 < G ? ld16(q_rows + c16 * kRowBytes + (8 * grp + 32 * ks) * 2)
                       : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt] = mf_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m_run = -__builtin_inff();
    l_run = 0.0f;
  }

  // A new (b, h) row: its query rows (B operand layout, as init loads them)
  // and an empty state.
  __device__ __forceinline__ void restart(const uint4 (&q)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[ks] = q[ks];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt] = mf_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m_run = -__builtin_inff();
    l_run = 0.0f;
  }

  // Pages as in WaveAttn::run. vlds: this wave's kLdsBytes of LDS. A source
  // whose page list spans several (b, h) rows reports, with each page, a
  // nonzero segment word when the page is the last of its row's run
  // (src.seg()); after that page is processed, hook(*this, word) takes the
  // row's result and resets the state for the next row.
  template <class Src, class Hook = NoSegments>
  __device__ __forceinline__ void run(Src& src, const char* kbase, const char* vbase,
                                      size_t page_stride, float scale_log2, char* vlds, int lane,
                                      Hook hook = Hook{}) {
    const int c16 = lane & 15;
    const int grp = lane >> 4;

    // K tile in the A layout of S^T (lane: key c16, dims 8 grp + 32 ks),
    // V tile linear (lane: chunk c16 of rows grp + 4 r). Branch-free.
    auto issue = [&](uint4 (&kA)[4], uint4 (&vB)[4], int& segw) -> int {
      int p, valid;
      src.next(&p, &valid);
      if constexpr (Hook::kActive)
        segw = src.seg();
      else
        segw = 0;
      const char* kt = kbase + (size_t)p * page_stride;
      const char* vt = vbase + (size_t)p * page_stride;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kA[ks] = ld16_as<kStream>(kt + c16 * kRowBytes + ks * 64 + grp * 16);
#pragma unroll
      for (int r = 0; r < 4; ++r) vB[r] = ld16_as<kStream>(vt + r * 1024 + lane * 16);
      return valid;
    };

    auto process = [&](int sp, int valid, const uint4 (&kA)[4], const uint4 (&vB)[4]) {
      if (valid <= 0) {  // skipped page: retire its loads only (see WaveAttn)
        __builtin_amdgcn_s_waitcnt(kSkipWait);
        return;
      }
      // ---- V tile to LDS; rows past the page's valid tokens become zeros
      // (they may hold anything, and 0 * NaN would poison the product)
      char* vt = vlds + (sp & 1) * kVTileBytes;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * r + grp;
        const uint4 v = row < valid ? vB[r] : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(vt + row * (kVPitch * 2) + c16 * 16) = v;
      }

      // ---- S^T = K . Q^T: lane holds keys 4 grp + i of head c16
      // (two accumulation chains, summed at the end, halve the dependent
      // latency of the four products)
      mf_f32x4_t s0 = mf_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, s1 = s0;
      s0 = mfma_k32(kA[0], qb[0], s0);
      s1 = mfma_k32(kA[1], qb[1], s1);
      s0 = mfma_k32(kA[2], qb[2], s0);
      s1 = mfma_k32(kA[3], qb[3], s1);
      const mf_f32x4_t s = s0 + s1;
      float z[4];
      float mx = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i] = (4 * grp + i < valid) ? s[i] * scale_log2 : -__builtin_inff();
        mx = fmaxf(mx, z[i]);
      }
      // ---- lazily moved reference max: the lane's own keys decide whether
      // it must move (the ballot is the cross-lane OR); only then is the
      // head's max reduced over the lane groups (every lane of a head agrees)
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyTau) != 0) {
        mx = fmaxf(mx, xshfl(mx, 16));
        mx = fmaxf(mx, xshfl(mx, 32));
        const float mn = fmaxf(m_run, mx);
        const float alpha = (mn == -__builtin_inff()) ? 1.0f : fast_exp2(m_run - mn);
        m_run = mn;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[dt] *= alpha;
      }
      // ---- probabilities: fp32 into the sum, hi + lo bf16 into the product
      // (m_run is finite here: the wave's first attended page has a valid
      // key in every column, so the reference moved on it; the bf16
      // conversions round to nearest even in hardware)
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = fast_exp2(z[i] - m_run);
        l_run += p[i];
      }
      uint32_t hi[2], lo[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const mf_bf16x2_t h = {(__bf16)p[2 * e], (__bf16)p[2 * e + 1]};
        hi[e] = __builtin_bit_cast(uint32_t, h);
        const mf_bf16x2_t r = {(__bf16)(p[2 * e] - __uint_as_float(hi[e] << 16)),
                               (__bf16)(p[2 * e + 1] - __uint_as_float(hi[e] & 0xFFFF0000u))};
        lo[e] = __builtin_bit_cast(uint32_t, r);
      }
      const uint2 phi = make_uint2(hi[0], hi[1]);
      const uint2 plo = make_uint2(lo[0], lo[1]);
      wave_lds_sync();  // the V tile stores, before the transposing reads
      // ---- O^T += V^T . P^T, dims 16 dt .. +15
      const char* vsrc = vt + (4 * grp + (c16 >> 2)) * (kVPitch * 2) + (c16 & 3) * 8;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        typedef short lds_v4i16 __attribute__((ext_vector_type(4)));
        const lds_v4i16 a4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) lds_v4i16*)(vsrc + dt * 32));
        const uint2 a = __builtin_bit_cast(uint2, a4);
        oacc[dt] = mfma_k16(a, phi, oacc[dt]);
        oacc[dt] = mfma_k16(a, plo, oacc[dt]);
      }
    };

    // Software pipeline as in WaveAttn::run: the loads of the next kStages-1
    // pages are in flight while one page is processed.
    if (src.empty()) return;
    uint4 kA[kStages][4], vB[kStages][4];
    int vld[kStages], segw[kStages];
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) {
      vld[s] = issue(kA[s], vB[s], segw[s]);
      __builtin_amdgcn_sched_barrier(0);
    }
    int sp = 0;
    while (true) {
#pragma unroll
      for (int r = 0; r < kStages; ++r) {
        const int nx = (r + kStages - 1) % kStages;
        vld[nx] = issue(kA[nx], vB[nx], segw[nx]);
        process(sp, vld[r], kA[r], vB[r]);
        if (Hook::kActive && segw[r] != 0) hook(*this, segw[r]);
        ++sp;
      }
      bool more = false;
#pragma unroll
      for (int s = 0; s < kStages - 1; ++s) more |= vld[s] >= 0;
      if (!more) break;
    }
  }

  // Wave epilogue: o[hh][d] (unnormalised, relative to m) and (m, l) of the
  // wave's G heads into o_out [G][D] / ml_out [G][2] (LDS).
  __device__ __forceinline__ void store(float* o_out, float* ml_out, int lane) {
    const int c16 = lane & 15;
    const int grp = lane >> 4;
    float l = l_run;
    l += xshfl(l, 16);
    l += xshfl(l, 32);
    if (c16 < G) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<float4*>(o_out + c16 * D + 16 * dt + 4 * grp) =
            make_float4(oacc[dt][0], oacc[dt][1], oacc[dt][2], oacc[dt][3]);
      if (grp == 0) {
        ml_out[c16 * 2 + 0] = m_run;
        ml_out[c16 * 2 + 1] = l;
      }
    }
  }
};

}  // namespace qsa
