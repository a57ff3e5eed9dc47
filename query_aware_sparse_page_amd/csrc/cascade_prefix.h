// The cascade prefix's workgroup body (cascade.hip describes the kernel), as
// a function of the workgroup index so that other kernels can run prefix
// workgroups among their own.
#pragma once

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace cascade {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kCD = 128;            // head dim
constexpr int kQT = 2;              // 16-query tiles per wave (180 VGPRs: one workgroup of 8 waves per CU)
// W waves per workgroup: 32 W query rows; a block's 512 16-byte K and V
// chunks are staged kStageReps per thread
template <int W>
struct PrefixCfg {
  static constexpr int kWaves = W;
  static constexpr int kThreads = 64 * W;
  static constexpr int kRowsPerWG = W * 16 * kQT;
  static constexpr int kStageReps = 512 / kThreads;
  static_assert(kStageReps >= 1 && kStageReps * kThreads == 512, "a block is 32 keys x 16 chunks");
};
constexpr int kKeyBlock = 32;       // keys per block
constexpr int kDepth = 2;           // blocks whose global loads are in flight
constexpr int kKPitch = kCD + 16;   // LDS row of K in bf16 (256 B + 32 B pad: no bank conflicts in the A-operand reads)
constexpr int kVPitch = kCD + 16;   // LDS row of V in bf16 (256 B + 32 B pad)
constexpr int kMaxSplitPages = 80;  // pages of one split (the host keeps splits <= 1056 tokens)
constexpr float kCasTau = 8.0f;

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct CascadeShared {
  alignas(16) uint16_t k[2][kKeyBlock][kKPitch];
  alignas(16) uint16_t v[2][kKeyBlock][kVPitch];
};

// One prefix workgroup of W waves: query rows of row tile `block / (Hkv
// n_splits)` against one split of the prefix, partials into pre_o / pre_ml.
template <int W>
__device__ __forceinline__ void prefix_block(
    CascadeShared& sh, int block, int tid, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, int num_phys, int B, int Hkv, int G,
    const int* __restrict__ prefix_pages, int prefix_len, int split_tokens, int n_splits,
    float scale_log2, float* __restrict__ pre_o, float* __restrict__ pre_ml,
    unsigned int* __restrict__ err) {
  constexpr int kThreads = PrefixCfg<W>::kThreads;
  constexpr int kRowsPerWG = PrefixCfg<W>::kRowsPerWG;
  constexpr int kStageReps = PrefixCfg<W>::kStageReps;

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4;   // lane group 0..3
  const int c16 = lane & 15;  // lane within group
  // Workgroup -> (row tile, KV head, split): the row tiles of one (head,
  // split) are kHS apart, so (with workgroups dealt round-robin over the 8
  // XCDs and kHS a multiple of 8) they share an XCD and its L2.
  const int kHS = Hkv * n_splits;
  const int rt = block / kHS;
  const int hs = block - rt * kHS;
  const int h = hs / n_splits;
  const int split = hs - h * n_splits;
  const int R = B * G;
  const int Hq = Hkv * G;
  const int row0 = rt * kRowsPerWG + wave * (16 * kQT);

  const int kbeg = split * split_tokens;
  const int kend = min(prefix_len, kbeg + split_tokens);
  const int nblk = kend > kbeg ? (kend - kbeg + kKeyBlock - 1) / kKeyBlock : 0;
  const int n_pre_pages = (prefix_len + kPage - 1) / kPage;
  const int pg0 = kbeg / kPage;

  // the split's physical pages in registers, entry i in lane i % 64 of
  // pgr[i / 64] (-1: outside the prefix or out of range); a block's page is
  // then one v_readlane away instead of an LDS round trip
  int pgr[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int i = lane + 64 * half;
    const int pgi = pg0 + i;
    int p = -1;
    if (i < kMaxSplitPages && pgi < n_pre_pages && pgi * kPage < kend) {
      p = prefix_pages[pgi];
      if (p < 0 || p >= num_phys) {
        if (rt == 0 && wave == 0) report_bad(err, kErrPhys);
        p = -1;
      }
    }
    pgr[half] = p;
  }

  // B operand of S^T: Q^T[dims 8g + 32ks .. +8][query c16] per query tile
  uint4 qb[kQT][4];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int r = row0 + qt * 16 + c16;
    const bool ok = r < R;
    const int b = ok ? r / G : 0;
    const int hh = ok ? r - b * G : 0;
    const char* qrow = reinterpret_cast<const char*>(q) + ((size_t)b * Hq + h * G + hh) * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qb[qt][ks] = ok ? ld16(qrow + (8 * g4 + 32 * ks) * 2) : make_uint4(0, 0, 0, 0);
  }

  const size_t page_stride = (size_t)Hkv * kTileBytes;
  const char* kbase = reinterpret_cast<const char*>(k_pool) + (size_t)h * kTileBytes;
  const char* vbase = reinterpret_cast<const char*>(v_pool) + (size_t)h * kTileBytes;

  // Staging of block bi: chunk idx = tid + kThreads * rep (rep <
  // kStageReps) is key idx / 16 (page idx / 256 of the block's two, row
  // (idx / 16) % 16), 16-byte chunk idx % 16, of K and of V. Blocks past the
  // split load its last block again (cache hits); keys past the split, or on
  // pages out of range, are staged as zeros.
  const int last_blk = nblk > 0 ? nblk - 1 : 0;
  const int last_pg = kend > kbeg ? (kend - 1) / kPage - pg0 : 0;  // the split's last page (relative)
  const uint32_t toff = ((tid >> 4) & 15) * kRowBytes + (tid & 15) * 16;  // (unsigned: a 32-bit offset to a uniform base)
  // A wave's 64 threads stage rows of one page (idx / 256 is the same for
  // all of them), so the page and its tile address are wave-uniform.
  auto page_of = [&](int bi, int pg) -> int {  // physical page, -1 if out of range
    const int i = min(2 * min(bi, last_blk) + pg, last_pg);  // < kMaxSplitPages <= 128
    return __builtin_amdgcn_readlane(i < 64 ? pgr[0] : pgr[1], i & 63);  // (a select, not a branch)
  };
  // pv: the staged page of each chunk, kept for stage() (-1: staged as zeros)
  auto issue = [&](int bi, uint4 (&kr)[kStageReps], uint4 (&vr)[kStageReps], int (&pv)[kStageReps]) {
#pragma unroll
    for (int rep = 0; rep < kStageReps; ++rep) {
      pv[rep] = page_of(bi, (wave * 64 + kThreads * rep) >> 8);  // = idx >> 8, wave-uniform
      const size_t poff = (size_t)max(pv[rep], 0) * page_stride;
      kr[rep] = ld16(kbase + poff + toff);
      vr[rep] = ld16(vbase + poff + toff);
    }
  };
  // (a block whose keys are all in the split, on a page in range, is staged
  // as loaded behind a wave-uniform test; otherwise the zeros come from a
  // per-lane mask, without a divergent branch)
  auto stage = [&](int bi, int buf, const uint4 (&kr)[kStageReps], const uint4 (&vr)[kStageReps],
                   const int (&pv)[kStageReps]) {
#pragma unroll
    for (int rep = 0; rep < kStageReps; ++rep) {
      const int idx = tid + kThreads * rep;
      const int key = idx >> 4;
      uint4* kd = reinterpret_cast<uint4*>(&sh.k[buf][key][(idx & 15) * 8]);
      uint4* vd = reinterpret_cast<uint4*>(&sh.v[buf][key][(idx & 15) * 8]);
      if (bi < nblk && kbeg + (bi + 1) * kKeyBlock <= kend && pv[rep] >= 0) {
        *kd = kr[rep];
        *vd = vr[rep];
      } else {
        const bool ok = bi < nblk && kbeg + bi * kKeyBlock + key < kend && pv[rep] >= 0;
        const uint32_t m = ok ? 0xFFFFFFFFu : 0u;
        *kd = make_uint4(kr[rep].x & m, kr[rep].y & m, kr[rep].z & m, kr[rep].w & m);
        *vd = make_uint4(vr[rep].x & m, vr[rep].y & m, vr[rep].z & m, vr[rep].w & m);
      }
    }
  };

  f32x4_t oacc[kQT][8];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[qt][dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // Softmax state per query column: the reference max, and this lane's
  // share of the sum of the fp32 weights (its keys 4 g4 .. +3 of each
  // tile; the four lane groups are added at the end).
  float l_run[kQT];
  float m_run[kQT];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    m_run[qt] = -__builtin_inff();
    l_run[qt] = 0.0f;
  }

  // Attention over the block staged in LDS buffer buf (keys from kb);
  // after_s runs once the S^T products are issued.
  auto compute = [&](int kb, int buf, auto&& after_s) {
    // ---- S^T tiles: keys kb + 16 kt + c16 (A rows), dims 8g + 32 ks
    f32x4_t sacc[2][kQT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) sacc[kt][qt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // (ks outermost: the 2 x kQT accumulation chains interleave, so
    // consecutive products never wait on each other's results)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 a[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        a[kt] = *reinterpret_cast<const uint4*>(&sh.k[buf][16 * kt + c16][8 * g4 + 32 * ks]);
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) sacc[kt][qt] = mfma16(a[kt], qb[qt][ks], sacc[kt][qt]);
    }
    after_s();
    // ---- online softmax over this block, per query column c16 of each tile
    // (only a split's last block can hold keys past its end; a key tile on
    // a page out of range, staged as zeros, is masked like keys past the end)
    const int bi = (kb - kbeg) / kKeyBlock;
    const bool bad0 = page_of(bi, 0) < 0;
    const bool bad1 = page_of(bi, 1) < 0;
    const bool full = kb + kKeyBlock <= kend && !bad0 && !bad1;
    uint4 phi[kQT], plo[kQT];  // B operands: P^T (keys 4g .. 4g+3 of tile 0, then of tile 1), hi and lo
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      float s[8];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[4 * kt + i] = sacc[kt][qt][i] * scale_log2;
      if (!full) {  // (workgroup-uniform: the split's last block, or a page out of range)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kb + 16 * kt + 4 * g4 + i >= kend || (kt == 0 ? bad0 : bad1))
              s[4 * kt + i] = -__builtin_inff();
      }
      float mx = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 8; ++i) mx = fmaxf(mx, s[i]);
      // the lane's own keys decide whether the reference must move (the
      // ballot is the cross-lane OR); only then is the column max reduced
      if (__builtin_amdgcn_ballot_w64(mx > m_run[qt] + kCasTau) != 0) {
        mx = fmaxf(mx, xshfl(mx, 16));
        mx = fmaxf(mx, xshfl(mx, 32));
        const float mn = fmaxf(m_run[qt], mx);
        const float al = (mn == -__builtin_inff()) ? 1.0f : fast_exp2(m_run[qt] - mn);
        m_run[qt] = mn;
        l_run[qt] *= al;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[qt][dt] *= al;
      }
      // m_run is finite once a block with a key on a page in range has
      // been seen; before that every logit is -inf and its weight must be 0
      // (exp2(-inf - 0)), not exp2(-inf + inf). The fp32 weights go into the
      // sum; the products take them as bf16 high and low parts (p = hi + lo
      // to about 2^-17; the conversions round to nearest even in hardware),
      // so the output carries no bf16 rounding of the weights.
      const float mref = m_run[qt] == -__builtin_inff() ? 0.0f : m_run[qt];
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float w0 = fast_exp2(s[2 * e] - mref);
        const float w1 = fast_exp2(s[2 * e + 1] - mref);
        l_run[qt] += w0 + w1;
        const bf16x2_t wh = {(__bf16)w0, (__bf16)w1};
        hi[e] = __builtin_bit_cast(uint32_t, wh);
        const bf16x2_t wl = {(__bf16)(w0 - __uint_as_float(hi[e] << 16)),
                             (__bf16)(w1 - __uint_as_float(hi[e] & 0xFFFF0000u))};
        lo[e] = __builtin_bit_cast(uint32_t, wl);
      }
      phi[qt] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      plo[qt] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    // ---- O^T += V^T . P^T, one product per 16 dims over the block's 32
    // keys: A rows = dims 16 dt + c16, keys 4 g4 .. +3 of tile 0 then of
    // tile 1, each read transposed
    typedef short lds_v4i16 __attribute__((ext_vector_type(4)));
    const uint16_t* vsrc = &sh.v[buf][4 * g4 + (c16 >> 2)][4 * (c16 & 3)];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint2 a[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        a[kt] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) lds_v4i16*)(vsrc + 16 * kt * kVPitch + 16 * dt)));
      const uint4 a8 = make_uint4(a[0].x, a[0].y, a[1].x, a[1].y);
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) {
        oacc[qt][dt] = mfma16(a8, phi[qt], oacc[qt][dt]);
        oacc[qt][dt] = mfma16(a8, plo[qt], oacc[qt][dt]);
      }
    }
  };

  // ---- pipeline: loads of blocks bi+1 .. bi+kDepth in flight while block
  // bi is computed; buffers rotate through an unrolled loop (no copies)
  if (nblk > 0) {
    uint4 kr[kDepth][kStageReps], vr[kDepth][kStageReps];
    int pv[kDepth][kStageReps];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      issue(d, kr[d], vr[d], pv[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
    stage(0, 0, kr[0], vr[0], pv[0]);
    __syncthreads();
    const int rounds = (nblk + kDepth - 1) / kDepth;
    int bi = 0;
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
      for (int r = 0; r < kDepth; ++r) {
        // slot r held block bi, staged in the previous step: reload it with bi + kDepth
        issue(bi + kDepth, kr[r], vr[r], pv[r]);
        __builtin_amdgcn_sched_barrier(0);
        // the next block goes to the other LDS buffer (free since the last
        // barrier) while this block's products and softmax run, so its
        // writes have completed by the barrier; its loads were issued a step
        // earlier and have arrived
        compute(kbeg + bi * kKeyBlock, bi & 1, [&]() {
          stage(bi + 1, (bi + 1) & 1, kr[(r + 1) % kDepth], vr[(r + 1) % kDepth], pv[(r + 1) % kDepth]);
        });
        __syncthreads();
        ++bi;
      }
    }
  }

  // ---- partial (o relative to m_run, m_run, l) per query row
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    float l = l_run[qt];
    l += xshfl(l, 16);
    l += xshfl(l, 32);  // the column's sum in every lane group (lanes 0..15 store it)
    const int r = row0 + qt * 16 + c16;
    if (r < R) {
      const size_t pr = ((size_t)h * n_splits + split) * (size_t)R + r;
      float* po = pre_o + pr * kCD;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const float4 v = make_float4(oacc[qt][dt][0], oacc[qt][dt][1], oacc[qt][dt][2], oacc[qt][dt][3]);
        *reinterpret_cast<float4*>(po + 16 * dt + 4 * g4) = v;
      }
      if (g4 == 0) {
        pre_ml[pr * 2 + 0] = m_run[qt];
        pre_ml[pr * 2 + 1] = l;
      }
    }
  }
}

}  // namespace cascade
}  // namespace qsa
