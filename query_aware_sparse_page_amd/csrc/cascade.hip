// Step 5 (prefix half): the shared prefix of a cascade (Quail page, join
// attention: every suffix query attends the shared anchor once; the partial
// result is merged with the suffix's by log-sum-exp rescaling).
//
// With B sequences sharing the prefix, the queries of one KV head form a
// dense [R = B*g, D] block and the prefix a [D, prefix_len] block: a real
// contraction, so it runs on the matrix cores (v_mfma_f32_16x16x32_bf16,
// fp32 accumulate). Flash-attention style: a workgroup owns 128 query rows
// (32 per wave, two 16-column tiles) and one split of the prefix keys; it
// walks the split in blocks of 32 keys (two pages), keeping an online
// softmax per query.
//
// Orientation: the wave computes S^T = K . Q^T (rows = keys, cols = queries),
// so the probabilities come out of the MFMA already in the layout of the B
// operand of O^T = V^T . P^T and never leave registers. K blocks are staged
// row-major in LDS (padded rows: conflict-free operand reads), V blocks
// transposed; both double-buffered, with the global loads of the next
// kDepth blocks in flight in registers while a block is computed.
//
// MFMA 16x16x32 operand layouts (lane l, g = l/16):
//   A[i][k]: i = l%16, k = 8g .. 8g+7     B[k][j]: j = l%16, k = 8g .. 8g+7
//   C[i][j]: j = l%16, i = 4g .. 4g+3
// The k-slots 8g+e of a 32-key block hold keys 4g+e (e < 4) and 16+4g+e-4
// (e >= 4): exactly the rows the two 16-key S^T tiles leave in lane l.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kCD = 128;            // head dim
constexpr int kQT = 2;              // 16-query tiles per wave
constexpr int kRowsPerWG = 4 * 16 * kQT;
constexpr int kKeyBlock = 32;       // keys per block
constexpr int kDepth = 2;           // blocks whose global loads are in flight
constexpr int kKPitch = kCD + 8;    // LDS row of K in bf16 (256 B + 16 B pad)
constexpr int kVtRow = 36;          // LDS row of V^T in bf16 (32 keys + pad)
constexpr int kMaxSplitPages = 80;  // pages of one split (the host keeps splits <= 1056 tokens)
constexpr float kCasTau = 8.0f;

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

struct CascadeShared {
  alignas(16) uint16_t k[2][kKeyBlock][kKPitch];
  alignas(16) uint16_t vt[2][kCD][kVtRow];
  int pg[kMaxSplitPages];
};

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) cascade_prefix_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, int num_phys, int B, int Hkv, int G,
    const int* __restrict__ prefix_pages, int prefix_len, int split_tokens, int n_splits,
    float scale_log2, float* __restrict__ pre_o, float* __restrict__ pre_ml) {
  __shared__ CascadeShared sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4;   // lane group 0..3
  const int c16 = lane & 15;  // lane within group
  // Workgroup -> (row tile, KV head, split): the row tiles of one (head,
  // split) are kHS apart, so (with workgroups dealt round-robin over the 8
  // XCDs and kHS a multiple of 8) they share an XCD and its L2.
  const int kHS = Hkv * n_splits;
  const int rt = blockIdx.x / kHS;
  const int hs = blockIdx.x - rt * kHS;
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

  // the split's physical pages (-1: outside the prefix or out of range)
  for (int i = tid; i < kMaxSplitPages; i += 256) {
    const int pgi = pg0 + i;
    int p = -1;
    if (pgi < n_pre_pages && pgi * kPage < kend) {
      p = prefix_pages[pgi];
      p = (p >= 0 && p < num_phys) ? p : -1;
    }
    sh.pg[i] = p;
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
  __syncthreads();  // page list

  const size_t page_stride = (size_t)Hkv * kTileBytes;
  const char* kbase = reinterpret_cast<const char*>(k_pool) + (size_t)h * kTileBytes;
  const char* vbase = reinterpret_cast<const char*>(v_pool) + (size_t)h * kTileBytes;

  // Staging of block bi: thread -> K (key = idx/16, chunk = idx%16) and
  // V (key = idx%32, chunk = idx/32) for idx = tid, tid + 256. Blocks past
  // the split load its last block again (cache hits); keys past the split,
  // or on pages out of range, are staged as zeros.
  const int last_blk = nblk > 0 ? nblk - 1 : 0;
  auto key_src = [&](int bi, int key, const char* base) -> const char* {
    const int gk = kbeg + min(bi, last_blk) * kKeyBlock + key;
    const int p = sh.pg[min(gk, kend > 0 ? kend - 1 : 0) / kPage - pg0];
    return base + (size_t)(p >= 0 ? p : 0) * page_stride + (gk & 15) * kRowBytes;
  };
  auto issue = [&](int bi, uint4 (&kr)[2], uint4 (&vr)[2]) {
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int idx = tid + 256 * rep;
      kr[rep] = ld16(key_src(bi, idx >> 4, kbase) + (idx & 15) * 16);
      vr[rep] = ld16(key_src(bi, idx & 31, vbase) + (idx >> 5) * 16);
    }
  };
  auto stage = [&](int bi, int buf, const uint4 (&kr)[2], const uint4 (&vr)[2]) {
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int idx = tid + 256 * rep;
      {
        const int key = idx >> 4;
        const int gk = kbeg + bi * kKeyBlock + key;
        const bool ok = bi < nblk && gk < kend && sh.pg[gk / kPage - pg0] >= 0;
        *reinterpret_cast<uint4*>(&sh.k[buf][key][(idx & 15) * 8]) = ok ? kr[rep] : make_uint4(0, 0, 0, 0);
      }
      {
        const int key = idx & 31;
        const int chunk = idx >> 5;
        const int gk = kbeg + bi * kKeyBlock + key;
        const bool ok = bi < nblk && gk < kend && sh.pg[gk / kPage - pg0] >= 0;
        const uint4 v = ok ? vr[rep] : make_uint4(0, 0, 0, 0);
        const uint32_t* w = reinterpret_cast<const uint32_t*>(&v);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sh.vt[buf][chunk * 8 + 2 * e][key] = (uint16_t)(w[e] & 0xFFFFu);
          sh.vt[buf][chunk * 8 + 2 * e + 1][key] = (uint16_t)(w[e] >> 16);
        }
      }
    }
  };

  f32x4_t oacc[kQT][8];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[qt][dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run[kQT], l_part[kQT];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    m_run[qt] = -__builtin_inff();
    l_part[qt] = 0.0f;
  }

  // Attention over the block staged in LDS buffer buf (keys from kb).
  auto compute = [&](int kb, int buf) {
    // ---- S^T tiles: keys kb + 16 kt + c16 (A rows), dims 8g + 32 ks
    f32x4_t sacc[2][kQT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) sacc[kt][qt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(&sh.k[buf][16 * kt + c16][8 * g4 + 32 * ks]);
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt) sacc[kt][qt] = mfma16(a, qb[qt][ks], sacc[kt][qt]);
      }
    // ---- online softmax over this block, per query column c16 of each tile
    uint4 pb[kQT];
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      float s[8];
      float mx = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int gk = kb + 16 * kt + 4 * g4 + i;
          const float v = gk < kend ? sacc[kt][qt][i] * scale_log2 : -__builtin_inff();
          s[4 * kt + i] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, xshfl(mx, 16));
      mx = fmaxf(mx, xshfl(mx, 32));
      if (__builtin_amdgcn_ballot_w64(mx > m_run[qt] + kCasTau) != 0) {
        const float mn = fmaxf(m_run[qt], mx);
        const float al = (mn == -__builtin_inff()) ? 1.0f : fast_exp2(m_run[qt] - mn);
        m_run[qt] = mn;
        l_part[qt] *= al;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[qt][dt] *= al;
      }
      // k-slot 8g+e holds s[e]: key 4g+e of tile 0 (e < 4), of tile 1 (e >= 4)
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = (m_run[qt] == -__builtin_inff()) ? 0.0f : fast_exp2(s[2 * e] - m_run[qt]);
        const float p1 = (m_run[qt] == -__builtin_inff()) ? 0.0f : fast_exp2(s[2 * e + 1] - m_run[qt]);
        const uint32_t b0 = bf16_rne(p0), b1 = bf16_rne(p1);
        // the denominator sums the same bf16-rounded weights the MFMA uses
        l_part[qt] += __uint_as_float(b0 << 16) + __uint_as_float(b1 << 16);
        pk[e] = b0 | (b1 << 16);
      }
      pb[qt] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    }
    // ---- O^T += V^T . P^T : A rows = dims 16 dt + c16, k-slots as above
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint16_t* vrow = &sh.vt[buf][16 * dt + c16][0];
      const uint2 lo = *reinterpret_cast<const uint2*>(vrow + 4 * g4);
      const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16 + 4 * g4);
      const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) oacc[qt][dt] = mfma16(a, pb[qt], oacc[qt][dt]);
    }
  };

  // ---- pipeline: loads of blocks bi+1 .. bi+kDepth in flight while block
  // bi is computed; buffers rotate through an unrolled loop (no copies)
  if (nblk > 0) {
    uint4 kr[kDepth][2], vr[kDepth][2];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      issue(d, kr[d], vr[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
    stage(0, 0, kr[0], vr[0]);
    __syncthreads();
    const int rounds = (nblk + kDepth - 1) / kDepth;
    int bi = 0;
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
      for (int r = 0; r < kDepth; ++r) {
        // slot r held block bi, staged in the previous step: reload it with bi + kDepth
        issue(bi + kDepth, kr[r], vr[r]);
        __builtin_amdgcn_sched_barrier(0);
        compute(kbeg + bi * kKeyBlock, bi & 1);
        stage(bi + 1, (bi + 1) & 1, kr[(r + 1) % kDepth], vr[(r + 1) % kDepth]);
        __syncthreads();
        ++bi;
      }
    }
  }

  // ---- partial (o relative to m_run, m_run, l) per query row
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    float l = l_part[qt];
    l += xshfl(l, 16);
    l += xshfl(l, 32);
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

}  // namespace

hipError_t launch_cascade_prefix(const LaunchCommon& c, const void* q, const int* prefix_pages,
                                 int prefix_len, int n_splits, float scale_log2, Partials prefix,
                                 hipStream_t stream) {
  if (!c.bf16 || c.D != kCD) return hipErrorInvalidValue;
  const int R = c.B * c.G;
  int split_tokens = (prefix_len + n_splits - 1) / n_splits;
  split_tokens = (split_tokens + kKeyBlock - 1) / kKeyBlock * kKeyBlock;
  if (split_tokens / kPage + 1 > kMaxSplitPages) return hipErrorInvalidValue;
  const int row_tiles = (R + kRowsPerWG - 1) / kRowsPerWG;
  hipLaunchKernelGGL(cascade_prefix_kernel, dim3(row_tiles * c.Hkv * n_splits), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(c.k_pool),
                     static_cast<const uint16_t*>(c.v_pool), c.num_phys, c.B, c.Hkv, c.G,
                     prefix_pages, prefix_len, split_tokens, n_splits, scale_log2, prefix.o,
                     prefix.ml);
  return hipGetLastError();
}

}  // namespace qsa
