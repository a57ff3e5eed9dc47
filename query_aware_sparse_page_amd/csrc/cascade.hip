// Step 5 (prefix half): the shared prefix of a cascade (Quail page, join
// attention: every suffix query attends the shared anchor once; the partial
// result is merged with the suffix's by log-sum-exp rescaling).
//
// With B sequences sharing the prefix, the queries of one KV head form a
// dense [R = B*g, D] block and the prefix a [D, prefix_len] block: a real
// contraction, so it runs on the matrix cores (v_mfma_f32_16x16x32_bf16,
// fp32 accumulate). Flash-attention style: a workgroup owns 64 query rows
// (16 per wave) and one split of the prefix keys; it walks the split in
// blocks of 32 keys (two pages), keeping an online softmax per query.
//
// Orientation: the wave computes S^T = K . Q^T (rows = keys, cols = queries),
// so the probabilities come out of the MFMA already in the layout of the B
// operand of O^T = V^T . P^T and never leave registers. V^T is the A operand;
// the workgroup stages each V block transposed in LDS (double-buffered).
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

constexpr int kCD = 128;           // head dim
constexpr int kRowsPerWG = 64;     // query rows per workgroup
constexpr int kKeyBlock = 32;      // keys per step
constexpr int kVtRow = 36;         // LDS row of V^T in bf16 elements (32 keys + pad)
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

__global__ void __launch_bounds__(256) cascade_prefix_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, int num_phys, int B, int Hkv, int G,
    const int* __restrict__ prefix_pages, int prefix_len, int split_tokens, float scale_log2,
    float* __restrict__ pre_o, float* __restrict__ pre_ml) {
  __shared__ uint16_t vt[2][kCD][kVtRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4;   // lane group 0..3
  const int c16 = lane & 15;  // lane within group
  const int h = blockIdx.z;
  const int split = blockIdx.y;
  const int n_splits = gridDim.y;
  const int R = B * G;
  const int Hq = Hkv * G;
  const int r = blockIdx.x * kRowsPerWG + wave * 16 + c16;  // this lane's query row
  const bool row_ok = r < R;

  const int kbeg = split * split_tokens;
  const int kend = min(prefix_len, kbeg + split_tokens);
  const int n_pre_pages = (prefix_len + kPage - 1) / kPage;

  // B operand of S^T: Q^T[dims 8g + 32ks .. +8][query c16]
  uint4 qb[4];
  {
    const int b = row_ok ? r / G : 0;
    const int hh = row_ok ? r - b * G : 0;
    const char* qrow = reinterpret_cast<const char*>(q) + ((size_t)b * Hq + h * G + hh) * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qb[ks] = row_ok ? ld16(qrow + (8 * g4 + 32 * ks) * 2) : make_uint4(0, 0, 0, 0);
  }

  f32x4_t oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -__builtin_inff();
  float l_part = 0.0f;

  const size_t page_stride = (size_t)Hkv * kTileBytes;
  const char* kbase = reinterpret_cast<const char*>(k_pool) + (size_t)h * kTileBytes;
  const char* vbase = reinterpret_cast<const char*>(v_pool) + (size_t)h * kTileBytes;

  int it = 0;
  for (int kb = kbeg; kb < kend; kb += kKeyBlock, ++it) {
    const int buf = it & 1;
    // ---- stage V block transposed: thread -> (key = idx%32, chunk = idx/32)
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int idx = tid + 256 * rep;
      const int key = idx & 31;
      const int chunk = idx >> 5;
      const int gk = kb + key;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (gk < kend) {
        const int pg = gk >> 4;
        const int p = pg < n_pre_pages ? prefix_pages[pg] : -1;
        if (p >= 0 && p < num_phys) v = ld16(vbase + (size_t)p * page_stride + (gk & 15) * kRowBytes + chunk * 16);
      }
      const uint32_t* w = reinterpret_cast<const uint32_t*>(&v);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vt[buf][chunk * 8 + 2 * e][key] = (uint16_t)(w[e] & 0xFFFFu);
        vt[buf][chunk * 8 + 2 * e + 1][key] = (uint16_t)(w[e] >> 16);
      }
    }
    // ---- S^T tiles: keys kb + 16 kt + c16 (A rows), dims 8g + 32 ks
    f32x4_t sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      sacc[kt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      const int gk = kb + 16 * kt + c16;
      const char* krow = nullptr;
      if (gk < kend) {
        const int pg = gk >> 4;
        const int p = pg < n_pre_pages ? prefix_pages[pg] : -1;
        if (p >= 0 && p < num_phys) krow = kbase + (size_t)p * page_stride + (gk & 15) * kRowBytes;
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 a = krow ? ld16(krow + (8 * g4 + 32 * ks) * 2) : make_uint4(0, 0, 0, 0);
        sacc[kt] = mfma16(a, qb[ks], sacc[kt]);
      }
    }
    // ---- online softmax over this block for query column c16
    float s[8];
    float mx = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int gk = kb + 16 * kt + 4 * g4 + i;
        const float v = gk < kend ? sacc[kt][i] * scale_log2 : -__builtin_inff();
        s[4 * kt + i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, xshfl(mx, 16));
    mx = fmaxf(mx, xshfl(mx, 32));
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kCasTau) != 0) {
      const float mn = fmaxf(m_run, mx);
      const float a = (mn == -__builtin_inff()) ? 1.0f : fast_exp2(m_run - mn);
      m_run = mn;
      l_part *= a;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oacc[dt] *= a;
    }
    uint32_t pk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = (m_run == -__builtin_inff()) ? 0.0f : fast_exp2(s[2 * e] - m_run);
      const float p1 = (m_run == -__builtin_inff()) ? 0.0f : fast_exp2(s[2 * e + 1] - m_run);
      const uint32_t b0 = bf16_rne(p0), b1 = bf16_rne(p1);
      // the denominator sums the same bf16-rounded weights the MFMA uses
      l_part += __uint_as_float(b0 << 16) + __uint_as_float(b1 << 16);
      pk[e] = b0 | (b1 << 16);
    }
    const uint4 pb = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    __syncthreads();  // V^T block staged
    // ---- O^T += V^T . P^T : A rows = dims 16 dt + c16, k-slots 8g .. 8g+7
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint16_t* vrow = &vt[buf][16 * dt + c16][0];
      const uint2 lo = *reinterpret_cast<const uint2*>(vrow + 4 * g4);
      const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16 + 4 * g4);
      oacc[dt] = mfma16(make_uint4(lo.x, lo.y, hi.x, hi.y), pb, oacc[dt]);
    }
  }

  // ---- partial (o relative to m_run, m_run, l) for this query row
  float l = l_part;
  l += xshfl(l, 16);
  l += xshfl(l, 32);
  if (row_ok) {
    const size_t pr = ((size_t)h * n_splits + split) * (size_t)R + r;
    float* po = pre_o + pr * kCD;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      float4 v = make_float4(oacc[dt][0], oacc[dt][1], oacc[dt][2], oacc[dt][3]);
      *reinterpret_cast<float4*>(po + 16 * dt + 4 * g4) = v;
    }
    if (g4 == 0) {
      pre_ml[pr * 2 + 0] = m_run;
      pre_ml[pr * 2 + 1] = l;
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
  dim3 grid((R + kRowsPerWG - 1) / kRowsPerWG, n_splits, c.Hkv);
  hipLaunchKernelGGL(cascade_prefix_kernel, grid, dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(c.k_pool),
                     static_cast<const uint16_t*>(c.v_pool), c.num_phys, c.B, c.Hkv, c.G,
                     prefix_pages, prefix_len, split_tokens, scale_log2, prefix.o, prefix.ml);
  return hipGetLastError();
}

}  // namespace qsa
