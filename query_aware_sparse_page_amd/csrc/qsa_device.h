// Device-side helpers shared by the libqsa kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

constexpr int kPage = 16;        // tokens per KV page
constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kRowBytes = 256;   // one key/value/query row: D * sizeof(element)
constexpr int kTileBytes = 4096; // one (page, KV head) tile: 16 rows x 256 B

// Element storage types. bf16 is kept as raw 16-bit patterns; arithmetic
// widens to fp32 (exact) or uses the bf16 dot instructions.
struct bf16s {
  uint16_t bits;
};

template <typename T>
struct Elem;
template <>
struct Elem<bf16s> {
  static constexpr int kPerChunk = 8;  // elements per 16-byte chunk
};
template <>
struct Elem<float> {
  static constexpr int kPerChunk = 4;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
// The same load with the non-temporal hint (the instruction's nt bit), for
// bytes a launch reads once. Taken where it measured faster: the metadata
// build's key tiles (c4-shaped build 0.478 -> 0.446 ms), the scoring
// kernel's record stream and the split/stream decode kernels' K/V tiles (a
// dense 64-sequence step 0.874 -> 0.795 ms). The fused and short-row kernels
// keep plain loads: there the hint raised the HBM bytes fetched by a quarter.
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}
template <bool kStream>
__device__ __forceinline__ uint4 ld16_as(const void* p) {
  if constexpr (kStream)
    return ld16_stream(p);
  else
    return ld16(p);
}
__device__ __forceinline__ void st16(void* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

// bf16 pair packed in a dword -> fp32 (exact).
__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// acc + a.lo*b.lo + a.hi*b.hi on bf16 pairs, fp32 accumulate (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Dot product of one 16-byte chunk of q with one 16-byte chunk of k.
__device__ __forceinline__ float chunk_dot(const uint4& q, const uint4& k, float acc, bf16s) {
  acc = dot2_bf16(q.x, k.x, acc);
  acc = dot2_bf16(q.y, k.y, acc);
  acc = dot2_bf16(q.z, k.z, acc);
  acc = dot2_bf16(q.w, k.w, acc);
  return acc;
}
__device__ __forceinline__ float chunk_dot(const uint4& q, const uint4& k, float acc, float) {
  acc = __builtin_fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
  acc = __builtin_fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
  acc = __builtin_fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
  acc = __builtin_fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  return acc;
}

// Unpack one 16-byte chunk to fp32.
__device__ __forceinline__ void chunk_unpack(const uint4& c, float* f, bf16s) {
  f[0] = bf_lo(c.x); f[1] = bf_hi(c.x);
  f[2] = bf_lo(c.y); f[3] = bf_hi(c.y);
  f[4] = bf_lo(c.z); f[5] = bf_hi(c.z);
  f[6] = bf_lo(c.w); f[7] = bf_hi(c.w);
}
__device__ __forceinline__ void chunk_unpack(const uint4& c, float* f, float) {
  f[0] = __uint_as_float(c.x); f[1] = __uint_as_float(c.y);
  f[2] = __uint_as_float(c.z); f[3] = __uint_as_float(c.w);
}

// Sign split of a query chunk: neg keeps the negative-signed elements (others
// +0), pos the rest. q.neg . m + q.pos . M equals sum_i q_i (q_i > 0 ? M_i : m_i)
// (a zero q_i contributes zero either way).
__device__ __forceinline__ void chunk_sign_split(const uint4& q, uint4& neg, uint4& pos, bf16s) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&q);
  uint32_t* n = reinterpret_cast<uint32_t*>(&neg);
  uint32_t* p = reinterpret_cast<uint32_t*>(&pos);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // per 16-bit half: all-ones mask where the sign bit is set
    uint32_t s = (w[e] >> 15) & 0x00010001u;
    uint32_t mask = s * 0xFFFFu;
    n[e] = w[e] & mask;
    p[e] = w[e] & ~mask;
  }
}
__device__ __forceinline__ void chunk_sign_split(const uint4& q, uint4& neg, uint4& pos, float) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&q);
  uint32_t* n = reinterpret_cast<uint32_t*>(&neg);
  uint32_t* p = reinterpret_cast<uint32_t*>(&pos);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t mask = (uint32_t)((int32_t)w[e] >> 31);
    n[e] = w[e] & mask;
    p[e] = w[e] & ~mask;
  }
}

// ---- order-preserving integer keys (IEEE total order, -0 < +0) ----------
// bf16 pair: per 16-bit half, flip all bits of negatives, the sign of others.
__device__ __forceinline__ uint32_t bf2_to_key(uint32_t x) {
  uint32_t s = (x >> 15) & 0x00010001u;
  return x ^ (s * 0x7FFFu | 0x80008000u);
}
__device__ __forceinline__ uint32_t key_to_bf2(uint32_t k) {
  uint32_t s = ((~k) >> 15) & 0x00010001u;  // 1 where the value was negative
  return k ^ (s * 0x7FFFu | 0x80008000u);
}
__device__ __forceinline__ uint32_t f32_to_key(uint32_t x) {
  return x ^ ((uint32_t)((int32_t)x >> 31) | 0x80000000u);
}
__device__ __forceinline__ uint32_t key_to_f32(uint32_t k) {
  return k ^ ((uint32_t)((int32_t)(~k) >> 31) | 0x80000000u);
}
__device__ __forceinline__ uint32_t umin2x16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2_t, a),
                                                                 __builtin_bit_cast(u16x2_t, b)));
}
__device__ __forceinline__ uint32_t umax2x16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a),
                                                                 __builtin_bit_cast(u16x2_t, b)));
}

// Order-key operations on one dword of storage (a bf16 pair or one fp32):
// to key, back, and element-wise min / max of keys.
template <typename T>
struct KeyOps;
template <>
struct KeyOps<bf16s> {
  static __device__ __forceinline__ uint32_t key(uint32_t x) { return bf2_to_key(x); }
  static __device__ __forceinline__ uint32_t unkey(uint32_t k) { return key_to_bf2(k); }
  static __device__ __forceinline__ uint32_t vmin(uint32_t a, uint32_t b) { return umin2x16(a, b); }
  static __device__ __forceinline__ uint32_t vmax(uint32_t a, uint32_t b) { return umax2x16(a, b); }
};
template <>
struct KeyOps<float> {
  static __device__ __forceinline__ uint32_t key(uint32_t x) { return f32_to_key(x); }
  static __device__ __forceinline__ uint32_t unkey(uint32_t k) { return key_to_f32(k); }
  static __device__ __forceinline__ uint32_t vmin(uint32_t a, uint32_t b) { return a < b ? a : b; }
  static __device__ __forceinline__ uint32_t vmax(uint32_t a, uint32_t b) { return a > b ? a : b; }
};

// Score -> ascending uint32 key; -0 is folded onto +0 so equal values tie.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = (s == 0.0f) ? 0u : __float_as_uint(s);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// ---- DPP lane exchange (wave64, gfx9 DPP controls) ----------------------
enum : int {
  kDppQuadXor1 = 0xB1,       // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,       // quad_perm [2,3,0,1]
  kDppRowHalfMirror = 0x141, // lane i <-> 7-i within each 8-lane half row
  kDppRowMirror = 0x140,     // lane i <-> 15-i within each 16-lane row
};

template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, true));
}

// Sum over aligned groups of 8 lanes; every lane of the group gets the total.
__device__ __forceinline__ float sum8(float v) {
  v += dpp_mov<kDppQuadXor1>(v);
  v += dpp_mov<kDppQuadXor2>(v);
  v += dpp_mov<kDppRowHalfMirror>(v);
  return v;
}
// Sum over aligned groups of 16 lanes (one DPP row); every lane gets it.
__device__ __forceinline__ float sum16(float v) {
  v = sum8(v);
  v += dpp_mov<kDppRowMirror>(v);
  return v;
}

// Cross-lane xor exchange through the LDS crossbar (no LDS allocation).
__device__ __forceinline__ float xshfl(float v, int mask) {
  int lane = __lane_id();
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __builtin_bit_cast(int, v)));
}
__device__ __forceinline__ uint32_t xshfl_u(uint32_t v, int mask) {
  int lane = __lane_id();
  return (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, (int)v);
}

__device__ __forceinline__ float readlane_f_(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// ---- wave64 scans / reductions on DPP (no LDS crossbar) ----------------
template <int kCtrl, int kRowMask = 0xF, int kBankMask = 0xF>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  // lanes whose source is outside the row (or not enabled) read 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, kBankMask, true);
}

// Inclusive prefix sum over the 64 lanes: Hillis-Steele inside each 16-lane
// row (row_shr 1, 2, 4, 8), then row_bcast:15 / row_bcast:31 carry the row
// totals into the following rows.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t v) {
  v += dpp_u<0x111>(v);  // row_shr:1
  v += dpp_u<0x112>(v);  // row_shr:2
  v += dpp_u<0x114>(v);  // row_shr:4
  v += dpp_u<0x118>(v);  // row_shr:8
  v += dpp_u<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_u<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Exclusive prefix sum over the workgroup (thread order); *total gets the
// sum. Contains barriers: every thread must call it.
template <int kWaves>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t incl = wave_scan_incl(v);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t t = wsum[w];
    before += (w < wave) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + incl - v;
}

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_full_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kCtrl, 0xF, 0xF, true);
}
// Minimum / maximum over the 64 lanes, returned in every lane (uniform).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_full_u<kDppQuadXor1>(v));
  v = min(v, dpp_full_u<kDppQuadXor2>(v));
  v = min(v, dpp_full_u<kDppRowHalfMirror>(v));
  v = min(v, dpp_full_u<kDppRowMirror>(v));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return min(min(a, b), min(c, d));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_full_u<kDppQuadXor1>(v));
  v = max(v, dpp_full_u<kDppQuadXor2>(v));
  v = max(v, dpp_full_u<kDppRowHalfMirror>(v));
  v = max(v, dpp_full_u<kDppRowMirror>(v));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}
// Sum / max of floats over the 64 lanes, returned in every lane.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v = sum16(v);
  return readlane_f_(v, 0) + readlane_f_(v, 16) + readlane_f_(v, 32) + readlane_f_(v, 48);
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// The rows of one (page, KV head) tile (16 rows x 256 B) as the tile
// reductions below take them: four 16-byte loads per lane, each reading 1 KiB
// contiguous; lane l holds chunk l%16 of rows {l/16, 4 + l/16, 8 + l/16,
// 12 + l/16}. kStream: the loads carry the non-temporal hint (ld16_stream).
template <bool kStream = false>
__device__ __forceinline__ void tile_load_rows(const char* tile, int lane, uint4 (&rows)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) rows[r] = ld16_as<kStream>(tile + r * 1024 + lane * 16);
}

// Element-wise min and max of the first `valid` key rows of one tile (rows
// as tile_load_rows leaves them), exact (order keys, -0 < +0). After the
// in-lane reduction lanes l, l^16, l^32, l^48 combine, so on return every
// lane holds the tile's min / max of chunk l%16.
template <typename T>
__device__ __forceinline__ void tile_minmax_rows(const uint4 (&rows)[4], int valid, int lane, uint4& vmn,
                                                 uint4& vmx) {
  using Ops = KeyOps<T>;
  uint32_t mn[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  uint32_t mx[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (4 * r + (lane >> 4) < valid) {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(&rows[r]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kk = Ops::key(w[e]);
        mn[e] = Ops::vmin(mn[e], kk);
        mx[e] = Ops::vmax(mx[e], kk);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    mn[e] = Ops::vmin(mn[e], xshfl_u(mn[e], 16));
    mx[e] = Ops::vmax(mx[e], xshfl_u(mx[e], 16));
    mn[e] = Ops::vmin(mn[e], xshfl_u(mn[e], 32));
    mx[e] = Ops::vmax(mx[e], xshfl_u(mx[e], 32));
  }
  vmn = make_uint4(Ops::unkey(mn[0]), Ops::unkey(mn[1]), Ops::unkey(mn[2]), Ops::unkey(mn[3]));
  vmx = make_uint4(Ops::unkey(mx[0]), Ops::unkey(mx[1]), Ops::unkey(mx[2]), Ops::unkey(mx[3]));
}

// tile_minmax_rows of the tile at `tile`.
template <typename T, bool kStream = false>
__device__ __forceinline__ void tile_minmax(const char* tile, int valid, int lane, uint4& vmn,
                                            uint4& vmx) {
  uint4 rows[4];
  tile_load_rows<kStream>(tile, lane, rows);
  tile_minmax_rows<T>(rows, valid, lane, vmn, vmx);
}

// fp64 -> nearest bf16 (ties to even), as the bf16 bit pattern: the value is
// rounded to 8 significant bits inside the fp64 encoding (a carry moves into
// the exponent by itself), after which the conversion to fp32 is exact.
// Values of magnitude below 2^-126 are not handled (bf16 subnormals).
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double x) {
  unsigned long long b = (unsigned long long)__double_as_longlong(x);
  b += 0x00000FFFFFFFFFFFull + ((b >> 45) & 1ull);
  b &= ~0x00001FFFFFFFFFFFull;
  return __float_as_uint((float)__longlong_as_double((long long)b)) >> 16;
}

__device__ __forceinline__ double xshfl_d(double v, int mask) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = xshfl_u((uint32_t)b, mask);
  const uint32_t hi = xshfl_u((uint32_t)(b >> 32), mask);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Mean of the valid rows of one tile (rows as tile_load_rows leaves them),
// element-wise, rounded once to the element type: the row sums are taken in
// fp64 (the sum of up to 16 bf16 values is exact there unless their
// magnitudes span more than about 2^41), divided by `valid` in fp64
// (correctly rounded), then rounded to bf16 (ties to even) or converted to
// fp32. On return every lane holds the mean of chunk lane % 16.
template <typename T>
__device__ __forceinline__ uint4 tile_mean_rows(const uint4 (&rows)[4], int valid, int lane) {
  constexpr int E = Elem<T>::kPerChunk;
  double acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (4 * r + (lane >> 4) < valid) {
      float f[E];
      chunk_unpack(rows[r], f, T{});
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += (double)f[e];
    }
  }
  const double count = (double)valid;
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    acc[e] += xshfl_d(acc[e], 16);
    acc[e] += xshfl_d(acc[e], 32);
    acc[e] = acc[e] / count;
  }
  if constexpr (E == 8) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = f64_to_bf16_rne(acc[2 * e]) | (f64_to_bf16_rne(acc[2 * e + 1]) << 16);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = __float_as_uint((float)acc[e]);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// tile_mean_rows of the tile at `tile`.
template <typename T, bool kStream = false>
__device__ __forceinline__ uint4 tile_mean(const char* tile, int valid, int lane) {
  uint4 rows[4];
  tile_load_rows<kStream>(tile, lane, rows);
  return tile_mean_rows<T>(rows, valid, lane);
}

// Orders this wave's LDS accesses before and after the call point (all lanes
// of one wave; no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace qsa
