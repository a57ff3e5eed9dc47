// Step 4: split-K flash-decode over the selected pages (TinyServe page, §2.3
// stages 3-4: load only the selected pages' K/V, attention fused with the
// load; flash decoding's split + log-sum-exp merge per the CS336 page §9.2
// and the Quail page's join attention).
//
// Two work splits, chosen by the host's plan:
//  * stream (bf16 groups of 4 or more heads, up to kStreamMaxB sequences):
//    decode_stream_kernel gives every wave an equal, contiguous share of all
//    rows' page lists; below.
//  * units: work unit = (sequence b, KV head h, a chunk of `chunk`
//    consecutive entries of the row's page list), block (h, b, chunk). The unit's workgroup has 4 waves; wave w takes
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
// The matrix-core page loop of the split and stream kernels, whose K/V tiles
// are read with the non-temporal hint (ld16_stream).
template <int G>
using DecodeMfma = WaveAttnMfma<G, 2, true>;

template <typename T, int G, int kW, bool kMfma = use_mfma<T, G>()>
struct DecodeShared {
  static constexpr int D = WaveAttn<T, G>::D;
  float p[kW][WaveAttn<T, G>::kPBufFloats];  // per wave, double-buffered page probabilities
  float o[kW][G][D];                         // per-wave results for the workgroup combine
  float ml[kW][G][2];
  uint4 q[WaveAttn<T, G>::kQInLds ? G * kRowBytes / 16 : 1];  // the group's query rows
};
template <typename T, int G, int kW>
struct DecodeShared<T, G, kW, true> {
  static constexpr int D = DecodeMfma<G>::D;
  alignas(16) char v[kW][DecodeMfma<G>::kLdsBytes];  // per wave, the staged V tiles
  alignas(16) float o[kW][G][D];
  float ml[kW][G][2];
};

constexpr int kSplitWaves = 4;  // waves per unit workgroup of the split decode

template <typename T, int G, int kW>
__global__ void __launch_bounds__(64 * kW) __attribute__((amdgpu_waves_per_eu(2)))
decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ k_pool, const T* __restrict__ v_pool,
    int num_phys, int Hkv, const int* __restrict__ page_indptr,
    const int* __restrict__ page_indices, const int* __restrict__ seq_lens,
    const int* __restrict__ sel, const int* __restrict__ sel_count, int k_stride,
    float scale_log2, int chunk, int max_units, float* __restrict__ part_o,
    float* __restrict__ part_ml, unsigned int* __restrict__ err) {
  using WA = WaveAttn<T, G>;
  constexpr int EPC = WA::EPC;
  constexpr int D = WA::D;
  constexpr bool kMfma = use_mfma<T, G>();
  __shared__ DecodeShared<T, G, kW> sh;

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
  const int idx = ubeg + wave + kW * lane;
  int jsel = idx;
  if (sel != nullptr && lane < (chunk + kW - 1) / kW && idx < k_stride) jsel = sel[row * k_stride + idx];
  const int n = L > 0 ? (L + kPage - 1) / kPage : 0;
  int count = n;
  if (sel != nullptr) {
    count = cnt_sel < k_stride ? cnt_sel : k_stride;
    count = count < n ? count : n;  // a row selects distinct pages of the sequence
    count = count > 0 ? count : 0;
  }
  if (sel != nullptr && u == 0 && tid == 0 && (cnt_sel < 1 || cnt_sel > min(k_stride, n)))
    report_bad(err, kErrCount);
  int units = (count + chunk - 1) / chunk;
  units = units < 1 ? 1 : (units < max_units ? units : max_units);
  if (u >= units) return;  // whole workgroup: nothing in this unit
  const int uend = min(ubeg + chunk, count);
  const int npw = (uend - ubeg > wave) ? (uend - ubeg - wave + kW - 1) / kW : 0;

  // This wave's pages: physical slot and valid-token count, one per lane.
  int my_p = 0, my_valid = 0;
  if (lane < npw) {
    const int j = jsel;
    if (j >= 0 && j < n) {
      const int p = page_indices[tbase + j];
      if (p >= 0 && p < num_phys) {
        my_p = p;
        my_valid = min(kPage, L - kPage * j);
      } else {
        report_bad(err, kErrPhys);
      }
    } else {
      report_bad(err, kErrSel);
    }
  }

  const char* qrows = reinterpret_cast<const char*>(q) + ((size_t)b * Hq + h * G) * kRowBytes;
  LanePages src{my_p, my_valid, npw};
  const char* kbase = reinterpret_cast<const char*>(k_pool) + (size_t)h * kTileBytes;
  const char* vbase = reinterpret_cast<const char*>(v_pool) + (size_t)h * kTileBytes;
  const size_t page_stride = (size_t)Hkv * kTileBytes;
  if constexpr (kMfma) {
    DecodeMfma<G> wa;
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
  // ---- the workgroup combine of the kW waves -> one partial per (unit, head)
  __syncthreads();

  const size_t unit = row * (size_t)max_units + u;
  for (int idx2 = tid; idx2 < G * D; idx2 += 64 * kW) {
    const int hh = idx2 / D;
    const int d = idx2 - hh * D;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kW; ++w) M = fmaxf(M, sh.ml[w][hh][0]);
    float acc = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
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

// ---- stream split ---------------------------------------------------------
// Rows r = b * Hkv + h are concatenated in that order, row r holding c_b
// entries: its selected pages (c_b = min(k, n_b)) or every page (c_b = n_b),
// at least one. Wave w of W takes entries [w T / W, (w + 1) T / W) of the T
// in all, so every wave attends the same number of pages, and runs them as
// one pipelined page loop: where its share crosses from one row into the
// next, the finished row segment's (o, max, sum) goes to partial slot w + r
// and the state restarts with the next row's query while the next page's
// loads are already in flight. A row's slots are consecutive (from its first
// wave's to its last wave's); row_slots[r] = (first wave, last wave) for the
// merge. No workgroup barrier follows the table set-up, so a wave never
// waits for another.

struct StreamTables {
  long long pre[kStreamMaxB + 1];  // pre[b] = c_0 + ... + c_{b-1}
  int len[kStreamMaxB];            // seq_lens
  int base[kStreamMaxB];           // page_indptr
  __device__ __forceinline__ int count(int b) const { return (int)(pre[b + 1] - pre[b]); }
};

// A wave's share of the entries, fetched 64 at a time (one entry per lane) a
// batch ahead of use. Pages are returned as tile indices p * Hkv + h.
struct StreamSrc {
  const StreamTables* t;
  const char* q;
  const int* page_indices;
  const int* sel;
  const int* sel_count;
  unsigned int* err;
  int Hkv, G, k, num_phys, lane;
  long long e_next, e_end;  // next entry to fetch; end of the share
  int fb, fh, fj;           // (b, h, j) of entry e_next
  int row0, first0;         // the share's first row; 1 if the share starts at its j = 0
  // current batch, one entry per lane: tile, valid tokens, row, segment word
  int c_p = 0, c_v = 0, c_r = 0, c_w = 0;
  // next batch (raw): row, logical page, loaded table entry, word
  int n_r = 0, n_j = -1, n_raw = -1, n_w = 0;
  int c_n = 0, n_n = 0, i = 0;
  int segw = 0;
  int cur_row;
  uint4 qn[4];  // query of the row most recently entered (B operand layout)

  // nothing left to return (the first batch is fetched before the page loop
  // asks, which already moves e_next)
  __device__ __forceinline__ bool empty() const { return i >= c_n && n_n <= 0; }

  // Fill the next batch with the entries from e_next on.
  __device__ __forceinline__ void fill() {
    const long long left = e_end - e_next;
    const int n = left < 64 ? (int)left : 64;
    n_n = n;
    if (n <= 0) return;
    int b = fb, h = fh, j = fj;
    if (lane < n) {
      int rem = lane;
      int c = t->count(b);
      while (rem >= c - j) {  // each step leaves a row: at most lane steps
        rem -= c - j;
        j = 0;
        if (++h == Hkv) {
          h = 0;
          ++b;
        }
        c = t->count(b);
      }
      j += rem;
    }
    const int row = b * Hkv + h;
    // the entry after this batch: (fb, fh, fj) for the next fill
    {
      int lb = __builtin_amdgcn_readlane(b, n - 1), lh = __builtin_amdgcn_readlane(h, n - 1);
      int lj = __builtin_amdgcn_readlane(j, n - 1) + 1;
      if (lj == t->count(lb)) {
        lj = 0;
        if (++lh == Hkv) {
          lh = 0;
          ++lb;
        }
      }
      fb = lb;
      fh = lh;
      fj = lj;
    }
    e_next += n;
    const int row_after = e_next < e_end ? fb * Hkv + fh : -1;
    const int nxt_lane = __builtin_amdgcn_ds_bpermute(((lane + 1) & 63) * 4, row);
    const int next_row = lane + 1 < n ? nxt_lane : row_after;
    int word = 0;
    if (lane < n && next_row != row) {
      const int first = (row != row0 || first0) ? 2 : 0;
      const int last = j == t->count(b) - 1 ? 4 : 0;
      word = 1 | first | last | (row << 3);
    }
    n_r = row;
    n_w = word;
    n_j = -1;  // logical page of the entry, -1 when it attends nothing
    n_raw = -1;
    if (lane < n) {
      const int L = t->len[b];
      const int np = L > 0 ? (L + kPage - 1) / kPage : 0;
      if (sel == nullptr) {
        if (j < np) {
          n_j = j;
          n_raw = page_indices[t->base[b] + j];
        }
      } else {
        // two dependent levels: the list entry (j < c_b <= k), then its
        // table entry; entries past the row's count attend nothing
        const int cnt = sel_count[row];
        const int act = min(min(cnt, k), np);
        const int jl = sel[(size_t)row * k + j];
        if (j < act && jl >= 0 && jl < np) {
          n_j = jl;
          n_raw = page_indices[t->base[b] + jl];
        } else if (j < act) {
          report_bad(err, kErrSel);
        }
        if (j == 0 && (cnt < 1 || cnt > min(k, np))) report_bad(err, kErrCount);
      }
    }
  }

  // Validate the raw next batch into the current one.
  __device__ __forceinline__ void take() {
    c_n = n_n;
    i = 0;
    const int b = n_r / Hkv;
    const int h = n_r - b * Hkv;
    const int L = t->len[b];
    const int jl = n_j;
    const bool ok = lane < c_n && jl >= 0 && n_raw >= 0 && n_raw < num_phys;
    if (lane < c_n && jl >= 0 && !ok) report_bad(err, kErrPhys);
    c_p = ok ? n_raw * Hkv + h : 0;
    c_v = ok ? min(kPage, L - kPage * jl) : 0;
    c_r = n_r;
    c_w = lane < c_n ? n_w : 0;
    fill();
  }

  __device__ __forceinline__ void next(int* p, int* valid) {
    if (i == c_n) {
      if (n_n <= 0) {
        *p = 0;
        *valid = -1;
        segw = 0;
        return;
      }
      take();
    }
    *p = __builtin_amdgcn_readlane(c_p, i);
    *valid = __builtin_amdgcn_readlane(c_v, i);
    segw = __builtin_amdgcn_readlane(c_w, i);
    const int row = __builtin_amdgcn_readlane(c_r, i);
    if (row != cur_row) {  // entering a row: its query, for the hook to swap in
      cur_row = row;
      load_q(row);
    }
    ++i;
  }
  __device__ __forceinline__ int seg() const { return segw; }

  __device__ __forceinline__ void load_q(int row) {
    const int c16 = lane & 15;
    const int grp = lane >> 4;
    const char* qr = q + (size_t)row * G * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qn[ks] = c16 < G ? ld16(qr + c16 * kRowBytes + (8 * grp + 32 * ks) * 2) : make_uint4(0, 0, 0, 0);
  }
};

template <int G>
struct StreamHook {
  static constexpr bool kActive = true;
  StreamSrc* src;
  float* part_o;
  float* part_ml;
  int* row_slots;
  int w, lane;
  __device__ __forceinline__ void operator()(DecodeMfma<G>& wa, int word) const {
    const int r = word >> 3;
    const size_t slot = (size_t)w + r;
    wa.store(part_o + slot * G * DecodeMfma<G>::D, part_ml + slot * G * 2, lane);
    if (lane == 0) {
      if (word & 2) row_slots[2 * r] = w;
      if (word & 4) row_slots[2 * r + 1] = w;
    }
    wa.restart(src->qn);
  }
};

template <int G>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
decode_stream_kernel(
    const bf16s* __restrict__ q, const bf16s* __restrict__ k_pool, const bf16s* __restrict__ v_pool,
    int num_phys, int B, int Hkv, const int* __restrict__ page_indptr,
    const int* __restrict__ page_indices, const int* __restrict__ seq_lens,
    const int* __restrict__ sel, const int* __restrict__ sel_count, int k, float scale_log2,
    int nwaves, float* __restrict__ part_o, float* __restrict__ part_ml,
    int* __restrict__ row_slots, unsigned int* __restrict__ err) {
  using WA = DecodeMfma<G>;
  __shared__ StreamTables tab;
  __shared__ alignas(16) char vl[4][WA::kLdsBytes];
  __shared__ long long wtot[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- per-sequence tables: lengths, table bases, prefix of the counts
  constexpr int kPer = kStreamMaxB / 256;
  const int b0 = tid * kPer;
  int cnt[kPer];
  long long local = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int b = b0 + e;
    cnt[e] = 0;
    if (b < B) {
      const int L = seq_lens[b];
      tab.len[b] = L;
      tab.base[b] = page_indptr[b];
      const int np = L > 0 ? (L + kPage - 1) / kPage : 0;
      const int c = sel != nullptr ? min(k, np) : np;
      cnt[e] = c > 1 ? c : 1;
      local += cnt[e];
    }
  }
  long long incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  long long excl = incl - local;
  for (int w2 = 0; w2 < wave; ++w2) excl += wtot[w2];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int b = b0 + e;
    if (b < B) tab.pre[b] = excl;
    excl += cnt[e];
  }
  if (tid == 0) tab.pre[B] = wtot[0] + wtot[1] + wtot[2] + wtot[3];
  __syncthreads();

  // ---- this wave's share
  const long long T = (long long)Hkv * tab.pre[B];
  const int w = blockIdx.x * 4 + wave;
  const long long e0 = (long long)w * T / nwaves;
  const long long e1 = (long long)(w + 1) * T / nwaves;
  if (e0 >= e1) return;
  int lo = 0, hi = B;  // largest b with Hkv * pre[b] <= e0
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((long long)Hkv * tab.pre[mid] <= e0)
      lo = mid;
    else
      hi = mid;
  }
  const long long off = e0 - (long long)Hkv * tab.pre[lo];
  const int c0 = tab.count(lo);
  const int h0 = (int)(off / c0);
  const int j0 = (int)(off - (long long)h0 * c0);

  StreamSrc src;
  src.t = &tab;
  src.q = reinterpret_cast<const char*>(q);
  src.page_indices = page_indices;
  src.sel = sel;
  src.sel_count = sel_count;
  src.err = err;
  src.Hkv = Hkv;
  src.G = G;
  src.k = k;
  src.num_phys = num_phys;
  src.lane = lane;
  src.e_next = e0;
  src.e_end = e1;
  src.fb = lo;
  src.fh = h0;
  src.fj = j0;
  src.row0 = lo * Hkv + h0;
  src.first0 = j0 == 0;
  src.cur_row = src.row0;
  src.fill();

  WA wa;
  wa.init(reinterpret_cast<const char*>(q) + (size_t)src.row0 * G * kRowBytes, lane);
  StreamHook<G> hook{&src, part_o, part_ml, row_slots, w, lane};
  wa.run(src, reinterpret_cast<const char*>(k_pool), reinterpret_cast<const char*>(v_pool),
         (size_t)kTileBytes, scale_log2, vl[wave], lane, hook);
}

// One wave per (b, hq): log-sum-exp merge of the unit partials (and of the
// shared-prefix partials for the cascade), then normalisation. The partials
// are loaded without waiting for the row's unit count (every slot the row can
// own is in bounds), so the merge costs one round of dependent loads.
// kBatch: partial slots loaded per round. A cascade row of 512-token prefix
// splits over a 4096-token prefix has 8 prefix slots and usually one or two
// suffix segments, so 10 take it in one round (16 loaded 6 unused slots and
// measured 2.5 us slower on that merge; 12 in between); rows of at most 5
// slots (units of a short list, or 4 prefix splits and one suffix partial)
// take the 5-slot instance (10 loaded 5 unused slots: c5's one-call step
// 71.1 against 67.9 us).
template <int D, int kBatch>
__global__ void __launch_bounds__(256) merge_kernel(
    int B, int Hkv, int G, const int* __restrict__ seq_lens, const int* __restrict__ sel_count,
    int k_stride, int chunk, int max_units, const float* __restrict__ part_o,
    const float* __restrict__ part_ml, const float* __restrict__ pre_o,
    const float* __restrict__ pre_ml, int n_pre, const int* __restrict__ row_slots, int nwaves,
    float* __restrict__ out, float* __restrict__ lse) {
  constexpr int PER = D / 64;
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
  // the row's unit slots: ucap of them from ubase (stream split: the slots of
  // its first to last wave, known once row_slots is read; units: every slot
  // the row can own, loaded before its unit count is known)
  int ubase = (int)(row * max_units), ucap = max_units, units = -1;
  if (row_slots != nullptr) {
    const int f = min(max(row_slots[2 * row], 0), nwaves - 1);
    const int l = min(max(row_slots[2 * row + 1], f), nwaves - 1);
    ubase = f + (int)row;
    ucap = l - f + 1;
    units = ucap;
  }
  const int slots = ucap + n_pre;

  float M = -__builtin_inff(), lsum = 0.0f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
  for (int base = 0; base < slots; base += kBatch) {
    float m[kBatch], l[kBatch], v[kBatch][PER];
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      const int i = min(base + t, slots - 1);
      const float* po;
      const float* pml;
      if (i < ucap) {
        const size_t un = (size_t)ubase + i;
        po = part_o + (un * G + hh) * D;
        pml = part_ml + (un * G + hh) * 2;
      } else {
        const size_t pr = ((size_t)h * n_pre + (i - ucap)) * ((size_t)B * G) + pre_row;
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
      const bool use = i < slots && (i < units || i >= ucap);
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

// The same merge with one wave per (b, h_kv) row for all G query heads of its
// group. A slot's partials of the group's heads are contiguous (G D floats;
// so are the group's outputs), so lane l merges the E = G D / 64
// consecutive floats at l E (of head l / (64 / G)) with 16-byte loads and
// stores: a quarter of the waves and of the load instructions of the kernel
// above, and per head the same arithmetic in the same order.
template <int D, int G, int kBatch>
__global__ void __launch_bounds__(256) merge_group_kernel(
    int B, int Hkv, const int* __restrict__ seq_lens, const int* __restrict__ sel_count, int k_stride, int chunk,
    int max_units, const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const float* __restrict__ pre_o, const float* __restrict__ pre_ml, int n_pre,
    const int* __restrict__ row_slots, int nwaves, float* __restrict__ out, float* __restrict__ lse) {
  constexpr int E = G * D / 64;  // floats per lane
  constexpr int LPH = 64 / G;    // lanes per head
  static_assert(E % 4 == 0 && LPH * E == D, "16-byte pieces within one head");
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (gw >= B * Hkv) return;
  const int b = gw / Hkv;
  const int h = gw - b * Hkv;
  const int hh = lane / LPH;
  const int off = lane * E;  // = hh D + (lane % LPH) E
  const size_t row = (size_t)gw;
  const int Hq = Hkv * G;
  const int L = seq_lens[b];
  const int cnt_sel = sel_count != nullptr ? sel_count[row] : 0;
  int ubase = (int)(row * max_units), ucap = max_units, units = -1;
  if (row_slots != nullptr) {
    const int f = min(max(row_slots[2 * row], 0), nwaves - 1);
    const int l = min(max(row_slots[2 * row + 1], f), nwaves - 1);
    ubase = f + (int)row;
    ucap = l - f + 1;
    units = ucap;
  }
  const int slots = ucap + n_pre;

  float M = -__builtin_inff(), lsum = 0.0f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  for (int base = 0; base < slots; base += kBatch) {
    float m[kBatch], l[kBatch];
    float4 v[kBatch][E / 4];
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      const int i = min(base + t, slots - 1);
      const float* po;
      const float* pml;
      if (i < ucap) {
        const size_t un = (size_t)ubase + i;
        po = part_o + un * G * D + off;
        pml = part_ml + (un * G + hh) * 2;
      } else {
        const size_t pr = ((size_t)h * n_pre + (i - ucap)) * ((size_t)B * G) + (size_t)b * G;
        po = pre_o + pr * D + off;
        pml = pre_ml + (pr + hh) * 2;
      }
      const float2 ml = *reinterpret_cast<const float2*>(pml);
      m[t] = ml.x;
      l[t] = ml.y;
#pragma unroll
      for (int e = 0; e < E / 4; ++e) v[t][e] = reinterpret_cast<const float4*>(po)[e];
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
      const bool use = i < slots && (i < units || i >= ucap);
      if (!use || m[t] == -__builtin_inff()) continue;
      if (m[t] > M) {
        const float a = (M == -__builtin_inff()) ? 0.0f : fast_exp2(M - m[t]);
        lsum *= a;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] *= a;
        M = m[t];
      }
      const float w = fast_exp2(m[t] - M);
      lsum = __builtin_fmaf(w, l[t], lsum);
#pragma unroll
      for (int e = 0; e < E / 4; ++e) {
        acc[4 * e + 0] = __builtin_fmaf(w, v[t][e].x, acc[4 * e + 0]);
        acc[4 * e + 1] = __builtin_fmaf(w, v[t][e].y, acc[4 * e + 1]);
        acc[4 * e + 2] = __builtin_fmaf(w, v[t][e].z, acc[4 * e + 2]);
        acc[4 * e + 3] = __builtin_fmaf(w, v[t][e].w, acc[4 * e + 3]);
      }
    }
  }
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  float4* o4 = reinterpret_cast<float4*>(out + ((size_t)b * Hq + (size_t)h * G) * D + off);
#pragma unroll
  for (int e = 0; e < E / 4; ++e)
    o4[e] = make_float4(acc[4 * e] * inv, acc[4 * e + 1] * inv, acc[4 * e + 2] * inv, acc[4 * e + 3] * inv);
  if (lse != nullptr && lane % LPH == 0) {
    lse[(size_t)b * Hq + h * G + hh] = lsum > 0.0f ? (M + __log2f(lsum)) * 0.69314718055994530942f : -__builtin_inff();
  }
}

constexpr int kMergeNarrow = 5;
constexpr int kMergeWide = 10;

hipError_t launch_merge_kernel(const LaunchCommon& c, int max_slots, const int* sel_count, int k, int chunk,
                               int max_units, Partials part, Partials prefix, int n_prefix, const int* row_slots,
                               int nwaves, float* out, float* lse, hipStream_t stream) {
  const bool narrow = max_slots <= kMergeNarrow;
  // (the group kernel's 16-byte accesses need 16-byte aligned partials and
  // output; workspace regions are, a caller's output normally is)
  const uintptr_t al = reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(part.o) |
                       reinterpret_cast<uintptr_t>(part.ml) | reinterpret_cast<uintptr_t>(prefix.o) |
                       reinterpret_cast<uintptr_t>(prefix.ml);
  // (with fewer rows than four waves per CU the group kernel leaves the chip
  // short of waves and the per-head merge is faster: c2's 128 rows 4.41
  // against 4.61 us, c3's 512 rows 6.54 against 7.23 us; c5's 2048 rows 6.67
  // against 7.68 us)
  const bool many_rows = c.B * c.Hkv >= 1024;
  if (c.D == 128 && (c.G == 4 || c.G == 8) && al % 16 == 0 && many_rows) {
    dim3 ggrid((c.B * c.Hkv + 3) / 4);
#define QSA_MERGE_G(GG, NB)                                                                                  \
  hipLaunchKernelGGL((merge_group_kernel<128, GG, NB>), ggrid, dim3(256), 0, stream, c.B, c.Hkv, c.seq_lens, \
                     sel_count, k, chunk, max_units, part.o, part.ml, prefix.o, prefix.ml, n_prefix, row_slots,  \
                     nwaves, out, lse)
    if (c.G == 4) {
      if (narrow)
        QSA_MERGE_G(4, kMergeNarrow);
      else
        QSA_MERGE_G(4, kMergeWide);
    } else {
      QSA_MERGE_G(8, kMergeNarrow);  // (16 floats per lane and slot: the narrow batch)
    }
#undef QSA_MERGE_G
    return hipGetLastError();
  }
  dim3 mgrid((c.B * c.Hq + 3) / 4);
#define QSA_MERGE(DD, NB)                                                                                 \
  hipLaunchKernelGGL((merge_kernel<DD, NB>), mgrid, dim3(256), 0, stream, c.B, c.Hkv, c.G, c.seq_lens,    \
                     sel_count, k, chunk, max_units, part.o, part.ml, prefix.o, prefix.ml, n_prefix, row_slots, \
                     nwaves, out, lse)
  if (c.D == 128) {
    if (narrow)
      QSA_MERGE(128, kMergeNarrow);
    else
      QSA_MERGE(128, kMergeWide);
  } else {
    if (narrow)
      QSA_MERGE(64, kMergeNarrow);
    else
      QSA_MERGE(64, kMergeWide);
  }
#undef QSA_MERGE
  return hipGetLastError();
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
  if constexpr (IsBf16<T>::value) {
    if (plan.stream) {
      const bf16s* kb = static_cast<const bf16s*>(c.k_pool);
      const bf16s* vb = static_cast<const bf16s*>(c.v_pool);
#define QSA_STREAM_CASE(GG)                                                                      \
  case GG:                                                                                       \
    hipLaunchKernelGGL((decode_stream_kernel<GG>), dim3(plan.waves / 4), dim3(256), 0, stream, qq, \
                       kb, vb, c.num_phys, c.B, c.Hkv, c.page_indptr, c.page_indices, c.seq_lens,  \
                       sel, sel_count, k, scale_log2, plan.waves, part.o, part.ml, part.row_slots, \
                       c.err);                                                                    \
    break;
      switch (c.G) {
        QSA_STREAM_CASE(4)
        QSA_STREAM_CASE(8)
        default:
          return hipErrorInvalidValue;
      }
#undef QSA_STREAM_CASE
    }
  }
  const T* kk = static_cast<const T*>(c.k_pool);
  const T* vv = static_cast<const T*>(c.v_pool);
  if (!plan.stream) {
#define QSA_DECODE_CASE(GG)                                                                     \
  case GG:                                                                                      \
    hipLaunchKernelGGL((decode_split_kernel<T, GG, kSplitWaves>), grid, dim3(64 * kSplitWaves), 0, stream, qq, \
                       kk, vv, c.num_phys, c.Hkv, c.page_indptr, c.page_indices, c.seq_lens, sel, \
                       sel_count, k, scale_log2, plan.chunk, plan.max_units, part.o, part.ml,  \
                       c.err);                                                                 \
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
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int* sc = sel != nullptr ? sel_count : nullptr;
  // (the stream split's rows own a data-dependent number of slots)
  const int max_slots = plan.stream ? kMergeWide + 1 : plan.max_units + n_prefix;
  return launch_merge_kernel(c, max_slots, sc, k, plan.chunk, plan.max_units, part, prefix, n_prefix,
                             plan.stream ? part.row_slots : nullptr, plan.waves, out, lse, stream);
}

}  // namespace

hipError_t launch_merge(const LaunchCommon& c, Partials part, int max_units, int chunk, Partials prefix,
                        int n_prefix, float* out, float* lse, hipStream_t stream) {
  if (c.D != 128) return hipErrorInvalidValue;
  return launch_merge_kernel(c, max_units + n_prefix, nullptr, 0, chunk, max_units, part, prefix, n_prefix, nullptr,
                             0, out, lse, stream);
}

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
