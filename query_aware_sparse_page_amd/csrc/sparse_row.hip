// Steps 2-4 of one decode step fused into one workgroup per (sequence, KV
// head) row: bound scores, top-K and attention over the selected pages, with
// the scores, the selection and the partial results kept in LDS (TinyServe
// page, §3.2: one kernel per decode step that scores pages, picks the top-K and
// attends over them, with the scores held on chip; the score is §2.2, the
// selection §2.3, the per-page attention decode_wave.h).
//
// Workgroup = 8 waves. Phases, separated by workgroup barriers:
//  1. Score: the row's metadata is one contiguous stream of 512-byte [m | M]
//     records (logical page order). 16 lanes per page, 4 pages per wave-step;
//     a wave scores chunks of 8 consecutive pages with two chunks of records
//     in flight (8 KiB per wave: smaller and fewer chunks in flight measured
//     faster than 16-page ones). The score arithmetic is the same as
//     score_kernel's (q split by sign, v_dot2 / fma, DPP sum, group max), so
//     both paths produce bit-identical group scores. With refresh_tail set the
//     wave owning the tail page rebuilds its min/max from the keys first and
//     writes it back. The row's page table is copied to LDS on the way.
//  2. Select: MSB-first radix select on the order-preserving keys of the
//     scores in LDS (8-bit digits, starting below the bits shared by the row's
//     min and max key; it stops as soon as the boundary digit's bin is taken
//     whole), then a compaction in page order: pages with key above the
//     threshold, plus the first ones equal to it (ties go to the smaller
//     logical page). The list is in ascending page order.
//  3. Attend: wave w takes list entries w, w+8, ... through the per-wave
//     paged attention of decode_wave.h (K/V read with the non-temporal hint:
//     each selected tile is read by one wave of one workgroup).
//  4. Merge: the 8 waves' (max, sum, o) are combined by log-sum-exp in LDS and
//     the normalised output and LSE are written; with one workgroup per row
//     no partials leave the chip.
// kCentroid = true runs phase 1 on centroid rows instead (the Vortex digest's
// mean-key page summary: 256-byte records scored as q . c, the tail page's
// centroid rebuilt with tile_mean); phases 2-4 are unchanged.
#include "decode_wave.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kRowWaves = 8;
constexpr int kRowThreads = kRowWaves * kWave;
static_assert(kRowThreads >= 256, "the radix histogram is cleared by 256 threads");
constexpr int kKeysPerThread = (kRowMaxPages + kRowThreads - 1) / kRowThreads;
constexpr int kChunkSteps = 2;                 // score steps per chunk (4 pages a step)
constexpr int kChunkPages = 4 * kChunkSteps;    // consecutive pages scored by one wave
constexpr int kScoreBufs = 2;                   // chunks of records in flight per wave

// Page buffers of the per-wave attention (see WaveAttn).
constexpr int row_stages(int gw) { return 2; }

template <typename T, int GW>
struct RowShared {
  using WA = WaveAttn<T, GW, row_stages(GW), true>;
  static constexpr int D = WA::D;
  union {
    struct {
      uint32_t key[kRowMaxPages];  // order keys of the group scores
      int phys[kRowMaxPages];      // the row's page table
    } s;
    struct {
      float o[kRowWaves][GW][D];
      float ml[kRowWaves][GW][2];
    } c;
  } u;
  int list[kRowMaxSelect];   // selected logical pages, ascending
  int plist[kRowMaxSelect];  // their physical slots (-1: out of range)
  uint4 q[WA::kQInLds ? GW * kRowBytes / 16 : 1];  // the attended query rows
  float p[kRowWaves][WA::kPBufFloats];
  uint32_t hist[2][256];
  uint32_t red[2][kRowWaves];
  uint32_t wsum[kRowWaves];
  uint32_t pick[3];
};

// S = 2 workgroups share one row when there are too few rows to fill the
// chip: each scores and selects the whole row (the group score needs every
// head of the group) and attends for every head over its share of the
// selected pages (list entries part, part + 2, ...), so that each K/V tile is
// read once. Workgroup w serves part (w / 8) % S of row (w % 8) + 8 * (w / (8
// S)), so the two workgroups of a row are dispatched to the same XCD
// (workgroups go round-robin over the 8 XCDs) and share its L2 for the row's
// records, which both stream. The two partial results (per head: max, sum
// and unnormalised output, G * (D + 2) floats) meet in the exchange buffer:
// each workgroup stores its own with agent-scope stores, waits for them to
// complete (s_waitcnt 0: the stores have reached the agent's coherence point
// before the counter is touched), then adds one to the row's arrival counter
// (agent scope); the
// one that finds the counter at 1 arrived second. It sets the counter back to
// 0 for the next call, reads the other partial (agent-scope loads), merges
// and writes O and LSE. The merge adds part 0's term to part 1's whichever
// workgroup does it, so the result does not depend on the arrival order. The
// counters must be zero before the first call and every call leaves them zero.
template <typename T, int G, int S, bool kCentroid>
__global__ void __launch_bounds__(kRowThreads) sparse_row_kernel(
    const T* __restrict__ q, T* __restrict__ meta, int stride, const T* __restrict__ k_pool,
    const T* __restrict__ v_pool, int num_phys, int Hkv, int rows,
    const int* __restrict__ page_indptr, const int* __restrict__ page_indices,
    const int* __restrict__ seq_lens, int refresh_tail, int k, float scale_log2,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ group_scores,
    int* __restrict__ sel, int* __restrict__ sel_count, unsigned int* __restrict__ xcnt,
    float* __restrict__ xpart, unsigned int* __restrict__ err) {
  static_assert(S == 1 || S == 2, "one or two workgroups per row");
  using WA = typename RowShared<T, G>::WA;
  constexpr int EPC = WA::EPC;
  constexpr int D = WA::D;
  __shared__ RowShared<T, G> sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = blockIdx.x;
  const int part = (wg >> 3) % S;
  const int row_i = (wg & 7) + 8 * (wg / (8 * S));
  if (row_i >= rows) return;  // padding of the last group of 8 rows (whole workgroup)
  const bool writer = part == 0;  // one workgroup of the row writes the shared outputs
  if (!writer) {
    group_scores = nullptr;
    sel = nullptr;
    sel_count = nullptr;
  }
  const int b = row_i / Hkv;
  const int h = row_i - b * Hkv;
  const int Hq = Hkv * G;
  const size_t row = (size_t)row_i;
  const int c = lane & 15;     // chunk within a metadata record
  const int slot = lane >> 4;  // which of the wave's 4 pages of a step

  // ---- phase 1: scores ---------------------------------------------------
  // The row's pages are scored in chunks of kChunkPages consecutive pages,
  // wave w taking chunks w, w + W, w + 2W, ... (W waves). With two
  // workgroups per row both then read a chunk's records at about the same
  // time; this measured faster than handing chunks out on demand from an
  // LDS counter (and needs no barrier before the loop).
  const int L = seq_lens[b];
  const int tbase = page_indptr[b];
  // page records: [m | M] (512 bytes) or a centroid row (256 bytes)
  constexpr int kRec = kCentroid ? kRowBytes : 2 * kRowBytes;
  const char* mrow = reinterpret_cast<const char*>(meta) + row * stride * kRec;
  // Records of chunk ci (pages past the row read the last slot of the
  // row's stride, which is in bounds; their scores are masked).
  auto issue = [&](int ci, uint4 (&bm)[kChunkSteps], uint4 (&bM)[kChunkSteps]) {
#pragma unroll
    for (int t = 0; t < kChunkSteps; ++t) {
      const int j = min(ci * kChunkPages + 4 * t + slot, stride - 1);
      bm[t] = ld16(mrow + (size_t)j * kRec + c * 16);
      if (!kCentroid) bM[t] = ld16(mrow + (size_t)j * kRec + 256 + c * 16);
    }
  };
  // the query rows first: the scores wait for them but not for the records
  uint4 qn[G], qp[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const char* qrow = reinterpret_cast<const char*>(q) + ((size_t)b * Hq + h * G + hh) * kRowBytes;
    qn[hh] = ld16(qrow + c * 16);
  }
  __builtin_amdgcn_sched_barrier(0);
  uint4 bm[kScoreBufs][kChunkSteps], bM[kScoreBufs][kChunkSteps];
  int cc[kScoreBufs];
#pragma unroll
  for (int u = 0; u < kScoreBufs; ++u) {
    cc[u] = wave + u * kRowWaves;
    issue(cc[u], bm[u], bM[u]);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (!kCentroid) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const uint4 qc = qn[hh];
      chunk_sign_split(qc, qn[hh], qp[hh], T{});
    }
  }
  // (the host keeps rows within kRowMaxPages; the clamp guards the LDS arrays)
  const int n = L > 0 ? min(min((L + kPage - 1) / kPage, stride), kRowMaxPages) : 0;
  // (values needed only after scoring are loaded now and stored to LDS
  // after the chunk loop: a store would wait for the records in flight)
  uint4 qstage = make_uint4(0, 0, 0, 0);
  if constexpr (WA::kQInLds) {
    if (tid < G * kRowBytes / 16)
      qstage = ld16(reinterpret_cast<const char*>(q) + ((size_t)b * Hq + h * G) * kRowBytes + tid * 16);
  }
  const int nchunks = (n + kChunkPages - 1) / kChunkPages;

  // the row's page table (to LDS for the attention phase)
  // (unconditional loads: a fixed number of loads in flight keeps the
  // memory-counter waits of the chunk loop partial)
  int ph[kKeysPerThread];
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) {
    const int j = tid + i * kRowThreads;
    ph[i] = page_indices[n > 0 ? tbase + min(j, n - 1) : 0];
  }

  // Tail-page refresh: wave 0 rebuilds the tail page's record, writes it
  // back and scores the page; the chunk loop leaves that page alone.
  const int jt = n - 1;
  bool tail_ok = false;  // workgroup-uniform
  int tail_p = -1;
  if (refresh_tail && n > 0) {
    tail_p = page_indices[tbase + jt];
    tail_ok = tail_p >= 0 && tail_p < num_phys;  // else the stored record is scored unchanged
    if (!tail_ok && tid == 0) report_bad(err, kErrPhys);
  }
  auto score_page = [&](const uint4& m, const uint4& M) -> float {
    float gmax = -__builtin_inff();
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float acc = 0.0f;
      acc = chunk_dot(qn[hh], m, acc, T{});
      if (!kCentroid) acc = chunk_dot(qp[hh], M, acc, T{});
      gmax = fmaxf(gmax, sum16(acc));
    }
    return gmax;
  };
  if (tail_ok && wave == 0) {
    uint4 tmn, tmx;
    const int valid = min(kPage, L - kPage * jt);
    const char* tile = reinterpret_cast<const char*>(k_pool) + ((size_t)tail_p * Hkv + h) * kTileBytes;
    char* trec = reinterpret_cast<char*>(meta) + (row * stride + jt) * kRec;
    if constexpr (kCentroid) {
      tmn = tile_mean<T>(tile, valid, lane);
      tmx = tmn;
      if (writer && lane < 16) st16(trec + c * 16, tmn);
    } else {
      tile_minmax<T>(tile, valid, lane, tmn, tmx);
      if (writer && lane < 32) st16(trec + (lane >> 4) * 256 + c * 16, lane < 16 ? tmn : tmx);
    }
    const float gmax = score_page(tmn, tmx);
    if (lane == 0) sh.u.s.key[jt] = score_key(gmax);
  }

  auto score = [&](int ci, const uint4 (&bm)[kChunkSteps], const uint4 (&bM)[kChunkSteps]) {
#pragma unroll
    for (int t = 0; t < kChunkSteps; ++t) {
      const int j = ci * kChunkPages + 4 * t + slot;
      // (branch-free: records of masked pages may hold anything; their
      // score is replaced, never used)
      const bool ok = j < n && !(tail_ok && j == jt);
      const float gmax = score_page(bm[t], bM[t]);
      if (c == 0 && ok) sh.u.s.key[j] = score_key(gmax);
    }
  };
  // kScoreBufs buffers in rotation: while one buffer's chunk is scored the
  // others' records are in flight; a scored buffer is refilled with the next
  // chunk at once. The loop body has no early exit (chunks past the row are
  // masked and only cost cache hits), so the memory-counter waits stay
  // partial; the scheduling barriers keep the loads in issue order.
  while (true) {
    bool more = false;
#pragma unroll
    for (int u = 0; u < kScoreBufs; ++u) {
      score(cc[u], bm[u], bM[u]);
      cc[u] += kScoreBufs * kRowWaves;
      issue(min(cc[u], nchunks), bm[u], bM[u]);
      __builtin_amdgcn_sched_barrier(0);
      more |= cc[u] < nchunks;
    }
    if (!more) break;
  }
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) {
    const int j = tid + i * kRowThreads;
    if (j < n) sh.u.s.phys[j] = ph[i];
  }
  if constexpr (WA::kQInLds) {
    if (tid < G * kRowBytes / 16) sh.q[tid] = qstage;
  }
  if (tid < 256) sh.hist[0][tid] = 0u;

  // ---- phase 2: top-K ----------------------------------------------------
  const int keff = min(min(k, n), kRowMaxSelect);  // the host keeps min(k, n) within the list
  const int kpt = (n + kRowThreads - 1) / kRowThreads;  // keys per thread, contiguous
  const int j0 = tid * kpt;
  uint32_t keys[kKeysPerThread];
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) {
    keys[i] = 0u;
    if (i < kpt && j0 + i < n) {
      keys[i] = sh.u.s.key[j0 + i];
      kmin = min(kmin, keys[i]);
      kmax = max(kmax, keys[i]);
    }
  }
  if (group_scores != nullptr) {
    // the key is invertible (only -0 comes back as +0)
    for (int j = tid; j < stride; j += kRowThreads)
      group_scores[row * stride + j] =
          j < n ? __uint_as_float(key_to_f32(sh.u.s.key[j])) : -__builtin_inff();
  }
  uint32_t krem = (uint32_t)keff;
  uint32_t thr = 0u;  // threshold prefix at granularity `shift`
  int shift = 0;
  if (keff < n) {
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
    if (lane == 0) {
      sh.red[0][wave] = kmin;
      sh.red[1][wave] = kmax;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) {
      kmin = min(kmin, sh.red[0][w]);
      kmax = max(kmax, sh.red[1][w]);
    }
    const uint32_t diff = kmin ^ kmax;
    thr = kmin;
    if (diff != 0u) {
      shift = 32 - __builtin_clz(diff);
      thr = (uint32_t)((uint64_t)kmin >> shift);
      int pass = 0;
      while (shift > 0) {
        const int nb = shift < 8 ? shift : 8;
        const int lo = shift - nb;
        const uint32_t nbins = 1u << nb;
        uint32_t* hcur = sh.hist[pass & 1];
#pragma unroll
        for (int i = 0; i < kKeysPerThread; ++i) {
          if (i < kpt && j0 + i < n && (uint32_t)((uint64_t)keys[i] >> shift) == thr)
            atomicAdd(&hcur[(keys[i] >> lo) & (nbins - 1u)], 1u);
        }
        if (tid >= kRowThreads - 256) sh.hist[(pass + 1) & 1][tid - (kRowThreads - 256)] = 0u;
        __syncthreads();
        if (wave == 0) {
          // lane l scans digits nbins-1 - (4l .. 4l+3), i.e. descending
          uint32_t cnt[4];
          uint32_t local = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int pos = lane * 4 + i;
            cnt[i] = pos < (int)nbins ? hcur[nbins - 1 - pos] : 0u;
            local += cnt[i];
          }
          uint32_t above = wave_scan_incl(local) - local;
          if (above < krem && above + local >= krem) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (above < krem && above + cnt[i] >= krem) {
                sh.pick[0] = nbins - 1u - (uint32_t)(lane * 4 + i);
                sh.pick[1] = krem - above;
                sh.pick[2] = cnt[i];
              }
              above += cnt[i];
            }
          }
        }
        __syncthreads();
        thr = (thr << nb) | sh.pick[0];
        krem = sh.pick[1];
        shift = lo;
        if (krem == sh.pick[2]) break;  // the boundary bin is taken whole
        ++pass;
      }
    }
  }

  // compaction in page order: above the threshold, then the first krem equal
  uint32_t gt_n = 0, eq_n = 0;
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) {
    if (i < kpt && j0 + i < n) {
      const uint32_t kk = (uint32_t)((uint64_t)keys[i] >> shift);
      gt_n += kk > thr ? 1u : 0u;
      eq_n += kk == thr ? 1u : 0u;
    }
  }
  if (keff == n) {  // every page: nothing to compare
    gt_n = (uint32_t)max(0, min(kpt, n - j0));
    eq_n = 0;
  }
  uint32_t total;
  const uint32_t excl = block_excl_scan<kRowWaves>(gt_n | (eq_n << 16), sh.wsum, &total);
  uint32_t gt_before = excl & 0xFFFFu;
  uint32_t eq_before = excl >> 16;
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) {
    const int j = j0 + i;
    if (i < kpt && j < n) {
      const uint32_t kk = (uint32_t)((uint64_t)keys[i] >> shift);
      const bool gt = keff == n || kk > thr;
      const bool eq = keff < n && kk == thr;
      if (gt || (eq && eq_before < krem)) {  // keff <= kRowMaxSelect bounds pos
        const uint32_t pos = gt_before + (eq_before < krem ? eq_before : krem);
        if (pos < (uint32_t)keff) {
          const int pp = sh.u.s.phys[j];
          sh.list[pos] = j;
          const bool pok = pp >= 0 && pp < num_phys;
          sh.plist[pos] = pok ? pp : -1;
          if (!pok && part == 0) report_bad(err, kErrPhys);
          if (sel != nullptr) sel[row * k + pos] = j;
        }
      }
      gt_before += gt ? 1u : 0u;
      eq_before += eq ? 1u : 0u;
    }
  }
  if (sel != nullptr)
    for (int i = keff + tid; i < k; i += kRowThreads) sel[row * k + i] = -1;
  if (sel_count != nullptr && tid == 0) sel_count[row] = keff;
  __syncthreads();

  // ---- phase 3: attention over the selected pages --------------------------
  // Wave w of part p takes list entries p + S (w + 8 i), i = 0, 1, ... (a
  // fixed split keeps the summation order, and so the result, the same from
  // run to run).
  const int first_e = part + S * wave;
  const int npw = keff > first_e ? (keff - first_e + S * kRowWaves - 1) / (S * kRowWaves) : 0;
  int my_p = 0, my_valid = 0;
  if (lane < npw) {
    const int e = first_e + S * kRowWaves * lane;
    const int pp = sh.plist[e];
    if (pp >= 0) {
      my_p = pp;
      my_valid = min(kPage, L - kPage * sh.list[e]);
    }
  }
  LanePages src{my_p, my_valid, npw};

  WA wa;
  wa.init(WA::kQInLds ? reinterpret_cast<const char*>(sh.q)
                      : reinterpret_cast<const char*>(q) + ((size_t)b * Hq + h * G) * kRowBytes,
          lane);
  wa.run(src, reinterpret_cast<const char*>(k_pool) + (size_t)h * kTileBytes,
         reinterpret_cast<const char*>(v_pool) + (size_t)h * kTileBytes,
         (size_t)Hkv * kTileBytes, scale_log2, sh.p[wave], lane);

  // ---- phase 4: merge of the 8 waves ----------------------------------------
  float mw, lw;
  wa.reduce(&mw, &lw);
  if (lane < 16) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < EPC; ++e) sh.u.c.o[wave][hh][lane * EPC + e] = wa.o[hh][e];
  }
  if (lane < G) {
    sh.u.c.ml[wave][lane][0] = mw;
    sh.u.c.ml[wave][lane][1] = lw;
  }
  __syncthreads();
  // this workgroup's result per (head, dim): max, sum, unnormalised output
  constexpr int kPer = (G * D + kRowThreads - 1) / kRowThreads;
  float accv[kPer], mv[kPer], lv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int idx = tid + i * kRowThreads;
    accv[i] = 0.0f;
    mv[i] = -__builtin_inff();
    lv[i] = 0.0f;
    if (idx < G * D) {
      const int hh = idx / D;
      const int d = idx - hh * D;
      float M = -__builtin_inff();
#pragma unroll
      for (int w = 0; w < kRowWaves; ++w) M = fmaxf(M, sh.u.c.ml[w][hh][0]);
      float acc = 0.0f, lsum = 0.0f;
#pragma unroll
      for (int w = 0; w < kRowWaves; ++w) {
        const float m2 = sh.u.c.ml[w][hh][0];
        const float sc = (m2 == -__builtin_inff()) ? 0.0f : fast_exp2(m2 - M);
        acc += sh.u.c.o[w][hh][d] * sc;
        lsum += sh.u.c.ml[w][hh][1] * sc;
      }
      accv[i] = acc;
      mv[i] = M;
      lv[i] = lsum;
      if constexpr (S == 2) {
        // exchange slot of (row, part): [G][D] outputs, then [G][2] (max, sum)
        float* xo = xpart + (row * 2 + part) * (size_t)(G * (D + 2));
        __hip_atomic_store(xo + idx, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0) {
          __hip_atomic_store(xo + G * D + 2 * hh, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(xo + G * D + 2 * hh + 1, lsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
  if constexpr (S == 2) {
    // every thread's stores complete before the arrival is counted
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const unsigned int old = __hip_atomic_fetch_add(xcnt + row, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old > 1u) report_bad(err, kErrExchange);  // the counters were not zero before the call
      sh.pick[0] = old;
    }
    __syncthreads();
    if (sh.pick[0] == 0u) return;  // first to arrive: the other workgroup merges
    if (tid == 0) __hip_atomic_store(xcnt + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int idx = tid + i * kRowThreads;
    if (idx < G * D) {
      const int hh = idx / D;
      const int d = idx - hh * D;
      float M = mv[i], acc = accv[i], lsum = lv[i];
      if constexpr (S == 2) {
        const float* xo = xpart + (row * 2 + (1 - part)) * (size_t)(G * (D + 2));
        const float acc1 = __hip_atomic_load(xo + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float m1 = __hip_atomic_load(xo + G * D + 2 * hh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float l1 = __hip_atomic_load(xo + G * D + 2 * hh + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // part 0's term first, whichever part merges: both workgroups then
        // evaluate the same expression on the same operands, so however it is
        // contracted into a fused multiply-add the rounding is the same
        const bool p0 = part == 0;
        const float aA = p0 ? acc : acc1, aB = p0 ? acc1 : acc;
        const float mA = p0 ? M : m1, mB = p0 ? m1 : M;
        const float lA = p0 ? lsum : l1, lB = p0 ? l1 : lsum;
        const float mn = fmaxf(mA, mB);
        const float sA = (mA == -__builtin_inff()) ? 0.0f : fast_exp2(mA - mn);
        const float sB = (mB == -__builtin_inff()) ? 0.0f : fast_exp2(mB - mn);
        acc = aA * sA + aB * sB;
        lsum = lA * sA + lB * sB;
        M = mn;
      }
      const size_t qrow = (size_t)b * Hq + h * G + hh;
      out[qrow * D + d] = lsum > 0.0f ? acc / lsum : 0.0f;
      if (lse != nullptr && d == 0)
        lse[qrow] = lsum > 0.0f ? (M + __log2f(lsum)) * 0.69314718055994530942f : -__builtin_inff();
    }
  }
}

template <typename T, int G, int S, bool kCentroid>
void launch_row(const LaunchCommon& c, const void* q, void* meta, int stride, int refresh_tail,
                int k, float scale_log2, float* out, float* lse, float* group_scores, int* sel,
                int* sel_count, const RowExchange& x, hipStream_t stream) {
  const int rows = c.B * c.Hkv;
  const int wgs = S == 1 ? rows : S * ((rows + 7) / 8 * 8);
  hipLaunchKernelGGL((sparse_row_kernel<T, G, S, kCentroid>), dim3(wgs), dim3(kRowThreads), 0, stream,
                     static_cast<const T*>(q), static_cast<T*>(meta), stride,
                     static_cast<const T*>(c.k_pool), static_cast<const T*>(c.v_pool), c.num_phys,
                     c.Hkv, rows, c.page_indptr, c.page_indices, c.seq_lens, refresh_tail, k,
                     scale_log2, out, lse, group_scores, sel, sel_count, x.counters, x.partials,
                     c.err);
}

template <typename T, bool kCen>
hipError_t launch_sparse_row_t(const LaunchCommon& c, const void* q, void* meta, int stride,
                               int refresh_tail, int k, float scale_log2, const RowExchange& x,
                               float* out, float* lse, float* group_scores, int* sel,
                               int* sel_count, hipStream_t stream) {
  const bool two = x.counters != nullptr;
#define QSA_ROW_ARGS c, q, meta, stride, refresh_tail, k, scale_log2, out, lse, group_scores, sel, \
                     sel_count, x, stream
  switch (c.G) {
    case 1: two ? launch_row<T, 1, 2, kCen>(QSA_ROW_ARGS) : launch_row<T, 1, 1, kCen>(QSA_ROW_ARGS); break;
    case 2: two ? launch_row<T, 2, 2, kCen>(QSA_ROW_ARGS) : launch_row<T, 2, 1, kCen>(QSA_ROW_ARGS); break;
    case 4: two ? launch_row<T, 4, 2, kCen>(QSA_ROW_ARGS) : launch_row<T, 4, 1, kCen>(QSA_ROW_ARGS); break;
    case 8: two ? launch_row<T, 8, 2, kCen>(QSA_ROW_ARGS) : launch_row<T, 8, 1, kCen>(QSA_ROW_ARGS); break;
    default:
      return hipErrorInvalidValue;
  }
#undef QSA_ROW_ARGS
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_row(const LaunchCommon& c, const void* q, void* meta, int stride,
                             int refresh_tail, int k, float scale_log2, const RowExchange& x,
                             bool centroid, float* out, float* lse, float* group_scores, int* sel,
                             int* sel_count, hipStream_t stream) {
#define QSA_ROW_CALL(TT, CC)                                                                      \
  launch_sparse_row_t<TT, CC>(c, q, meta, stride, refresh_tail, k, scale_log2, x, out, lse,      \
                              group_scores, sel, sel_count, stream)
  if (c.bf16) return centroid ? QSA_ROW_CALL(bf16s, true) : QSA_ROW_CALL(bf16s, false);
  return centroid ? QSA_ROW_CALL(float, true) : QSA_ROW_CALL(float, false);
#undef QSA_ROW_CALL
}

}  // namespace qsa
