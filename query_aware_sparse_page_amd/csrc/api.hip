// The libqsa C ABI: argument validation, work planning and kernel launches on
// the caller's stream. Declarations and contracts are in include/qsa.h.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "host.h"
#include "qsa.h"
#include "qsa_internal.h"

namespace qsa {
namespace host {

thread_local std::string g_last_error;

qsa_status fail(qsa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

qsa_status ok() {
  g_last_error.clear();
  return QSA_OK;
}

qsa_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(QSA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

int pages_of(int L) { return (L + 15) / 16; }

// Largest second or third launch grid dimension (the sequence index, the
// decode unit index).
constexpr int kMaxGridDim = 65535;

// Shape checks shared by every entry point.
qsa_status check_dims(const qsa_dims* d) {
  if (d == nullptr) return fail(QSA_ERR_INVALID_ARG, "dims is NULL");
  if (d->num_seqs < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->head_dim < 1)
    return fail(QSA_ERR_INVALID_ARG, "sizes must be >= 1 (B=%d Hq=%d Hkv=%d D=%d)", d->num_seqs,
                d->num_q_heads, d->num_kv_heads, d->head_dim);
  if (d->num_seqs > kMaxGridDim)
    return fail(QSA_ERR_UNSUPPORTED, "num_seqs %d > %d", d->num_seqs, kMaxGridDim);
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(QSA_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d",
                d->num_q_heads, d->num_kv_heads);
  if (d->page_size != 16) return fail(QSA_ERR_UNSUPPORTED, "page_size %d (only 16)", d->page_size);
  if (d->dtype != QSA_BF16 && d->dtype != QSA_F32)
    return fail(QSA_ERR_INVALID_ARG, "unknown dtype %d", d->dtype);
  if (!((d->dtype == QSA_BF16 && d->head_dim == 128) || (d->dtype == QSA_F32 && d->head_dim == 64)))
    return fail(QSA_ERR_UNSUPPORTED, "head_dim %d with dtype %d (built: bf16/128, f32/64)",
                d->head_dim, d->dtype);
  const int g = d->num_q_heads / d->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(QSA_ERR_UNSUPPORTED, "group size %d (built: 1, 2, 4, 8)", g);
  return QSA_OK;
}

qsa_status check_kv(const qsa_dims* d, const qsa_paged_kv* kv, bool need_v, int* max_pages) {
  if (kv == nullptr) return fail(QSA_ERR_INVALID_ARG, "kv is NULL");
  if (kv->k_pool == nullptr || (need_v && kv->v_pool == nullptr))
    return fail(QSA_ERR_INVALID_ARG, "k_pool/v_pool is NULL");
  if (kv->page_indptr == nullptr || kv->page_indices == nullptr || kv->seq_lens == nullptr ||
      kv->seq_lens_host == nullptr)
    return fail(QSA_ERR_INVALID_ARG, "page table or seq_lens pointer is NULL");
  if (kv->num_phys_pages < 1) return fail(QSA_ERR_INVALID_ARG, "num_phys_pages must be >= 1");
  int mx = 0;
  for (int b = 0; b < d->num_seqs; ++b) {
    const int L = kv->seq_lens_host[b];
    if (L < 1) return fail(QSA_ERR_INVALID_ARG, "seq_lens[%d] = %d (must be >= 1)", b, L);
    mx = std::max(mx, pages_of(L));
  }
  *max_pages = mx;
  return QSA_OK;
}

qsa::LaunchCommon common(const qsa_dims* d, const qsa_paged_kv* kv) {
  qsa::LaunchCommon c;
  c.B = d->num_seqs;
  c.Hq = d->num_q_heads;
  c.Hkv = d->num_kv_heads;
  c.D = d->head_dim;
  c.G = c.Hq / c.Hkv;
  c.bf16 = d->dtype == QSA_BF16;
  if (kv != nullptr) {
    c.k_pool = kv->k_pool;
    c.v_pool = kv->v_pool;
    c.num_phys = kv->num_phys_pages;
    c.page_indptr = kv->page_indptr;
    c.page_indices = kv->page_indices;
    c.seq_lens = kv->seq_lens;
  }
  return c;
}

// Compute units of the current device (queried once per device).
int device_cus() {
  static std::atomic<int> cus[64];  // per device, 0 until first asked (threads may ask at once)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cus[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// 4-wave workgroups that run at once: two per CU (two waves per SIMD).
int target_units() { return 2 * device_cus(); }

// Pages per unit: a multiple of 4 (one quarter per wave) sized so that the
// rows' pages fill about one unit per CU; counts per (b, h) row are min(k,
// n_b) (every page when k <= 0). Capped at 192 (48 pages per wave; the
// kernel takes up to 256). (One unit per CU measured faster than two on the
// short lists where units fit one round: 53.6 vs 54.6 us for the 8K-token,
// top-153 step's split path; one per two CUs was slower, 57.8 us.)
qsa::DecodePlan make_plan(const qsa_dims* d, const int32_t* lens, int32_t k) {
  qsa::DecodePlan plan;
  long long total = 0;
  int maxc = 0;
  for (int b = 0; b < d->num_seqs; ++b) {
    int c = pages_of(lens[b]);
    if (k > 0) c = std::min(c, (int)k);
    maxc = std::max(maxc, c);
    total += (long long)d->num_kv_heads * c;
  }
  const long long per = (total + device_cus() - 1) / device_cus();
  // (long rows: 192-256 pages per unit measured fastest; each unit start
  // and end costs a few microseconds, which smaller units pay more often,
  // while larger ones leave a longer tail in the last round)
  int chunk = (int)std::min<long long>(192, std::max<long long>(4, (per + 3) / 4 * 4));
  plan.chunk = chunk;
  plan.max_units = (maxc + chunk - 1) / chunk;
  // Stream split when the units would take more than one round of
  // workgroups (many short rows, or long rows cut into many units): there
  // its equal per-wave shares avoid the rounds' restarts and uneven ends.
  // Within one round the units' shorter start (one level of independent
  // loads, one combined partial per unit) measured faster.
  long long unit_count = 0;
  for (int b = 0; b < d->num_seqs; ++b) {
    int c = pages_of(lens[b]);
    if (k > 0) c = std::min(c, (int)k);
    unit_count += (long long)d->num_kv_heads * ((c + chunk - 1) / chunk);
  }
  const int g = d->num_q_heads / d->num_kv_heads;
  if (d->dtype == QSA_BF16 && g >= 4 && d->num_seqs <= qsa::kStreamMaxB &&
      unit_count > target_units()) {
    // One wave per (total / waves) pages, at least kStreamMinPages each, two
    // 4-wave workgroups per CU at most.
    constexpr long long kStreamMinPages = 4;
    const long long wgs = std::max<long long>(
        1, std::min<long long>(target_units(), (total + 4 * kStreamMinPages - 1) / (4 * kStreamMinPages)));
    plan.stream = true;
    plan.waves = (int)(4 * wgs);
    plan.chunk = (int)((total + plan.waves - 1) / plan.waves);
    const long long per_wave = std::max<long long>(1, total / plan.waves);
    plan.max_units = (int)std::min<long long>(plan.waves, (maxc + per_wave - 1) / per_wave + 1);
  }
  return plan;
}

// The decode grid is (Hkv, B, units per row): a row may need at most
// kMaxGridDim units.
qsa_status check_plan(const qsa::DecodePlan& p) {
  if (p.max_units > kMaxGridDim)
    return fail(QSA_ERR_UNSUPPORTED, "a row needs %d decode units of %d pages (at most %d)", p.max_units,
                p.chunk, kMaxGridDim);
  return QSA_OK;
}

DecodeWs decode_ws(const qsa_dims* d, const qsa::DecodePlan& plan) {
  const size_t rows = (size_t)d->num_seqs * d->num_kv_heads;
  const size_t slots = plan.stream ? (size_t)plan.waves + rows : rows * plan.max_units;
  const int g = d->num_q_heads / d->num_kv_heads;
  DecodeWs w;
  w.o_bytes = slots * g * d->head_dim * sizeof(float);
  w.ml_bytes = slots * g * 2 * sizeof(float);
  w.rs_bytes = plan.stream ? rows * 2 * sizeof(int) : 0;
  return w;
}

qsa::Partials carve(void* ws, const DecodeWs& w) {
  char* base = static_cast<char*>(ws);
  qsa::Partials p;
  p.o = reinterpret_cast<float*>(base);
  p.ml = reinterpret_cast<float*>(base + align_up(w.o_bytes));
  if (w.rs_bytes > 0) p.row_slots = reinterpret_cast<int*>(base + align_up(w.o_bytes) + align_up(w.ml_bytes));
  return p;
}

constexpr int kPrefixSplitTokens = 512;  // prefix tokens per cascade split
// Splits of the one-launch selective cascade: its 4-wave prefix workgroups
// share the CUs with the suffix rows, and the merge reads every split's
// partials (512-token splits: c5 step 78.0 us; 1024: 71.6 us; 768: 78.4 us).
constexpr int kOverlapSplitTokens = 1024;

int prefix_splits(int prefix_len, int tokens = kPrefixSplitTokens) {
  return std::max(1, (prefix_len + tokens - 1) / tokens);
}

size_t prefix_ws_bytes(const qsa_dims* d, int prefix_len, int tokens = kPrefixSplitTokens) {
  const size_t rows = (size_t)d->num_kv_heads * prefix_splits(prefix_len, tokens) * d->num_q_heads /
                      d->num_kv_heads * d->num_seqs;
  return align_up(rows * d->head_dim * sizeof(float)) + align_up(rows * 2 * sizeof(float));
}

// Rows the fused path wants before it is chosen automatically: with one
// 8-wave workgroup per row, 64 rows already keep HBM busy at ~5.4 TB/s in a
// plain tile-streaming test and 128 reach ~6.9 TB/s, while the split path
// pays three more launches.
constexpr int kFusedMinRows = 64;

bool fused_supported(int max_pages, int k) {
  return max_pages <= qsa::kRowMaxPages && std::min(k, max_pages) <= qsa::kRowMaxSelect;
}

// Rows the one-wave-per-row kernel takes (bf16 groups of 4 or 8 heads, the
// bound scorer, at most 64 pages per row).
bool short_rows_supported(const qsa_dims* d, int max_pages, bool centroid) {
  const int g = d->num_q_heads / d->num_kv_heads;
  return d->dtype == QSA_BF16 && d->head_dim == 128 && (g == 4 || g == 8) && !centroid &&
         max_pages <= qsa::kShortMaxPages;
}

qsa_path choose_path(const qsa_dims* d, int max_pages, int k, int32_t path) {
  if (path != QSA_PATH_AUTO) return path == QSA_PATH_FUSED ? QSA_PATH_FUSED : QSA_PATH_SPLIT;
  const long long rows = (long long)d->num_seqs * d->num_kv_heads;
  return (fused_supported(max_pages, k) && rows >= kFusedMinRows) ? QSA_PATH_FUSED : QSA_PATH_SPLIT;
}

// Split-path workspace of qsa_sparse_decode: [group scores][sel][sel_count]
// [decode partials], each region 256-byte aligned.
struct SparseWs {
  size_t gs = 0, sel = 0, cnt = 0;
  DecodeWs dec;
  size_t total() const { return align_up(gs) + align_up(sel) + align_up(cnt) + dec.total(); }
};

// The fused path's exchange: with at most half as many (b, h) rows as CUs
// two workgroups share each row and merge their partial results through the
// workspace (per-row arrival counters, then per (row, part) G * (D + 2)
// floats). A workgroup fills a CU (its VGPRs allow two waves per SIMD), so
// with more rows the pairs would run in two rounds: at 136 to 248 rows of
// c2's shape one workgroup per row measured 47-69 us against 66-80 us.
bool fused_pair_split(const qsa_dims* d) { return 2 * d->num_seqs * d->num_kv_heads <= device_cus(); }

struct PairWs {
  size_t counters = 0, partials = 0;
  size_t total() const { return counters == 0 ? 0 : align_up(counters) + align_up(partials); }
};

PairWs pair_ws(const qsa_dims* d) {
  PairWs w;
  if (!fused_pair_split(d)) return w;
  const size_t rows = (size_t)d->num_seqs * d->num_kv_heads;
  const size_t g = (size_t)(d->num_q_heads / d->num_kv_heads);
  w.counters = rows * sizeof(unsigned int);
  w.partials = rows * 2 * g * (d->head_dim + 2) * sizeof(float);
  return w;
}

SparseWs sparse_ws(const qsa_dims* d, const int32_t* lens, int stride, int k) {
  const size_t rows = (size_t)d->num_seqs * d->num_kv_heads;
  SparseWs w;
  w.gs = rows * stride * sizeof(float);
  w.sel = rows * k * sizeof(int32_t);
  w.cnt = rows * sizeof(int32_t);
  w.dec = decode_ws(d, make_plan(d, lens, k));
  return w;
}

// ---- checked mode ----------------------------------------------------------
// Every kernel that skips a page because a table or selection entry is out
// of range can OR a bit into a device error word. In checked mode each entry
// point clears the word before its launches (with a one-thread kernel),
// passes it to them, then waits for the stream and reads it back: a set bit
// turns the call's status into QSA_ERR_DEVICE. Unchecked (the default), the
// kernels get no word and skip silently.

namespace {

// The error word: one per device (each GPU the library runs on holds its own
// copy, at its own address).
__device__ unsigned int g_err_word;

__global__ void clear_word_kernel(unsigned int* w) {
  if (threadIdx.x == 0) *w = 0u;
}

std::atomic<int> g_checked{-1};  // -1: not read from the environment yet

constexpr int kMaxDevices = 64;
std::mutex g_word_mu;
unsigned int* g_word_ptr[kMaxDevices] = {nullptr};

}  // namespace

bool checked_mode() {
  int v = g_checked.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = std::getenv("QSA_CHECKED");
    v = (e != nullptr && *e != '\0' && std::strcmp(e, "0") != 0) ? 1 : 0;
    int expect = -1;
    g_checked.compare_exchange_strong(expect, v);
    v = g_checked.load(std::memory_order_relaxed);
  }
  return v == 1;
}

void set_checked_mode(bool on) { g_checked.store(on ? 1 : 0); }

qsa_status Checked::begin(qsa::LaunchCommon& c, hipStream_t stream) {
  word_ = nullptr;
  if (!checked_mode()) return QSA_OK;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "checked mode: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(QSA_ERR_UNSUPPORTED, "checked mode: device %d (at most %d devices)", dev, kMaxDevices);
  {
    std::lock_guard<std::mutex> lock(g_word_mu);
    if (g_word_ptr[dev] == nullptr) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_err_word));
      if (e != hipSuccess) return device_status(e, "checked mode: hipGetSymbolAddress");
      g_word_ptr[dev] = static_cast<unsigned int*>(p);
    }
    word_ = g_word_ptr[dev];
  }
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(64), 0, stream, word_);
  e = hipGetLastError();
  if (e != hipSuccess) {
    word_ = nullptr;
    return device_status(e, "checked mode: clearing the error word");
  }
  c.err = word_;
  return QSA_OK;
}

qsa_status Checked::end(qsa_status s, hipStream_t stream) {
  if (word_ == nullptr || s != QSA_OK) return s;
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return device_status(e, "checked mode: hipStreamSynchronize");
  unsigned int v = 0;
  e = hipMemcpy(&v, word_, sizeof(v), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return device_status(e, "checked mode: reading the error word");
  if (v == 0u) return ok();
  std::string what;
  if (v & qsa::kErrPhys) what += " a page table entry outside [0, num_phys_pages);";
  if (v & qsa::kErrSel) what += " a selected logical page outside [0, n_b);";
  if (v & qsa::kErrCount) what += " a sel_count entry outside [1, min(k, n_b)];";
  if (v == qsa::kErrExchange)
    return fail(QSA_ERR_DEVICE,
                "device check (word 0x%x): a fused-path row counter in the workspace was neither 0 nor 1 "
                "(the workspace was not zeroed before its first use); the outputs are not valid", v);
  if (v & qsa::kErrExchange)
    what += " a fused-path row counter in the workspace was neither 0 nor 1 (not zeroed before first use);";
  return fail(QSA_ERR_DEVICE, "device range check (word 0x%x):%s the entries were skipped", v,
              what.c_str());
}

}  // namespace host
}  // namespace qsa

using namespace qsa::host;

extern "C" {

int32_t qsa_version(void) { return 1; }

void qsa_set_checked(int32_t on) { set_checked_mode(on != 0); }

int32_t qsa_get_checked(void) { return checked_mode() ? 1 : 0; }

const char* qsa_status_string(int32_t s) {
  switch (s) {
    case QSA_OK: return "ok";
    case QSA_ERR_INVALID_ARG: return "invalid argument";
    case QSA_ERR_UNSUPPORTED: return "unsupported shape";
    case QSA_ERR_WORKSPACE: return "workspace too small";
    case QSA_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* qsa_last_error(void) { return g_last_error.c_str(); }

int32_t qsa_budget_pages(int32_t budget_tokens, int32_t page_size) {
  if (budget_tokens <= 0 || page_size <= 0) return 0;
  return budget_tokens / page_size;
}

qsa_status qsa_build_page_meta(const qsa_dims* dims, const qsa_paged_kv* kv, int32_t tail_pages,
                               void* meta, int32_t stride, hipStream_t stream) {
  qsa_status s = check_dims(dims);
  if (s != QSA_OK) return s;
  int max_pages = 0;
  if ((s = check_kv(dims, kv, false, &max_pages)) != QSA_OK) return s;
  if (meta == nullptr) return fail(QSA_ERR_INVALID_ARG, "meta is NULL");
  if (tail_pages < 0) return fail(QSA_ERR_INVALID_ARG, "tail_pages %d < 0", tail_pages);
  if (stride < max_pages)
    return fail(QSA_ERR_INVALID_ARG, "stride %d < longest sequence's page count %d", stride,
                max_pages);
  qsa::LaunchCommon c = common(dims, kv);
  Checked chk;
  if ((s = chk.begin(c, stream)) != QSA_OK) return s;
  return chk.end(device_status(qsa::launch_build_meta(c, max_pages, tail_pages, meta, stride, stream),
                               "build_page_meta launch"),
                 stream);
}

qsa_status qsa_score_pages(const qsa_dims* dims, const void* q, const qsa_paged_kv* kv, void* meta,
                           float* group_scores, float* head_scores, int32_t stride,
                           int32_t refresh_tail, hipStream_t stream) {
  qsa_status s = check_dims(dims);
  if (s != QSA_OK) return s;
  int max_pages = 0;
  if ((s = check_kv(dims, kv, false, &max_pages)) != QSA_OK) return s;
  if (q == nullptr || meta == nullptr || group_scores == nullptr)
    return fail(QSA_ERR_INVALID_ARG, "q/meta/group_scores is NULL");
  if (stride < max_pages)
    return fail(QSA_ERR_INVALID_ARG, "stride %d < longest sequence's page count %d", stride,
                max_pages);
  if (refresh_tail != 0 && refresh_tail != 1)
    return fail(QSA_ERR_INVALID_ARG, "refresh_tail %d (0 or 1)", refresh_tail);
  qsa::LaunchCommon c = common(dims, kv);
  Checked chk;
  if ((s = chk.begin(c, stream)) != QSA_OK) return s;
  return chk.end(device_status(qsa::launch_score(c, q, meta, refresh_tail, group_scores, head_scores,
                                                 stride, stream),
                               "score_pages launch"),
                 stream);
}

qsa_status qsa_build_page_centroids(const qsa_dims* dims, const qsa_paged_kv* kv,
                                   int32_t tail_pages, void* cent, int32_t stride,
                                   hipStream_t stream) {
  qsa_status s = check_dims(dims);
  if (s != QSA_OK) return s;
  int max_pages = 0;
  if ((s = check_kv(dims, kv, false, &max_pages)) != QSA_OK) return s;
  if (cent == nullptr) return fail(QSA_ERR_INVALID_ARG, "cent is NULL");
  if (tail_pages < 0) return fail(QSA_ERR_INVALID_ARG, "tail_pages %d < 0", tail_pages);
  if (stride < max_pages)
    return fail(QSA_ERR_INVALID_ARG, "stride %d < longest sequence's page count %d", stride,
                max_pages);
  qsa::LaunchCommon c = common(dims, kv);
  Checked chk;
  if ((s = chk.begin(c, stream)) != QSA_OK) return s;
  return chk.end(
      device_status(qsa::launch_build_centroids(c, max_pages, tail_pages, cent, stride, stream),
                    "build_page_centroids launch"),
      stream);
}

qsa_status qsa_score_pages_centroid(const qsa_dims* dims, const void* q, const qsa_paged_kv* kv,
                                    void* cent, float* group_scores, float* head_scores,
                                    int32_t stride, int32_t refresh_tail, hipStream_t stream) {
  qsa_status s = check_dims(dims);
  if (s != QSA_OK) return s;
  int max_pages = 0;
  if ((s = check_kv(dims, kv, false, &max_pages)) != QSA_OK) return s;
  if (q == nullptr || cent == nullptr || group_scores == nullptr)
    return fail(QSA_ERR_INVALID_ARG, "q/cent/group_scores is NULL");
  if (stride < max_pages)
    return fail(QSA_ERR_INVALID_ARG, "stride %d < longest sequence's page count %d", stride,
                max_pages);
  if (refresh_tail != 0 && refresh_tail != 1)
    return fail(QSA_ERR_INVALID_ARG, "refresh_tail %d (0 or 1)", refresh_tail);
  qsa::LaunchCommon c = common(dims, kv);
  Checked chk;
  if ((s = chk.begin(c, stream)) != QSA_OK) return s;
  return chk.end(device_status(qsa::launch_score_centroid(c, q, cent, refresh_tail, group_scores,
                                                          head_scores, stride, stream),
                               "score_pages_centroid launch"),
                 stream);
}

size_t qsa_topk_workspace_size(const qsa_dims* dims, int32_t max_pages, int32_t k) {
  (void)dims;
  (void)max_pages;
  (void)k;
  return 0;
}

qsa_status qsa_topk_pages(const qsa_dims* dims, const qsa_paged_kv* kv, const float* group_scores,
                          int32_t stride, int32_t k, int32_t* sel, int32_t* sel_count,
                          int32_t* sel_phys, void* ws, size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  qsa_status s = check_dims(dims);
  if (s != QSA_OK) return s;
  int max_pages = 0;
  if ((s = check_kv(dims, kv, false, &max_pages)) != QSA_OK) return s;
  if (group_scores == nullptr || sel == nullptr || sel_count == nullptr)
    return fail(QSA_ERR_INVALID_ARG, "group_scores/sel/sel_count is NULL");
  if (k < 1) return fail(QSA_ERR_INVALID_ARG, "k = %d (must be >= 1)", k);
  if (stride > qsa::kTopkMaxPages)
    return fail(QSA_ERR_UNSUPPORTED, "stride %d > %d pages per row", stride, qsa::kTopkMaxPages);
  if (stride < max_pages)
    return fail(QSA_ERR_INVALID_ARG, "stride %d < longest sequence's page count %d", stride,
                max_pages);
  return device_status(
      qsa::launch_topk(common(dims, kv), group_scores, stride, k, sel, sel_count, sel_phys, stream),
      "topk_pages launch");
}

qsa_status qsa_topk_pages_approx(const qsa_dims* dims, const qsa_paged_kv* kv,
                                 const float* group_scores, int32_t stride, int32_t k,
                                 int32_t digit_bits, int32_t min_confident,
                                 const uint32_t* row_rand, int32_t* sel, int32_t* sel_count,
                                 int32_t* sel_phys, int32_t* passes, hipStream_t stream) {
  qsa_status s = check_dims(dims);
  if (s != QSA_OK) return s;
  int max_pages = 0;
  if ((s = check_kv(dims, kv, false, &max_pages)) != QSA_OK) return s;
  if (group_scores == nullptr || sel == nullptr || sel_count == nullptr || row_rand == nullptr)
    return fail(QSA_ERR_INVALID_ARG, "group_scores/row_rand/sel/sel_count is NULL");
  if (k < 1) return fail(QSA_ERR_INVALID_ARG, "k = %d (must be >= 1)", k);
  if (digit_bits < 4 || digit_bits > 13)
    return fail(QSA_ERR_INVALID_ARG, "digit_bits = %d (must be in 4..13)", digit_bits);
  if (min_confident < 0)
    return fail(QSA_ERR_INVALID_ARG, "min_confident = %d (must be >= 0)", min_confident);
  if (stride > qsa::kTopkMaxPages)
    return fail(QSA_ERR_UNSUPPORTED, "stride %d > %d pages per row", stride, qsa::kTopkMaxPages);
  if (stride < max_pages)
    return fail(QSA_ERR_INVALID_ARG, "stride %d < longest sequence's page count %d", stride,
                max_pages);
  return device_status(qsa::launch_topk_approx(common(dims, kv), group_scores, stride, k,
                                               digit_bits, min_confident, row_rand, sel,
                                               sel_count, sel_phys, passes, stream),
                       "topk_pages_approx launch");
}

qsa_status qsa_decode_plan(const qsa_dims* dims, const int32_t* seq_lens_host, int32_t k,
                           int32_t* chunk_pages, int32_t* max_units, int32_t* stream) {
  qsa_status s = check_dims(dims);
  if (s != QSA_OK) return s;
  if (seq_lens_host == nullptr || chunk_pages == nullptr || max_units == nullptr)
    return fail(QSA_ERR_INVALID_ARG, "NULL argument");
  for (int b = 0; b < dims->num_seqs; ++b)
    if (seq_lens_host[b] < 1) return fail(QSA_ERR_INVALID_ARG, "seq_lens[%d] < 1", b);
  qsa::DecodePlan p = make_plan(dims, seq_lens_host, k);
  if ((s = check_plan(p)) != QSA_OK) return s;
  *chunk_pages = p.chunk;
  *max_units = p.max_units;
  if (stream != nullptr) *stream = p.stream ? 1 : 0;
  return ok();
}

size_t qsa_decode_workspace_size(const qsa_dims* dims, const int32_t* seq_lens_host, int32_t k) {
  if (check_dims(dims) != QSA_OK || seq_lens_host == nullptr) return 0;
  for (int b = 0; b < dims->num_seqs; ++b)
    if (seq_lens_host[b] < 1) return 0;
  return decode_ws(dims, make_plan(dims, seq_lens_host, k)).total();
}

qsa_status qsa_paged_decode(const qsa_dims* dims, const void* q, const qsa_paged_kv* kv,
                            const int32_t* sel, const int32_t* sel_count, int32_t k, float sm_scale,
                            float* out, float* lse, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  qsa_status s = check_dims(dims);
  if (s != QSA_OK) return s;
  int max_pages = 0;
  if ((s = check_kv(dims, kv, true, &max_pages)) != QSA_OK) return s;
  if (q == nullptr || out == nullptr) return fail(QSA_ERR_INVALID_ARG, "q/out is NULL");
  if (sel != nullptr && (sel_count == nullptr || k < 1))
    return fail(QSA_ERR_INVALID_ARG, "sel given without sel_count or with k < 1");
  if (!std::isfinite(sm_scale)) return fail(QSA_ERR_INVALID_ARG, "sm_scale is not finite");
  const int32_t kk = sel != nullptr ? k : 0;
  const qsa::DecodePlan plan = make_plan(dims, kv->seq_lens_host, kk);
  if ((s = check_plan(plan)) != QSA_OK) return s;
  const DecodeWs w = decode_ws(dims, plan);
  if (ws_bytes < w.total() || (w.total() > 0 && ws == nullptr))
    return fail(QSA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, w.total());
  const qsa::Partials part = carve(ws, w);
  qsa::LaunchCommon c = common(dims, kv);
  Checked chk;
  if ((s = chk.begin(c, stream)) != QSA_OK) return s;
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  return chk.end(device_status(qsa::launch_decode(c, q, sel, sel_count, kk, scale_log2, plan, part,
                                                  qsa::Partials{}, 0, out, lse, stream),
                               "paged_decode launch"),
                 stream);
}

size_t qsa_cascade_workspace_size(const qsa_dims* dims, int32_t prefix_len,
                                  const int32_t* suffix_lens_host, int32_t k) {
  if (check_dims(dims) != QSA_OK || suffix_lens_host == nullptr || prefix_len < 1) return 0;
  for (int b = 0; b < dims->num_seqs; ++b)
    if (suffix_lens_host[b] < 1) return 0;
  return decode_ws(dims, make_plan(dims, suffix_lens_host, k)).total() +
         prefix_ws_bytes(dims, prefix_len);
}

qsa_status qsa_cascade_decode(const qsa_dims* dims, const void* q, const int32_t* prefix_pages,
                              int32_t prefix_len, const qsa_paged_kv* kv, const int32_t* sel,
                              const int32_t* sel_count, int32_t k, float sm_scale, float* out,
                              float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  qsa_status s = check_dims(dims);
  if (s != QSA_OK) return s;
  if (dims->dtype != QSA_BF16)
    return fail(QSA_ERR_UNSUPPORTED, "cascade decode is built for bf16 / head_dim 128 only");
  int max_pages = 0;
  if ((s = check_kv(dims, kv, true, &max_pages)) != QSA_OK) return s;
  if (q == nullptr || out == nullptr || prefix_pages == nullptr)
    return fail(QSA_ERR_INVALID_ARG, "q/out/prefix_pages is NULL");
  if (prefix_len < 1) return fail(QSA_ERR_INVALID_ARG, "prefix_len %d < 1", prefix_len);
  if (sel != nullptr && (sel_count == nullptr || k < 1))
    return fail(QSA_ERR_INVALID_ARG, "sel given without sel_count or with k < 1");
  if (!std::isfinite(sm_scale)) return fail(QSA_ERR_INVALID_ARG, "sm_scale is not finite");
  const int32_t kk = sel != nullptr ? k : 0;
  const qsa::DecodePlan plan = make_plan(dims, kv->seq_lens_host, kk);
  if ((s = check_plan(plan)) != QSA_OK) return s;
  const DecodeWs w = decode_ws(dims, plan);
  const size_t need = w.total() + prefix_ws_bytes(dims, prefix_len);
  if (ws_bytes < need || ws == nullptr)
    return fail(QSA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  char* base = static_cast<char*>(ws);
  const qsa::Partials part = carve(ws, w);
  const int nsplit = prefix_splits(prefix_len);
  const size_t rows = (size_t)dims->num_kv_heads * nsplit * (dims->num_q_heads / dims->num_kv_heads) *
                      dims->num_seqs;
  qsa::Partials pre;
  pre.o = reinterpret_cast<float*>(base + w.total());
  pre.ml = reinterpret_cast<float*>(base + w.total() + align_up(rows * dims->head_dim * sizeof(float)));
  qsa::LaunchCommon c = common(dims, kv);
  Checked chk;
  if ((s = chk.begin(c, stream)) != QSA_OK) return s;
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  hipError_t e = qsa::launch_cascade_prefix(c, q, prefix_pages, prefix_len, nsplit, scale_log2, pre,
                                            stream);
  if (e != hipSuccess) return device_status(e, "cascade prefix launch");
  e = qsa::launch_decode(c, q, sel, sel_count, kk, scale_log2, plan, part, pre, nsplit, out, lse,
                         stream);
  return chk.end(device_status(e, "cascade suffix launch"), stream);
}

qsa_status qsa_sparse_decode_path(const qsa_dims* dims, const int32_t* seq_lens_host,
                                  int32_t stride, int32_t k, int32_t path, qsa_path* chosen) {
  qsa_status s = check_dims(dims);
  if (s != QSA_OK) return s;
  if (seq_lens_host == nullptr || chosen == nullptr) return fail(QSA_ERR_INVALID_ARG, "NULL argument");
  if (path != QSA_PATH_AUTO && path != QSA_PATH_FUSED && path != QSA_PATH_SPLIT)
    return fail(QSA_ERR_INVALID_ARG, "unknown path %d", path);
  if (k < 1) return fail(QSA_ERR_INVALID_ARG, "k = %d (must be >= 1)", k);
  int max_pages = 0;
  for (int b = 0; b < dims->num_seqs; ++b) {
    if (seq_lens_host[b] < 1) return fail(QSA_ERR_INVALID_ARG, "seq_lens[%d] < 1", b);
    max_pages = std::max(max_pages, pages_of(seq_lens_host[b]));
  }
  if (stride < max_pages)
    return fail(QSA_ERR_INVALID_ARG, "stride %d < longest sequence's page count %d", stride,
                max_pages);
  const qsa_path p = choose_path(dims, max_pages, k, path);
  if (p == QSA_PATH_FUSED && !fused_supported(max_pages, k))
    return fail(QSA_ERR_UNSUPPORTED,
                "fused path: %d pages per row (max %d) and %d selected (max %d)", max_pages,
                qsa::kRowMaxPages, std::min(k, max_pages), qsa::kRowMaxSelect);
  if (p == QSA_PATH_SPLIT && stride > qsa::kTopkMaxPages)
    return fail(QSA_ERR_UNSUPPORTED, "stride %d > %d pages per row", stride, qsa::kTopkMaxPages);
  *chosen = p;
  return ok();
}

size_t qsa_sparse_decode_workspace_size(const qsa_dims* dims, const int32_t* seq_lens_host,
                                        int32_t stride, int32_t k, int32_t path) {
  qsa_path chosen;
  if (qsa_sparse_decode_path(dims, seq_lens_host, stride, k, path, &chosen) != QSA_OK) return 0;
  if (chosen == QSA_PATH_FUSED) return pair_ws(dims).total();
  return sparse_ws(dims, seq_lens_host, stride, k).total();
}

}  // extern "C"

namespace {

// One sparse decode step with the bound scorer or the centroid scorer (meta
// then holds centroid rows).
qsa_status sparse_decode_impl(const qsa_dims* dims, const void* q, const qsa_paged_kv* kv,
                              void* meta, int32_t stride, int32_t refresh_tail, int32_t k,
                              float sm_scale, float* out, float* lse, float* group_scores,
                              int32_t* sel, int32_t* sel_count, int32_t path, void* ws,
                              size_t ws_bytes, bool centroid, hipStream_t stream) {
  qsa_status s = check_dims(dims);
  if (s != QSA_OK) return s;
  int max_pages = 0;
  if ((s = check_kv(dims, kv, true, &max_pages)) != QSA_OK) return s;
  if (q == nullptr || meta == nullptr || out == nullptr)
    return fail(QSA_ERR_INVALID_ARG, "q/meta/out is NULL");
  if (refresh_tail != 0 && refresh_tail != 1)
    return fail(QSA_ERR_INVALID_ARG, "refresh_tail %d (0 or 1)", refresh_tail);
  if (!std::isfinite(sm_scale)) return fail(QSA_ERR_INVALID_ARG, "sm_scale is not finite");
  qsa_path chosen;
  if ((s = qsa_sparse_decode_path(dims, kv->seq_lens_host, stride, k, path, &chosen)) != QSA_OK)
    return s;
  qsa::LaunchCommon c = common(dims, kv);
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  Checked chk;
  if (chosen == QSA_PATH_FUSED && short_rows_supported(dims, max_pages, centroid)) {
    // rows of at most 64 pages: one wave per row
    if ((s = chk.begin(c, stream)) != QSA_OK) return s;
    return chk.end(device_status(qsa::launch_short_rows(c, q, meta, stride, refresh_tail, k, scale_log2,
                                                        qsa::Partials{}, 0, out, lse, group_scores, sel,
                                                        sel_count, stream),
                                 "sparse_decode (fused, short rows) launch"),
                   stream);
  }
  if (chosen == QSA_PATH_FUSED) {
    // at most half as many rows as CUs: two workgroups per row, each
    // attending over half of the selected pages, merged through the
    // workspace's exchange
    qsa::RowExchange x;
    const PairWs pw = pair_ws(dims);
    if (pw.total() > 0) {
      if (ws == nullptr || ws_bytes < pw.total())
        return fail(QSA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, pw.total());
      if (reinterpret_cast<uintptr_t>(ws) % 16 != 0)
        return fail(QSA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
      x.counters = static_cast<unsigned int*>(ws);
      x.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(pw.counters));
    }
    if ((s = chk.begin(c, stream)) != QSA_OK) return s;
    return chk.end(device_status(qsa::launch_sparse_row(c, q, meta, stride, refresh_tail, k,
                                                        scale_log2, x, centroid, out, lse,
                                                        group_scores, sel, sel_count, stream),
                                 "sparse_decode (fused) launch"),
                   stream);
  }
  const SparseWs w = sparse_ws(dims, kv->seq_lens_host, stride, k);
  if (ws_bytes < w.total() || ws == nullptr)
    return fail(QSA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, w.total());
  if ((s = chk.begin(c, stream)) != QSA_OK) return s;
  char* base = static_cast<char*>(ws);
  float* gs = reinterpret_cast<float*>(base);
  base += align_up(w.gs);
  int32_t* sl = reinterpret_cast<int32_t*>(base);
  base += align_up(w.sel);
  int32_t* cn = reinterpret_cast<int32_t*>(base);
  base += align_up(w.cnt);
  if (group_scores != nullptr) gs = group_scores;
  if (sel != nullptr) sl = sel;
  if (sel_count != nullptr) cn = sel_count;
  hipError_t e = centroid
                    ? qsa::launch_score_centroid(c, q, meta, refresh_tail, gs, nullptr, stride, stream)
                    : qsa::launch_score(c, q, meta, refresh_tail, gs, nullptr, stride, stream);
  if (e != hipSuccess) return device_status(e, "sparse_decode score launch");
  e = qsa::launch_topk(c, gs, stride, k, sl, cn, nullptr, stream);
  if (e != hipSuccess) return device_status(e, "sparse_decode top-K launch");
  const qsa::DecodePlan plan = make_plan(dims, kv->seq_lens_host, k);
  const qsa::Partials part = carve(base, w.dec);
  return chk.end(device_status(qsa::launch_decode(c, q, sl, cn, k, scale_log2, plan, part,
                                                  qsa::Partials{}, 0, out, lse, stream),
                               "sparse_decode decode launch"),
                 stream);
}

}  // namespace

extern "C" {

qsa_status qsa_sparse_decode(const qsa_dims* dims, const void* q, const qsa_paged_kv* kv, void* meta,
                             int32_t stride, int32_t refresh_tail, int32_t k, float sm_scale,
                             float* out, float* lse, float* group_scores, int32_t* sel,
                             int32_t* sel_count, int32_t path, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  return sparse_decode_impl(dims, q, kv, meta, stride, refresh_tail, k, sm_scale, out, lse,
                            group_scores, sel, sel_count, path, ws, ws_bytes, false, stream);
}

qsa_status qsa_sparse_decode_centroid(const qsa_dims* dims, const void* q, const qsa_paged_kv* kv,
                                      void* cent, int32_t stride, int32_t refresh_tail, int32_t k,
                                      float sm_scale, float* out, float* lse, float* group_scores,
                                      int32_t* sel, int32_t* sel_count, int32_t path, void* ws,
                                      size_t ws_bytes, hipStream_t stream) {
  return sparse_decode_impl(dims, q, kv, cent, stride, refresh_tail, k, sm_scale, out, lse,
                            group_scores, sel, sel_count, path, ws, ws_bytes, true, stream);
}

}  // extern "C"

namespace {

// The prefix partials of a cascade at the start of `base`.
qsa::Partials carve_prefix(char* base, const qsa_dims* d, int prefix_len, int tokens = kPrefixSplitTokens) {
  const size_t rows = (size_t)d->num_kv_heads * prefix_splits(prefix_len, tokens) *
                      (d->num_q_heads / d->num_kv_heads) * d->num_seqs;
  qsa::Partials pre;
  pre.o = reinterpret_cast<float*>(base);
  pre.ml = reinterpret_cast<float*>(base + align_up(rows * d->head_dim * sizeof(float)));
  return pre;
}

// The suffix rows' unmerged partials of the one-launch form (one unit per
// (sequence, KV head) row: o [rows][g][D], then (max, sum) [rows][g][2]).
DecodeWs suffix_ws(const qsa_dims* d) {
  const size_t rows = (size_t)d->num_seqs * d->num_kv_heads;
  const int g = d->num_q_heads / d->num_kv_heads;
  DecodeWs w;
  w.o_bytes = rows * g * d->head_dim * sizeof(float);
  w.ml_bytes = rows * g * 2 * sizeof(float);
  return w;
}

// Workspace of qsa_cascade_sparse_decode: the prefix partials, then the
// suffix rows' partials (rows of one wave each) or the split path's scores,
// selection and decode partials.
size_t cascade_sparse_ws(const qsa_dims* d, int prefix_len, const int32_t* lens, int max_pages, int stride,
                         int k) {
  if (short_rows_supported(d, max_pages, false))
    return prefix_ws_bytes(d, prefix_len, kOverlapSplitTokens) + suffix_ws(d).total();
  return prefix_ws_bytes(d, prefix_len) + sparse_ws(d, lens, stride, k).total();
}

}  // namespace

extern "C" {

size_t qsa_cascade_sparse_decode_workspace_size(const qsa_dims* dims, int32_t prefix_len,
                                                const int32_t* suffix_lens_host, int32_t stride, int32_t k) {
  if (check_dims(dims) != QSA_OK || suffix_lens_host == nullptr || prefix_len < 1 || k < 1) return 0;
  int max_pages = 0;
  for (int b = 0; b < dims->num_seqs; ++b) {
    if (suffix_lens_host[b] < 1) return 0;
    max_pages = std::max(max_pages, pages_of(suffix_lens_host[b]));
  }
  if (stride < max_pages) return 0;
  return cascade_sparse_ws(dims, prefix_len, suffix_lens_host, max_pages, stride, k);
}

qsa_status qsa_cascade_sparse_decode(const qsa_dims* dims, const void* q, const int32_t* prefix_pages,
                                     int32_t prefix_len, const qsa_paged_kv* kv, void* meta, int32_t stride,
                                     int32_t refresh_tail, int32_t k, float sm_scale, float* out, float* lse,
                                     float* group_scores, int32_t* sel, int32_t* sel_count, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  qsa_status s = check_dims(dims);
  if (s != QSA_OK) return s;
  if (dims->dtype != QSA_BF16)
    return fail(QSA_ERR_UNSUPPORTED, "cascade decode is built for bf16 / head_dim 128 only");
  int max_pages = 0;
  if ((s = check_kv(dims, kv, true, &max_pages)) != QSA_OK) return s;
  if (q == nullptr || out == nullptr || prefix_pages == nullptr || meta == nullptr)
    return fail(QSA_ERR_INVALID_ARG, "q/out/prefix_pages/meta is NULL");
  if (prefix_len < 1) return fail(QSA_ERR_INVALID_ARG, "prefix_len %d < 1", prefix_len);
  if (k < 1) return fail(QSA_ERR_INVALID_ARG, "k = %d (must be >= 1)", k);
  if (refresh_tail != 0 && refresh_tail != 1)
    return fail(QSA_ERR_INVALID_ARG, "refresh_tail %d (0 or 1)", refresh_tail);
  if (!std::isfinite(sm_scale)) return fail(QSA_ERR_INVALID_ARG, "sm_scale is not finite");
  if (stride < max_pages)
    return fail(QSA_ERR_INVALID_ARG, "stride %d < longest sequence's page count %d", stride, max_pages);
  const bool short_rows = short_rows_supported(dims, max_pages, false);
  if (!short_rows && stride > qsa::kTopkMaxPages)
    return fail(QSA_ERR_UNSUPPORTED, "stride %d > %d pages per row", stride, qsa::kTopkMaxPages);
  const size_t need = cascade_sparse_ws(dims, prefix_len, kv->seq_lens_host, max_pages, stride, k);
  if (ws_bytes < need || ws == nullptr)
    return fail(QSA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  qsa::DecodePlan plan;
  if (!short_rows) {
    plan = make_plan(dims, kv->seq_lens_host, k);
    if ((s = check_plan(plan)) != QSA_OK) return s;
  }
  char* base = static_cast<char*>(ws);
  const int tokens = short_rows ? kOverlapSplitTokens : kPrefixSplitTokens;
  const qsa::Partials pre = carve_prefix(base, dims, prefix_len, tokens);
  const int nsplit = prefix_splits(prefix_len, tokens);
  qsa::LaunchCommon c = common(dims, kv);
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  Checked chk;
  if ((s = chk.begin(c, stream)) != QSA_OK) return s;
  if (short_rows) {
    // the prefix and the suffix rows in one launch, then the merge
    const qsa::Partials suf = carve(base + prefix_ws_bytes(dims, prefix_len, tokens), suffix_ws(dims));
    hipError_t e = qsa::launch_cascade_overlap(c, q, prefix_pages, prefix_len, nsplit, scale_log2, pre, meta,
                                               stride, refresh_tail, k, suf, group_scores, sel, sel_count,
                                               device_cus() / 8, stream);
    if (e != hipSuccess) return device_status(e, "cascade (prefix and suffix rows) launch");
    return chk.end(device_status(qsa::launch_merge(c, suf, 1, 1 << 30, pre, nsplit, out, lse, stream),
                                 "cascade merge launch"),
                   stream);
  }
  hipError_t e = qsa::launch_cascade_prefix(c, q, prefix_pages, prefix_len, nsplit, scale_log2, pre, stream);
  if (e != hipSuccess) return device_status(e, "cascade prefix launch");
  // long suffix rows: the separate score, top-K and split-K kernels, with
  // the prefix partials folded into the merge
  const SparseWs w = sparse_ws(dims, kv->seq_lens_host, stride, k);
  char* sb = base + prefix_ws_bytes(dims, prefix_len);
  float* gs = reinterpret_cast<float*>(sb);
  sb += align_up(w.gs);
  int32_t* sl = reinterpret_cast<int32_t*>(sb);
  sb += align_up(w.sel);
  int32_t* cn = reinterpret_cast<int32_t*>(sb);
  sb += align_up(w.cnt);
  if (group_scores != nullptr) gs = group_scores;
  if (sel != nullptr) sl = sel;
  if (sel_count != nullptr) cn = sel_count;
  e = qsa::launch_score(c, q, meta, refresh_tail, gs, nullptr, stride, stream);
  if (e != hipSuccess) return device_status(e, "cascade suffix score launch");
  e = qsa::launch_topk(c, gs, stride, k, sl, cn, nullptr, stream);
  if (e != hipSuccess) return device_status(e, "cascade suffix top-K launch");
  e = qsa::launch_decode(c, q, sl, cn, k, scale_log2, plan, carve(sb, w.dec), pre, nsplit, out, lse, stream);
  return chk.end(device_status(e, "cascade suffix decode launch"), stream);
}

}  // extern "C"
