// qsa_paged_decode for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the same
// validation, plan and kernels as qsa_paged_decode, with the split-K partial
// results in a fixed device array of this file instead of a caller
// workspace. Nothing is allocated per call.
//
// The array lives in every GPU the library runs on, for the life of the
// process. Host code never passes its name to a kernel: on the host the name
// is only a stand-in, so each device's address is looked up once
// (hipGetSymbolAddress with that device current) and kept per device.
#include <cmath>
#include <mutex>

#include "host.h"
#include "qsa.h"
#include "qsa_internal.h"

namespace {

constexpr size_t kScratchBytes = QSA_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

// This device's address of `scratch` (looked up on its first use).
qsa_status scratch_address(void** out) {
  using qsa::host::device_status;
  using qsa::host::fail;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "paged_decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(QSA_ERR_UNSUPPORTED, "paged_decode_noalloc: device %d (at most %d devices)", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_status(e, "paged_decode_noalloc: hipGetSymbolAddress");
    if (p == nullptr) return fail(QSA_ERR_DEVICE, "paged_decode_noalloc: the scratch array has no address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QSA_OK;
}

}  // namespace

extern "C" qsa_status qsa_paged_decode_noalloc(const qsa_dims* dims, const void* q,
                                               const qsa_paged_kv* kv, const int32_t* sel,
                                               const int32_t* sel_count, int32_t k,
                                               float sm_scale, float* out, float* lse,
                                               hipStream_t stream) {
  using namespace qsa::host;
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
  if (w.total() > kScratchBytes)
    return fail(QSA_ERR_WORKSPACE,
                "paged_decode_noalloc: this batch needs %zu bytes of partial results; the static "
                "scratch holds %zu (use qsa_paged_decode with a workspace)",
                w.total(), kScratchBytes);
  void* base = nullptr;
  if ((s = scratch_address(&base)) != QSA_OK) return s;
  const qsa::Partials part = carve(base, w);
  qsa::LaunchCommon c = common(dims, kv);
  Checked chk;
  if ((s = chk.begin(c, stream)) != QSA_OK) return s;
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  return chk.end(device_status(qsa::launch_decode(c, q, sel, sel_count, kk, scale_log2, plan, part,
                                                  qsa::Partials{}, 0, out, lse, stream),
                               "paged_decode_noalloc launch"),
                 stream);
}
