// Host-side helpers of the libqsa C ABI shared by its source files: status
// and message handling, argument checks, the decode work plan and its
// workspace layout, and the checked mode. Not part of the public header.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "qsa.h"
#include "qsa_internal.h"

namespace qsa {
namespace host {

// Sets the calling thread's qsa_last_error() message and returns s.
qsa_status fail(qsa_status s, const char* fmt, ...);
// Clears the message and returns QSA_OK.
qsa_status ok();
// QSA_OK for hipSuccess, else QSA_ERR_DEVICE with "what: <HIP error>".
qsa_status device_status(hipError_t e, const char* what);

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int pages_of(int L);

// Shape checks shared by every entry point; check_kv also returns the
// longest sequence's page count.
qsa_status check_dims(const qsa_dims* d);
qsa_status check_kv(const qsa_dims* d, const qsa_paged_kv* kv, bool need_v, int* max_pages);
qsa::LaunchCommon common(const qsa_dims* d, const qsa_paged_kv* kv);

// Compute units of the current device.
int device_cus();

// The decode work split for these lengths (k <= 0: every page).
qsa::DecodePlan make_plan(const qsa_dims* d, const int32_t* lens, int32_t k);
qsa_status check_plan(const qsa::DecodePlan& p);

// Decode workspace: [partial outputs][partial (max, sum)][stream split: the
// rows' (first, last) waves], each region 256-byte aligned. Partial slots:
// rows x max_units (units), or waves + rows (stream: slot w + r for the
// segment of row r in wave w). Every slot a merge reads is written by the
// decode launch before it, so the workspace needs no clearing.
struct DecodeWs {
  size_t o_bytes = 0, ml_bytes = 0, rs_bytes = 0;
  size_t total() const { return align_up(o_bytes) + align_up(ml_bytes) + align_up(rs_bytes); }
};
DecodeWs decode_ws(const qsa_dims* d, const qsa::DecodePlan& plan);
qsa::Partials carve(void* ws, const DecodeWs& w);

// Checked mode (process-wide; QSA_CHECKED=1 in the environment, or
// qsa_set_checked): see api.hip.
bool checked_mode();
void set_checked_mode(bool on);

// One entry point's use of the device error word: begin() (after argument
// validation, before the launches) clears the word on the stream and puts it
// in c.err when checked mode is on; end(status of the launches) then waits
// for the stream and turns a set word into QSA_ERR_DEVICE. Both are no-ops
// when checked mode is off.
class Checked {
 public:
  qsa_status begin(qsa::LaunchCommon& c, hipStream_t stream);
  qsa_status end(qsa_status s, hipStream_t stream);

 private:
  unsigned int* word_ = nullptr;
};

}  // namespace host
}  // namespace qsa
