// cvr_score_noalloc: scoring for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).  The workspace is a
// fixed array in the library's own device memory instead of a caller-provided buffer.
//
// `scratch` below is a __device__ array: in host code its name is only a host-side stand-in,
// never a device address.  Its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that address is handed to the
// kernels (as the workspace pointer of an ordinary scoring call).
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "../../include/cvr.h"
#include "kernels.h"
#include "model.h"

namespace cvr {

// One copy per device, held until the process ends.  Every scoring call on a device uses the
// same copy: no part of it is assumed to hold anything at the start of a call (the call
// clears its error flag with a kernel and writes every other buffer before reading it).
static __device__ __align__(256) char scratch[CVR_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

// Device address of this device's scratch array (looked up on the device's first call).
static hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace cvr

extern "C" cvr_status cvr_score_noalloc(cvr_handle h, const cvr_batch* b, float* out_scores, void* hip_stream) {
  if (!h) return cvr::fail(nullptr, CVR_ERR_ARG, "null handle");
  if (!b) return cvr::fail(h, CVR_ERR_ARG, "null batch");
  if (b->n_requests < 0 || b->n_candidates < 0 || b->n_positions < 0)
    return cvr::fail(h, CVR_ERR_ARG, "negative size");
  const size_t need = cvr::plan_workspace(h, b->n_requests, b->n_candidates,
                                          h->spec.model == CVR_MODEL_DLRM ? 0 : b->n_positions).total;
  if (need > (size_t)CVR_NOALLOC_SCRATCH_BYTES)
    return cvr::fail(h, CVR_ERR_WORKSPACE,
                     "batch needs " + std::to_string(need) + " bytes of workspace; the allocation-free call holds " +
                         std::to_string((size_t)CVR_NOALLOC_SCRATCH_BYTES) + " (use cvr_score with a workspace)");
  void* ws = nullptr;
  const hipError_t e = cvr::scratch_ptr(&ws);
  if (e != hipSuccess)
    return cvr::fail(h, CVR_ERR_HIP, std::string("scratch address: ") + hipGetErrorString(e));
  return cvr::score_call(h, b, ws, (size_t)CVR_NOALLOC_SCRATCH_BYTES, out_scores, hip_stream);
}
