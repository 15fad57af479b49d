// noalloc.hip -- norm_bwd_noalloc: the backward with its workspace in a static device array, for
// callers that cannot allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The backward's kernels need scratch memory for the per-workgroup weight-gradient partials the
// finalize kernel reduces ([NVRTC-PR] "Migrate norms and softmax kernels to NVRTC", Flowchart:
// partial kernels, then finalize). norm_bwd takes it from the caller's workspace; this entry point
// takes it from `scratch`, a file-scope __device__ array of kScratchBytes that every GPU the
// library runs on holds until the process ends. In host code `scratch` is only a host-side
// stand-in for the symbol: its device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is ever passed to a kernel.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>
#include <unordered_map>

#include "../../include/normfp8.h"
#include "kernels.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;  // NORM_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == NORM_NOALLOC_SCRATCH_BYTES, "scratch size mismatch");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
std::unordered_map<int, void *> g_scratch;  // device -> device address of `scratch`
thread_local char g_msg[256];

// the device address of this device's copy of `scratch` (looked up on its first use)
int scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    snprintf(g_msg, sizeof(g_msg), "hipGetDevice: %s", hipGetErrorString(e));
    return NORM_ERR_HIP;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      snprintf(g_msg, sizeof(g_msg), "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      return NORM_ERR_HIP;
    }
    it = g_scratch.emplace(dev, ptr).first;
  }
  *out = it->second;
  return NORM_OK;
}

}  // namespace

extern "C" int norm_bwd_noalloc(void *stream, const void *dy, const void *x, const float *mu, const float *rsigma,
                                const void *gamma, void *dx, void *dgamma, void *dbeta, int64_t rows, int64_t hidden,
                                int in_dtype, int w_dtype, int norm_type, int zero_centered_gamma, int cu_margin) {
  size_t need = 0;
  int rc = norm_bwd_workspace_size(rows, hidden, in_dtype, w_dtype, norm_type, zero_centered_gamma, 0.0f,
                                   cu_margin, 0, &need);
  if (rc != NORM_OK) return rc;
  if (need > kScratchBytes) {
    snprintf(g_msg, sizeof(g_msg),
             "norm_bwd_noalloc: this shape needs %zu bytes of scratch; the static buffer holds %zu "
             "(use norm_bwd with a caller workspace)",
             need, kScratchBytes);
    return nf8::set_last_error(NORM_ERR_UNSUPPORTED, g_msg);
  }
  void *ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != NORM_OK) return nf8::set_last_error(rc, g_msg);
  // the backward reads nothing of the workspace it has not written in the same call (the
  // partial rows are written by the row kernel, then reduced by the finalize kernel), so the
  // previous call's contents need no clearing
  return norm_bwd(stream, dy, x, mu, rsigma, gamma, dx, dgamma, dbeta, ws, kScratchBytes, rows, hidden, in_dtype,
                  w_dtype, norm_type, zero_centered_gamma, cu_margin);
}
