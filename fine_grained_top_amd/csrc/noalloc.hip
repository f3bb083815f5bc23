// spattn_sparse_attn_fwd_noalloc: the forward attention call with its
// workspace taken from a fixed device array instead of the caller, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, until the process ends. Its
// device address is taken once per device with hipGetSymbolAddress (the
// device current at the first call on it) and only that address is handed to
// kernels; the array's name in host code is a host-side stand-in, not a
// device pointer. Nothing here allocates: no hipMalloc, no library call that
// does. Calls on one device share the array, so calls that overlap in time on
// one device (different streams, or host threads) race; calls ordered on one
// stream do not. The attention kernels write every scratch word they read
// before reading it, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "api_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;   // 32 MiB per device

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[64];     // device address of `scratch` per device, once taken

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return spapi::set_error(SPATTN_ERR_NO_DEVICE, "no HIP device for the fixed scratch array");
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      char msg[160];
      std::snprintf(msg, sizeof msg, "hipGetSymbolAddress of the scratch array failed on device %d: %s", dev,
                    hipGetErrorString(e));
      return spapi::set_error(SPATTN_ERR_LAUNCH, msg);
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SPATTN_OK;
}

}  // namespace

extern "C" {

SPATTN_API size_t spattn_noalloc_scratch_bytes(void) { return kScratchBytes; }

SPATTN_API int spattn_sparse_attn_fwd_noalloc(const spattn_tensor* q, const spattn_tensor* k,
                                              const spattn_tensor* v, const int32_t* ctx_len, float scale,
                                              const spattn_selection* sel, const spattn_tensor* o_out,
                                              float* lse_out, void* stream) {
  sp::AttnParams p;
  size_t need = 0;
  int rc;
  if ((rc = spapi::attn_fwd_prepare(q, k, v, nullptr, ctx_len, scale, sel, o_out, lse_out, p, need))) return rc;
  if (need > kScratchBytes) {
    char msg[200];
    std::snprintf(msg, sizeof msg,
                  "this call needs %zu bytes of scratch, more than the fixed %zu-byte array of the "
                  "no-allocation entry point; use spattn_sparse_attn_fwd with a workspace",
                  need, kScratchBytes);
    return spapi::set_error(SPATTN_ERR_WORKSPACE, msg);
  }
  if ((rc = spapi::device_check())) return rc;
  void* ws = nullptr;
  if (need && (rc = scratch_address(&ws))) return rc;
  return spapi::attn_fwd_launch(p, ws, need ? kScratchBytes : 0, stream);
}

}  // extern "C"
