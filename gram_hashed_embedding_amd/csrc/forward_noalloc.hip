// engram_forward for callers that cannot allocate device memory (code under
// HIP graph capture, serving loops that forbid hipMalloc): the workspace is a
// file-scope device array of ENGRAM_NOALLOC_WORKSPACE_BYTES, one per GPU,
// held until the process ends. Its device address is looked up once per
// device with hipGetSymbolAddress (in host code the array's name is not a
// device address) and passed to the same kernels engram_forward launches.
// Nothing in the forward path reads a workspace byte it has not written in
// the same call, so the array needs no clearing between calls; calls that
// overlap on one GPU share it and race.

#include <hip/hip_runtime.h>

#include <mutex>

#include "engram_internal.h"

namespace {

constexpr size_t kScratchBytes = ENGRAM_NOALLOC_WORKSPACE_BYTES;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the
// device's first call, with that device current).
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return engram::report(ENGRAM_EHIP, "engram_forward_noalloc: hipGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices)
    return engram::report(ENGRAM_EUNSUPPORTED, "engram_forward_noalloc: device ordinal above 63",
                          hipSuccess);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return engram::report(ENGRAM_EHIP, "engram_forward_noalloc: hipGetSymbolAddress", e);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ENGRAM_OK;
}

}  // namespace

extern "C" int engram_forward_noalloc(
    const uint32_t* tok, const int32_t* cu_seqlens, int32_t S, int64_t T, const uint32_t* hist,
    const uint32_t* token_map, uint32_t map_len, const engram_hash_params* params,
    const uint8_t* codes, const uint8_t* scales, const uint16_t* wkv, const uint16_t* wkv_packed,
    const float* wqk, uint16_t* hidden, int32_t H, int32_t hc, float eps, float dot_scale,
    float* gate_out, uint32_t* err_flags, hipStream_t stream) {
  if (H > 0 && hc > 0 && T > 0 && engram_forward_workspace(T, H, hc) > kScratchBytes)
    return engram::report(ENGRAM_EINVAL,
                          "engram_forward_noalloc: the workspace for this T, H and hc exceeds "
                          "ENGRAM_NOALLOC_WORKSPACE_BYTES (64 MiB: up to 1,055 tokens at H = 5120, hc = 4)",
                          hipSuccess);
  void* ws = nullptr;
  if (T > 0) {
    const int rc = scratch_address(&ws);
    if (rc != ENGRAM_OK) return rc;
  }
  return engram::forward_impl(tok, cu_seqlens, S, T, hist, token_map, map_len, params, codes, scales,
                              wkv, wkv_packed, wqk, hidden, H, hc, eps, dot_scale, ws,
                              T > 0 ? kScratchBytes : 0, gate_out, err_flags, nullptr, stream);
}
