// Allocation-free decode step: stage 1 + merge with the split partials held in a
// file-scope device array instead of caller-provided workspace, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Each GPU the library runs on holds its own copy of the array
// (kScratchBytes) until the process ends.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "pa.h"
#include "pa_internal.hpp"

namespace pa {

constexpr size_t kScratchBytes = size_t(128) << 20;     // partial O + partial LSE of one step
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this GPU's scratch array, looked up once per device (with that
// device current) and kept; host code uses only this address, never the symbol itself.
static int scratch_address(int dev, unsigned char** out) {
  static std::mutex mu;
  static unsigned char* addr[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    addr[dev] = static_cast<unsigned char*>(p);
  }
  *out = addr[dev];
  return 0;
}

}  // namespace pa

extern "C" pa_status pa_decode_noalloc(const pa_plan_info* info, const void* plan_dev, const void* q,
                                       const float* q_scale, const void* k_cache, const void* v_cache,
                                       const pa_kv_layout* kv, const float* k_scale, const float* v_scale,
                                       const pa_scale_layout* sc, const int32_t* page_indices, float sm_scale,
                                       void* out, pa_dtype out_dtype, float* out_lse, void* stream) {
  using namespace pa;
  if (!info) return (pa_status)report_error(PA_ERR_INVALID_ARGUMENT, "pa_decode_noalloc: info must be non-NULL");
  const int64_t o_bytes = info->needs_merge ? info->partial_o_bytes : 0;
  const int64_t lse_off = (o_bytes + 255) / 256 * 256;
  const int64_t need = info->needs_merge ? lse_off + info->partial_lse_bytes : 0;
  if (o_bytes < 0 || info->partial_lse_bytes < 0 || need > (int64_t)kScratchBytes) {
    char msg[200];
    snprintf(msg, sizeof msg, "pa_decode_noalloc: this plan's split partials need %lld bytes, above the %zu-byte "
             "scratch array (plan with a lower max_splits, or use pa_decode_stage1 with a workspace)",
             (long long)need, kScratchBytes);
    return (pa_status)report_error(PA_ERR_INSUFFICIENT_WORKSPACE, msg);
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  unsigned char* base = nullptr;
  int err = e == hipSuccess ? scratch_address(dev, &base) : (int)e;
  if (err) {
    char msg[200];
    snprintf(msg, sizeof msg, "pa_decode_noalloc: device scratch address: %s", hipGetErrorString((hipError_t)err));
    return (pa_status)report_error(PA_ERR_HIP, msg);
  }
  void* partial_o = info->needs_merge ? base : nullptr;
  float* partial_lse = info->needs_merge ? reinterpret_cast<float*>(base + lse_off) : nullptr;
  const pa_status st = pa_decode_stage1(info, plan_dev, q, q_scale, k_cache, v_cache, kv, k_scale, v_scale, sc,
                                        page_indices, sm_scale, partial_o, partial_lse, out, out_dtype, out_lse,
                                        stream);
  if (st != PA_OK) return st;
  return pa_decode_merge(info, plan_dev, partial_o, partial_lse, out, out_dtype, out_lse, stream);
}
