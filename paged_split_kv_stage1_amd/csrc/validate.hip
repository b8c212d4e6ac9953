// Debug check of the page table a plan reads: every page-table entry a work item's token
// range touches must name a page inside the cache.  Stage 1 itself never checks page
// numbers (its loads take them as given), so a caller that wants the check runs this first
// (the Python binding does so when the environment sets PA_VALIDATE=1).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdio>

#include "pa.h"
#include "pa_internal.hpp"

namespace pa {

// Per-device result of the last check: count of bad entries, and the lowest bad position.
static __device__ int bad_count;
static __device__ int bad_first;

__global__ __launch_bounds__(64) void validate_reset_kernel() {
  bad_count = 0;
  bad_first = INT_MAX;
}

__global__ __launch_bounds__(256) void validate_kernel(const PaItem* items, const int32_t* page_indices,
                                                       int64_t num_pages, int page_shift) {
  const PaItem it = items[blockIdx.x];
  if (it.tok_end <= it.tok_begin) return;
  const int p0 = it.tok_begin >> page_shift;
  const int p1 = (it.tok_end - 1) >> page_shift;
  for (int p = p0 + (int)threadIdx.x; p <= p1; p += 256) {
    const int pos = it.page_base + p;
    const int32_t pg = page_indices[pos];
    if (pg < 0 || (int64_t)pg >= num_pages) {
      atomicAdd(&bad_count, 1);
      atomicMin(&bad_first, pos);
    }
  }
}

}  // namespace pa

extern "C" pa_status pa_validate_page_indices(const pa_plan_info* info, const void* plan_dev,
                                              const int32_t* page_indices, int64_t num_pages, void* stream) {
  using namespace pa;
  if (!info || !plan_dev || !page_indices)
    return (pa_status)report_error(PA_ERR_INVALID_ARGUMENT, "pa_validate_page_indices: NULL pointer");
  if (num_pages < 0)
    return (pa_status)report_error(PA_ERR_INVALID_ARGUMENT, "pa_validate_page_indices: num_pages must be >= 0");
  int shift = 0;
  while ((1 << shift) < info->page_size) ++shift;
  const hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(validate_reset_kernel, dim3(1), dim3(1), 0, s);
  if (info->num_items > 0)
    hipLaunchKernelGGL(validate_kernel, dim3(info->num_items), dim3(256), 0, s, static_cast<const PaItem*>(plan_dev),
                       page_indices, num_pages, shift);
  int count = 0, first = 0;
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpyFromSymbolAsync(&count, HIP_SYMBOL(bad_count), sizeof count, 0,
                                                    hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyFromSymbolAsync(&first, HIP_SYMBOL(bad_first), sizeof first, 0,
                                                    hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    char msg[200];
    snprintf(msg, sizeof msg, "pa_validate_page_indices: %s", hipGetErrorString(e));
    return (pa_status)report_error(PA_ERR_HIP, msg);
  }
  if (count > 0) {
    char msg[200];
    snprintf(msg, sizeof msg, "pa_validate_page_indices: %d reads of page-table entries outside [0, %lld) by the "
             "plan's work items; the first offending entry is page_indices[%d]", count, (long long)num_pages, first);
    return (pa_status)report_error(PA_ERR_INVALID_ARGUMENT, msg);
  }
  return (pa_status)report_error(PA_OK, "");
}
