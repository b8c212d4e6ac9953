// Test hook: writes the physical slot (page * P + slot) that stage 1 reads for each
// token of each split, using the same page-gather code (token_page / token_slot).
#include "common.hpp"

namespace pa {

__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const PaItem it = a.items[blockIdx.x];
  if (it.kvh != 0 || it.qblk0 != 0) return;     // one item per token range
  const int64_t base = a.kv_tok_offset[it.req];
  const int P = 1 << a.page_shift;
  for (int j = it.tok_begin + (int)threadIdx.x; j < it.tok_end; j += 256) {
    const int32_t pg = token_page(a.page_indices, it.page_base, j, a.page_shift);
    const int32_t sl = token_slot(j, a.page_shift);
    a.phys_out[base + j] = (int64_t)pg * P + sl;
  }
}

int launch_gather(const GatherArgs& a, int num_items, void* stream) {
  if (num_items <= 0) return 0;
  hipLaunchKernelGGL(gather_kernel, dim3(num_items), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace pa
