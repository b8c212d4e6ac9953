// Stage 2 of split-KV decode: merge the per-split partial outputs of each
// (query row, query head) with their log-sum-exp weights (FreeToken PR #900,
// "Changes": stage 2 merges per row).  One 64-thread workgroup per
// (row, head, 64-wide slice of d); rows whose request has one split were written
// by stage 1 directly and are skipped.
#include "common.hpp"

namespace pa {

__global__ __launch_bounds__(64) void merge_kernel(MergeArgs a) {
  const int th = blockIdx.x;
  const int t = th / a.hq;
  const int ns = a.row_nsplit[t];
  if (ns <= 1) return;
  const int d = blockIdx.y * 64 + threadIdx.x;
  const float* lse = a.partial_lse + (int64_t)th * a.s_max;
  float mx = -INFINITY;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, lse[s]);
  const float muse = (mx == -INFINITY) ? 0.f : mx;
  float num = 0.f, den = 0.f;
  const float* po = a.partial_o + (int64_t)th * a.s_max * a.dh + d;
  for (int s = 0; s < ns; ++s) {
    const float l = lse[s];
    const float w = (l == -INFINITY) ? 0.f : expf(l - muse);
    den += w;
    num += w * po[(int64_t)s * a.dh];
  }
  const float o = den > 0.f ? num / den : 0.f;
  if (a.out_bf16)
    static_cast<__bf16*>(a.out)[(int64_t)th * a.dh + d] = (__bf16)o;
  else
    static_cast<float*>(a.out)[(int64_t)th * a.dh + d] = o;
  if (a.out_lse && blockIdx.y == 0 && threadIdx.x == 0) a.out_lse[th] = den > 0.f ? muse + logf(den) : -INFINITY;
}

int launch_merge(const MergeArgs& a, void* stream) {
  if (a.total_rows <= 0) return 0;
  dim3 grid((unsigned)(a.total_rows * a.hq), (unsigned)(a.dh / 64));
  hipLaunchKernelGGL(merge_kernel, grid, dim3(64), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace pa
