// Stage 2 of split-KV decode: merge the per-split partial outputs of each
// (query row, query head) with their log-sum-exp weights (FreeToken PR #900,
// "Changes": stage 2 merges per row).
//
// One 256-thread workgroup per (row, head, 64-wide slice of d).  All four waves read
// the row's S split LSEs to find their maximum; wave w then accumulates splits
// w, w+4, w+8, ... for its lane's d element, and the four partial sums are combined
// through LDS.  Rows whose request has a single split were written by stage 1
// directly and are skipped.
#include "common.hpp"

namespace pa {

__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  __shared__ float num_s[4][64];
  __shared__ float den_s[4];
  const int th = blockIdx.x;
  const int t = th / a.hq;
  const int ns = a.row_nsplit[t];
  if (ns <= 1) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int d = blockIdx.y * 64 + lane;
  const float* lse = a.partial_lse + (int64_t)th * a.s_max;
  float mx = -INFINITY;
  for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, lse[s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  const float muse = (mx == -INFINITY) ? 0.f : mx;
  const float* po = a.partial_o + (int64_t)th * a.s_max * a.dh + d;
  float num = 0.f, den = 0.f;
  int s = wave;
  for (; s + 12 < ns; s += 16) {           // four splits per wave in flight
    const float l0 = lse[s], l1 = lse[s + 4], l2 = lse[s + 8], l3 = lse[s + 12];
    const float o0 = po[(int64_t)s * a.dh], o1 = po[(int64_t)(s + 4) * a.dh];
    const float o2 = po[(int64_t)(s + 8) * a.dh], o3 = po[(int64_t)(s + 12) * a.dh];
    const float w0 = (l0 == -INFINITY) ? 0.f : __expf(l0 - muse);
    const float w1 = (l1 == -INFINITY) ? 0.f : __expf(l1 - muse);
    const float w2 = (l2 == -INFINITY) ? 0.f : __expf(l2 - muse);
    const float w3 = (l3 == -INFINITY) ? 0.f : __expf(l3 - muse);
    den += (w0 + w1) + (w2 + w3);
    num += (w0 * o0 + w1 * o1) + (w2 * o2 + w3 * o3);
  }
  for (; s < ns; s += 4) {
    const float l = lse[s];
    const float w = (l == -INFINITY) ? 0.f : __expf(l - muse);
    den += w;
    num += w * po[(int64_t)s * a.dh];
  }
  num_s[wave][lane] = num;
  if (lane == 0) den_s[wave] = den;
  __syncthreads();
  if (wave != 0) return;
  num = (num_s[0][lane] + num_s[1][lane]) + (num_s[2][lane] + num_s[3][lane]);
  den = (den_s[0] + den_s[1]) + (den_s[2] + den_s[3]);
  const float o = den > 0.f ? num / den : 0.f;
  if (a.out_bf16)
    static_cast<__bf16*>(a.out)[(int64_t)th * a.dh + d] = (__bf16)o;
  else
    static_cast<float*>(a.out)[(int64_t)th * a.dh + d] = o;
  if (a.out_lse && blockIdx.y == 0 && lane == 0) a.out_lse[th] = den > 0.f ? muse + __logf(den) : -INFINITY;
}

int launch_merge(const MergeArgs& a, void* stream) {
  if (a.total_rows <= 0) return 0;
  dim3 grid((unsigned)(a.total_rows * a.hq), (unsigned)(a.dh / 64));
  hipLaunchKernelGGL(merge_kernel, grid, dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace pa
