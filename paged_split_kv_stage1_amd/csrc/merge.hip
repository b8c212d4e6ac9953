// Stage 2 of split-KV decode: merge the per-split partial outputs of each
// (query row, query head) with their log-sum-exp weights (FreeToken PR #900,
// "Changes": stage 2 merges per row).
//
// The unit of work is one (row, head, 64-wide slice of d): lane i of a wave owns
// element d = 64 * slice + i.  Two launch shapes share one kernel:
//   WPU = 4 (many splits): the four waves of a workgroup share one unit, wave w
//     accumulates splits w, w+4, w+8, ... (sixteen of them in flight) and the four
//     partial sums are combined through LDS;
//   WPU = 1 (few splits): every wave merges a unit of its own, with its splits in
//     flight together, so that short merges do not pay one workgroup each.
// The partials were written just before by stage 1 and mostly come back from L2/MALL,
// so the loop is bound by load latency: the point of both shapes is loads in flight.
// Rows whose request has a single split were written by stage 1 directly and are
// skipped.
#include "common.hpp"

namespace pa {

// Largest LSE over the row-head's ns splits; every lane of the wave gets it.
__device__ __forceinline__ float lse_max(const float* lse, int ns, int lane) {
  float mx = -INFINITY;
  for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, lse[s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  return mx;
}

// Weighted sums over splits s0, s0 + STEP, ... < ns of one lane's d element.
template <int STEP>
__device__ __forceinline__ void accumulate(const float* lse, const float* po, int dh, int s0, int ns, float muse,
                                           float& num, float& den) {
  int s = s0;
  for (; s + 15 * STEP < ns; s += 16 * STEP) {
    float l[16], o[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      l[u] = lse[s + STEP * u];
      o[u] = po[(int64_t)(s + STEP * u) * dh];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const float wgt = (l[u] == -INFINITY) ? 0.f : __expf(l[u] - muse);
      den += wgt;
      num += wgt * o[u];
    }
  }
  for (; s + 3 * STEP < ns; s += 4 * STEP) {
    float l[4], o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      l[u] = lse[s + STEP * u];
      o[u] = po[(int64_t)(s + STEP * u) * dh];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wgt = (l[u] == -INFINITY) ? 0.f : __expf(l[u] - muse);
      den += wgt;
      num += wgt * o[u];
    }
  }
  for (; s < ns; s += STEP) {
    const float l = lse[s];
    const float wgt = (l == -INFINITY) ? 0.f : __expf(l - muse);
    den += wgt;
    num += wgt * po[(int64_t)s * dh];
  }
}

__device__ __forceinline__ void store_merged(const MergeArgs& a, int th, int d, float num, float den, float muse,
                                             bool write_lse) {
  const float o = den > 0.f ? num / den : 0.f;
  if (a.out_bf16)
    static_cast<__bf16*>(a.out)[(int64_t)th * a.dh + d] = (__bf16)o;
  else
    static_cast<float*>(a.out)[(int64_t)th * a.dh + d] = o;
  if (a.out_lse && write_lse) a.out_lse[th] = den > 0.f ? muse + __logf(den) : -INFINITY;
}

template <int WPU>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nsl = a.dh / 64;                          // d slices per row-head
  const int unit = WPU == 4 ? blockIdx.x : blockIdx.x * 4 + wave;
  if (unit >= a.total_rows * a.hq * nsl) return;     // (WPU = 1: whole waves past the end)
  const int th = unit / nsl;
  const int slice = unit - th * nsl;
  const int t = th / a.hq;
  const int ns = a.row_nsplit[t];
  if (ns <= 1) return;
  const int d = slice * 64 + lane;
  const float* lse = a.partial_lse + (int64_t)th * a.s_max;
  const float* po = a.partial_o + (int64_t)th * a.s_max * a.dh + d;
  const float mx = lse_max(lse, ns, lane);
  const float muse = (mx == -INFINITY) ? 0.f : mx;
  float num = 0.f, den = 0.f;
  if constexpr (WPU == 1) {
    accumulate<1>(lse, po, a.dh, 0, ns, muse, num, den);
    store_merged(a, th, d, num, den, muse, slice == 0 && lane == 0);
  } else {
    __shared__ float num_s[4][64];
    __shared__ float den_s[4];
    accumulate<4>(lse, po, a.dh, wave, ns, muse, num, den);
    num_s[wave][lane] = num;
    if (lane == 0) den_s[wave] = den;
    __syncthreads();
    if (wave != 0) return;
    num = (num_s[0][lane] + num_s[1][lane]) + (num_s[2][lane] + num_s[3][lane]);
    den = (den_s[0] + den_s[1]) + (den_s[2] + den_s[3]);
    store_merged(a, th, d, num, den, muse, slice == 0 && lane == 0);
  }
}

int launch_merge(const MergeArgs& a, void* stream) {
  if (a.total_rows <= 0) return 0;
  const int64_t units = (int64_t)a.total_rows * a.hq * (a.dh / 64);
  if (a.s_max >= 64) {
    hipLaunchKernelGGL(merge_kernel<4>, dim3((unsigned)units), dim3(256), 0, (hipStream_t)stream, a);
  } else {
    hipLaunchKernelGGL(merge_kernel<1>, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, (hipStream_t)stream, a);
  }
  return (int)hipGetLastError();
}

}  // namespace pa
