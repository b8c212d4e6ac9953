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
// so the loop is bound by load latency: the point of both shapes is loads in flight,
// and of the single pass (online maximum) that no load waits for another.
// Rows whose request has a single split were written by stage 1 directly and are
// skipped.
#include "common.hpp"

namespace pa {

// Weighted sums over splits s0, s0 + STEP, ... < ns of one lane's d element, in one
// pass: each batch's LSE and partial loads are issued together, and the running maximum
// m rescales the sums when a batch raises it (no separate pass for the maximum, whose
// loads would have to come back before the first partial is requested).
template <int B>
__device__ __forceinline__ void merge_batch(const float (&l)[B], const float (&o)[B], float& m, float& num,
                                            float& den) {
  float bm = l[0];
#pragma unroll
  for (int u = 1; u < B; ++u) bm = fmaxf(bm, l[u]);
  if (bm > m) {                                   // (false while every LSE so far is -inf)
    const float f = __expf(m - bm);               // 0 when m is still -inf
    num *= f;
    den *= f;
    m = bm;
  }
#pragma unroll
  for (int u = 0; u < B; ++u) {
    const float wgt = (l[u] == -INFINITY) ? 0.f : __expf(l[u] - m);
    den += wgt;
    num += wgt * o[u];
  }
}

template <int STEP, typename T>
__device__ __forceinline__ void accumulate(const float* lse, const T* po, int dh, int s0, int ns, float& m,
                                           float& num, float& den) {
  int s = s0;
  for (; s + 15 * STEP < ns; s += 16 * STEP) {
    float l[16], o[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      l[u] = lse[s + STEP * u];
      o[u] = (float)po[(int64_t)(s + STEP * u) * dh];
    }
    merge_batch(l, o, m, num, den);
  }
  for (; s + 3 * STEP < ns; s += 4 * STEP) {
    float l[4], o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      l[u] = lse[s + STEP * u];
      o[u] = (float)po[(int64_t)(s + STEP * u) * dh];
    }
    merge_batch(l, o, m, num, den);
  }
  for (; s < ns; s += STEP) {
    float l[1] = {lse[s]}, o[1] = {(float)po[(int64_t)s * dh]};
    merge_batch(l, o, m, num, den);
  }
}

__device__ __forceinline__ void store_merged(const MergeArgs& a, int th, int d, float num, float den, float m,
                                             bool write_lse) {
  const float o = den > 0.f ? num / den : 0.f;
  if (a.out_bf16)
    static_cast<__bf16*>(a.out)[(int64_t)th * a.dh + d] = (__bf16)o;
  else
    static_cast<float*>(a.out)[(int64_t)th * a.dh + d] = o;
  if (a.out_lse && write_lse) a.out_lse[th] = den > 0.f ? m + __logf(den) : -INFINITY;
}

template <int WPU, typename T>
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
  const T* po = static_cast<const T*>(a.partial_o) + (int64_t)th * a.s_max * a.dh + d;
  float m = -INFINITY, num = 0.f, den = 0.f;
  if constexpr (WPU == 1) {
    accumulate<1>(lse, po, a.dh, 0, ns, m, num, den);
    store_merged(a, th, d, num, den, m, slice == 0 && lane == 0);
  } else {
    __shared__ float num_s[4][64];
    __shared__ float den_s[4], m_s[4];
    accumulate<4>(lse, po, a.dh, wave, ns, m, num, den);
    num_s[wave][lane] = num;
    if (lane == 0) {
      den_s[wave] = den;
      m_s[wave] = m;
    }
    __syncthreads();
    if (wave != 0) return;
    const float mall = fmaxf(fmaxf(m_s[0], m_s[1]), fmaxf(m_s[2], m_s[3]));
    num = 0.f;
    den = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = m_s[w] == -INFINITY ? 0.f : __expf(m_s[w] - mall);
      num += num_s[w][lane] * f;
      den += den_s[w] * f;
    }
    store_merged(a, th, d, num, den, mall, slice == 0 && lane == 0);
  }
}

int launch_merge(const MergeArgs& a, void* stream) {
  if (a.total_rows <= 0) return 0;
  const int64_t units = (int64_t)a.total_rows * a.hq * (a.dh / 64);
  const dim3 g4((unsigned)units), g1((unsigned)((units + 3) / 4));
  if (a.s_max >= 64) {
    if (a.part_bf16) hipLaunchKernelGGL((merge_kernel<4, __bf16>), g4, dim3(256), 0, (hipStream_t)stream, a);
    else hipLaunchKernelGGL((merge_kernel<4, float>), g4, dim3(256), 0, (hipStream_t)stream, a);
  } else {
    if (a.part_bf16) hipLaunchKernelGGL((merge_kernel<1, __bf16>), g1, dim3(256), 0, (hipStream_t)stream, a);
    else hipLaunchKernelGGL((merge_kernel<1, float>), g1, dim3(256), 0, (hipStream_t)stream, a);
  }
  return (int)hipGetLastError();
}

}  // namespace pa
