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
#include <type_traits>

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

template <int STEP>
__device__ __forceinline__ void accumulate(const float* lse, const float* po, int dh, int s0, int ns, float& m,
                                           float& num, float& den) {
  int s = s0;
  for (; s + 15 * STEP < ns; s += 16 * STEP) {
    float l[16], o[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      l[u] = lse[s + STEP * u];
      o[u] = po[(int64_t)(s + STEP * u) * dh];
    }
    merge_batch(l, o, m, num, den);
  }
  for (; s + 3 * STEP < ns; s += 4 * STEP) {
    float l[4], o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      l[u] = lse[s + STEP * u];
      o[u] = po[(int64_t)(s + STEP * u) * dh];
    }
    merge_batch(l, o, m, num, den);
  }
  for (; s < ns; s += STEP) {
    float l[1] = {lse[s]}, o[1] = {po[(int64_t)s * dh]};
    merge_batch(l, o, m, num, den);
  }
}

// The same for bf16 partials, two adjacent d elements per lane (4-byte loads).
template <int B>
__device__ __forceinline__ void merge_batch2(const float (&l)[B], const f32x2 (&o)[B], float& m, f32x2& num,
                                             float& den) {
  float bm = l[0];
#pragma unroll
  for (int u = 1; u < B; ++u) bm = fmaxf(bm, l[u]);
  if (bm > m) {
    const float f = __expf(m - bm);
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

__device__ __forceinline__ f32x2 load_bf16x2(const __bf16* p) {
  const bf16x2 v = *reinterpret_cast<const bf16x2*>(p);
  return f32x2{(float)v[0], (float)v[1]};
}

template <int STEP>
__device__ __forceinline__ void accumulate2(const float* lse, const __bf16* po, int dh, int s0, int ns, float& m,
                                            f32x2& num, float& den) {
  int s = s0;
  for (; s + 15 * STEP < ns; s += 16 * STEP) {
    float l[16];
    f32x2 o[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      l[u] = lse[s + STEP * u];
      o[u] = load_bf16x2(po + (int64_t)(s + STEP * u) * dh);
    }
    merge_batch2(l, o, m, num, den);
  }
  for (; s + 3 * STEP < ns; s += 4 * STEP) {
    float l[4];
    f32x2 o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      l[u] = lse[s + STEP * u];
      o[u] = load_bf16x2(po + (int64_t)(s + STEP * u) * dh);
    }
    merge_batch2(l, o, m, num, den);
  }
  for (; s < ns; s += STEP) {
    float l[1] = {lse[s]};
    f32x2 o[1] = {load_bf16x2(po + (int64_t)s * dh)};
    merge_batch2(l, o, m, num, den);
  }
}

// Lanes l and l ^ 32 hold the same two d elements over interleaved splits: combine them
// (every lane of the pair gets the result).
__device__ __forceinline__ void combine_halves(float& m, f32x2& num, float& den) {
  auto sw = [](float x) __attribute__((always_inline)) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
  };
  const f32x2 mm = sw(m), dd = sw(den), n0 = sw(num[0]), n1 = sw(num[1]);
  const float mx = fmaxf(mm[0], mm[1]);
  const float f0 = mm[0] == -INFINITY ? 0.f : __expf(mm[0] - mx);
  const float f1 = mm[1] == -INFINITY ? 0.f : __expf(mm[1] - mx);
  m = mx;
  den = dd[0] * f0 + dd[1] * f1;
  num = f32x2{n0[0] * f0 + n0[1] * f1, n1[0] * f0 + n1[1] * f1};
}

__device__ __forceinline__ void store_merged2(const MergeArgs& a, int th, int d, f32x2 num, float den, float m,
                                              bool write_lse) {
  const f32x2 o = den > 0.f ? num * (1.f / den) : f32x2{0.f, 0.f};
  if (a.out_bf16)
    *reinterpret_cast<bf16x2*>(static_cast<__bf16*>(a.out) + (int64_t)th * a.dh + d) = bf16x2{(__bf16)o[0], (__bf16)o[1]};
  else
    *reinterpret_cast<f32x2*>(static_cast<float*>(a.out) + (int64_t)th * a.dh + d) = o;
  if (a.out_lse && write_lse) a.out_lse[th] = den > 0.f ? m + __logf(den) : -INFINITY;
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
  const float* lse = a.partial_lse + (int64_t)th * a.s_max;
  if constexpr (std::is_same<T, __bf16>::value) {
    // lane pair (j, j + 32) owns d = 64 * slice + 2j, +1; half h takes every other split
    const int h = lane >> 5, j = lane & 31;
    const int d = slice * 64 + 2 * j;
    const __bf16* po = static_cast<const __bf16*>(a.partial_o) + (int64_t)th * a.s_max * a.dh + d;
    float m = -INFINITY, den = 0.f;
    f32x2 num = {0.f, 0.f};
    if constexpr (WPU == 1) {
      accumulate2<2>(lse, po, a.dh, h, ns, m, num, den);
      combine_halves(m, num, den);
      if (h == 0) store_merged2(a, th, d, num, den, m, slice == 0 && j == 0);
    } else {
      __shared__ f32x2 num_s[4][32];
      __shared__ float den_s[4], m_s[4];
      accumulate2<8>(lse, po, a.dh, 2 * wave + h, ns, m, num, den);
      combine_halves(m, num, den);
      if (h == 0) num_s[wave][j] = num;
      if (lane == 0) {
        den_s[wave] = den;
        m_s[wave] = m;
      }
      __syncthreads();
      if (wave != 0 || h != 0) return;
      const float mall = fmaxf(fmaxf(m_s[0], m_s[1]), fmaxf(m_s[2], m_s[3]));
      num = f32x2{0.f, 0.f};
      den = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = m_s[w] == -INFINITY ? 0.f : __expf(m_s[w] - mall);
        num += num_s[w][j] * f;
        den += den_s[w] * f;
      }
      store_merged2(a, th, d, num, den, mall, slice == 0 && j == 0);
    }
    return;
  }
  const int d = slice * 64 + lane;
  const float* po = static_cast<const float*>(a.partial_o) + (int64_t)th * a.s_max * a.dh + d;
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
