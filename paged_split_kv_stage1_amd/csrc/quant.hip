// FP8 (OCP E4M3FN) quantiser for KV (and per-tensor Q): scale = amax / 448 over a
// row (one (token, KV head) vector; FreeToken PR #900 "fp8_per_token_head") or over
// the whole tensor (FlashMLA PR #54, symmetric per-tensor), codes =
// RNE(clamp(x / scale, -448, 448)).  The hardware fp32 -> e4m3 conversion rounds
// to nearest even without saturating, hence the clamp first.
#include "common.hpp"

namespace pa {

template <bool BF16SRC>
__device__ __forceinline__ float load_src(const void* src, int64_t i) {
  if constexpr (BF16SRC) return (float)static_cast<const __bf16*>(src)[i];
  else return static_cast<const float*>(src)[i];
}

__device__ __forceinline__ uint8_t encode_e4m3(float x, float scale) {
  float y = x / scale;                                     // IEEE fp32 divide
  y = fminf(fmaxf(y, -448.0f), 448.0f);
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, 0, false) & 0xFF);
}

__device__ __forceinline__ float scale_of(float amax) { return amax == 0.f ? 1.0f : amax / 448.0f; }

// one wave per row; EPL elements per lane (head_dim = 64 * EPL)
template <bool BF16SRC, int EPL>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* src, int64_t n_rows, uint8_t* dst,
                                                         float* scale) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;
  constexpr int D = 64 * EPL;
  float x[EPL];
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    x[e] = load_src<BF16SRC>(src, row * D + lane * EPL + e);
    amax = fmaxf(amax, fabsf(x[e]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float sc = scale_of(amax);
#pragma unroll
  for (int e = 0; e < EPL; ++e) dst[row * D + lane * EPL + e] = encode_e4m3(x[e], sc);
  if (lane == 0) scale[row] = sc;
}

__global__ void zero_word_kernel(float* p) { *p = 0.f; }

template <bool BF16SRC>
__global__ __launch_bounds__(256) void amax_kernel(const void* src, int64_t n, float* amax_word) {
  float m = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    m = fmaxf(m, fabsf(load_src<BF16SRC>(src, i)));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  // non-negative floats order like their bit patterns
  if ((threadIdx.x & 63) == 0) atomicMax(reinterpret_cast<unsigned int*>(amax_word), __float_as_uint(m));
}

template <bool BF16SRC>
__global__ __launch_bounds__(256) void quant_tensor_kernel(const void* src, int64_t n, uint8_t* dst,
                                                           const float* amax_word) {
  const float sc = scale_of(*amax_word);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = encode_e4m3(load_src<BF16SRC>(src, i), sc);
}

__global__ void finish_scale_kernel(float* scale) { scale[0] = scale_of(scale[0]); }

template <bool BF16SRC>
static int launch_rows(const void* src, int64_t n_rows, int head_dim, uint8_t* dst, float* scale, hipStream_t s) {
  const unsigned blocks = (unsigned)((n_rows + 3) / 4);
  switch (head_dim / 64) {
    case 1: hipLaunchKernelGGL((quant_rows_kernel<BF16SRC, 1>), dim3(blocks), dim3(256), 0, s, src, n_rows, dst, scale); break;
    case 2: hipLaunchKernelGGL((quant_rows_kernel<BF16SRC, 2>), dim3(blocks), dim3(256), 0, s, src, n_rows, dst, scale); break;
    case 4: hipLaunchKernelGGL((quant_rows_kernel<BF16SRC, 4>), dim3(blocks), dim3(256), 0, s, src, n_rows, dst, scale); break;
    case 8: hipLaunchKernelGGL((quant_rows_kernel<BF16SRC, 8>), dim3(blocks), dim3(256), 0, s, src, n_rows, dst, scale); break;
    case 16: hipLaunchKernelGGL((quant_rows_kernel<BF16SRC, 16>), dim3(blocks), dim3(256), 0, s, src, n_rows, dst, scale); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

template <bool BF16SRC>
static int launch_tensor(const void* src, int64_t n, uint8_t* dst, float* scale, hipStream_t s) {
  const int64_t want = (n + 255) / 256;
  const unsigned blocks = (unsigned)(want < 4096 ? (want > 0 ? want : 1) : 4096);
  hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(1), 0, s, scale);
  hipLaunchKernelGGL((amax_kernel<BF16SRC>), dim3(blocks), dim3(256), 0, s, src, n, scale);
  hipLaunchKernelGGL((quant_tensor_kernel<BF16SRC>), dim3(blocks), dim3(256), 0, s, src, n, dst, scale);
  hipLaunchKernelGGL(finish_scale_kernel, dim3(1), dim3(1), 0, s, scale);
  return (int)hipGetLastError();
}

int launch_quant(const void* src, int src_bf16, int64_t n_rows, int head_dim, int per_tensor, uint8_t* dst,
                 float* scale, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (n_rows <= 0) return 0;
  if (per_tensor) {
    const int64_t n = n_rows * head_dim;
    return src_bf16 ? launch_tensor<true>(src, n, dst, scale, s) : launch_tensor<false>(src, n, dst, scale, s);
  }
  return src_bf16 ? launch_rows<true>(src, n_rows, head_dim, dst, scale, s)
                  : launch_rows<false>(src, n_rows, head_dim, dst, scale, s);
}

}  // namespace pa
