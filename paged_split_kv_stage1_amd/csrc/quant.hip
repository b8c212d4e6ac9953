// FP8 (OCP E4M3FN) quantiser for KV (and per-tensor Q): scale = amax / 448 over a
// row (one (token, KV head) vector; FreeToken PR #900 "fp8_per_token_head") or over
// the whole tensor (FlashMLA PR #54, symmetric per-tensor), codes =
// RNE(clamp(x / scale, -448, 448)).  The hardware fp32 -> e4m3 conversion rounds
// to nearest even without saturating, hence the clamp first.
//
// The quotient x / scale must be the IEEE fp32 one (the codes are compared bit for bit
// with a reference that divides).  Instead of a full division per element, each row's
// reciprocal y = RN(1/scale) is divided once and every element takes Markstein's
// correction step q = RN(q0 + RN(x - q0*scale)*y) with q0 = RN(x*y): for
// round-to-nearest and a normal quotient this is the correctly rounded x / scale.  A
// subnormal quotient is far below e4m3's smallest step and encodes to zero either
// way; the sign is copied from x so that -0 keeps its code.
//
// Memory access: 8 consecutive elements per lane (16-byte loads of bf16, two of fp32)
// and 8-byte code stores.
#include "common.hpp"
#include "kv_append.hpp"

namespace pa {

template <bool BF16SRC>
__device__ __forceinline__ void load8(const void* src, int64_t i, float* x) {
  if constexpr (BF16SRC) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(src) + i);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(src) + i);
    const f32x4 b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(src) + i + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = a[k];
      x[4 + k] = b[k];
    }
  }
}

__device__ __forceinline__ float scale_of(float amax) { return amax == 0.f ? 1.0f : amax / 448.0f; }

// RN(x / b) from y = RN(1 / b) (see above)
__device__ __forceinline__ float div_rn(float x, float b, float y) {
  const float q0 = x * y;
  const float r = fmaf(-q0, b, x);
  return __builtin_copysignf(fmaf(r, y, q0), x);
}

// 8 elements -> 8 e4m3 codes (byte k = element k)
__device__ __forceinline__ uint2 encode8(const float* x, float sc, float inv) {
  float q[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) q[k] = fminf(fmaxf(div_rn(x[k], sc, inv), -448.0f), 448.0f);
  return uint2{f32x4_to_fp8x4(q[0], q[1], q[2], q[3]), f32x4_to_fp8x4(q[4], q[5], q[6], q[7])};
}

// Per-row scales.  A row of D elements is LPR lanes x EPL elements (EPL = 8, or D/64
// for D >= 512); a wave holds 64 / LPR rows and a workgroup four waves' worth.
template <bool BF16SRC, int D>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* src, int64_t n_rows, uint8_t* dst,
                                                         float* scale) {
  constexpr int EPL = D >= 512 ? D / 64 : 8;
  constexpr int LPR = D / EPL;
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const int part = lane % LPR;
  const bool live = row < n_rows;
  float x[EPL];
  float amax = 0.f;
  if (live) {
#pragma unroll
    for (int c = 0; c < EPL / 8; ++c) load8<BF16SRC>(src, row * D + (int64_t)part * EPL + 8 * c, x + 8 * c);
#pragma unroll
    for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if (!live) return;
  const float sc = scale_of(amax);
  const float inv = 1.0f / sc;                            // IEEE divide, once per row
#pragma unroll
  for (int c = 0; c < EPL / 8; ++c)
    *reinterpret_cast<uint2*>(dst + row * D + (int64_t)part * EPL + 8 * c) = encode8(x + 8 * c, sc, inv);
  if (part == 0) scale[row] = sc;
}

__global__ void zero_word_kernel(float* p) { *p = 0.f; }

// Per-tensor amax over n elements (n a multiple of 8), four 8-element groups in flight.
template <bool BF16SRC>
__global__ __launch_bounds__(256) void amax_kernel(const void* src, int64_t n, float* amax_word) {
  const int64_t groups = n / 8;
  const int64_t stride = (int64_t)gridDim.x * 256;
  float m = 0.f;
  int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; gi + 3 * stride < groups; gi += 4 * stride) {
    float x[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8<BF16SRC>(src, (gi + u * stride) * 8, x[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[u][e]));
  }
  for (; gi < groups; gi += stride) {
    float x[8];
    load8<BF16SRC>(src, gi * 8, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  // non-negative floats order like their bit patterns
  if ((threadIdx.x & 63) == 0) atomicMax(reinterpret_cast<unsigned int*>(amax_word), __float_as_uint(m));
}

template <bool BF16SRC>
__global__ __launch_bounds__(256) void quant_tensor_kernel(const void* src, int64_t n, uint8_t* dst,
                                                           const float* amax_word) {
  const float sc = scale_of(*amax_word);
  const float inv = 1.0f / sc;
  const int64_t groups = n / 8;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; gi + stride < groups; gi += 2 * stride) {
    float x[2][8];
    load8<BF16SRC>(src, gi * 8, x[0]);
    load8<BF16SRC>(src, (gi + stride) * 8, x[1]);
    *reinterpret_cast<uint2*>(dst + gi * 8) = encode8(x[0], sc, inv);
    *reinterpret_cast<uint2*>(dst + (gi + stride) * 8) = encode8(x[1], sc, inv);
  }
  for (; gi < groups; gi += stride) {
    float x[8];
    load8<BF16SRC>(src, gi * 8, x);
    *reinterpret_cast<uint2*>(dst + gi * 8) = encode8(x, sc, inv);
  }
}

__global__ void finish_scale_kernel(float* scale) { scale[0] = scale_of(scale[0]); }

template <bool BF16SRC>
static int launch_rows(const void* src, int64_t n_rows, int head_dim, uint8_t* dst, float* scale, hipStream_t s) {
  auto blocks = [&](int d) {
    const int rpw = 64 / (d / (d >= 512 ? d / 64 : 8));
    return (unsigned)((n_rows + 4 * rpw - 1) / (4 * rpw));
  };
  switch (head_dim) {
    case 64: hipLaunchKernelGGL((quant_rows_kernel<BF16SRC, 64>), dim3(blocks(64)), dim3(256), 0, s, src, n_rows, dst, scale); break;
    case 128: hipLaunchKernelGGL((quant_rows_kernel<BF16SRC, 128>), dim3(blocks(128)), dim3(256), 0, s, src, n_rows, dst, scale); break;
    case 256: hipLaunchKernelGGL((quant_rows_kernel<BF16SRC, 256>), dim3(blocks(256)), dim3(256), 0, s, src, n_rows, dst, scale); break;
    case 512: hipLaunchKernelGGL((quant_rows_kernel<BF16SRC, 512>), dim3(blocks(512)), dim3(256), 0, s, src, n_rows, dst, scale); break;
    case 1024: hipLaunchKernelGGL((quant_rows_kernel<BF16SRC, 1024>), dim3(blocks(1024)), dim3(256), 0, s, src, n_rows, dst, scale); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

template <bool BF16SRC>
static int launch_tensor(const void* src, int64_t n, uint8_t* dst, float* scale, hipStream_t s) {
  const int64_t want = (n / 8 + 255) / 256;
  const unsigned blocks = (unsigned)(want < 2048 ? (want > 0 ? want : 1) : 2048);
  hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(1), 0, s, scale);
  hipLaunchKernelGGL((amax_kernel<BF16SRC>), dim3(blocks), dim3(256), 0, s, src, n, scale);
  hipLaunchKernelGGL((quant_tensor_kernel<BF16SRC>), dim3(blocks), dim3(256), 0, s, src, n, dst, scale);
  hipLaunchKernelGGL(finish_scale_kernel, dim3(1), dim3(1), 0, s, scale);
  return (int)hipGetLastError();
}

// ---- KV append -------------------------------------------------------------------------
// Rows of the new tokens' K (first n_tokens * hkv rows) then V, laid out like the
// quantiser's rows, each written to its token's slot in the paged cache.  MODE: 0 bf16
// cache, 1 FP8 with the caches' per-tensor scales, 2 FP8 with per-token-head scales.
// Rows of skipped tokens (negative slot) and rows past the end take part in the row's
// lane shuffles but store nothing.
template <bool BF16SRC, int D, int MODE>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int EPL = D >= 512 ? D / 64 : 8;
  constexpr int LPR = D / EPL;
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int64_t per = a.n_tokens * a.hkv;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const int part = lane % LPR;
  const bool is_v = row >= per;
  const int64_t rr = is_v ? row - per : row;          // token * hkv + head
  const int64_t t = rr / a.hkv;
  const int h = (int)(rr - t * a.hkv);
  const int64_t slot = row < 2 * per ? a.slots[t] : -1;
  const bool live = slot >= 0;
  const void* src = is_v ? a.v_new : a.k_new;
  float x[EPL];
  float amax = 0.f;
  if (live) {
#pragma unroll
    for (int c = 0; c < EPL / 8; ++c) load8<BF16SRC>(src, rr * D + (int64_t)part * EPL + 8 * c, x + 8 * c);
#pragma unroll
    for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
  }
  if constexpr (MODE == 2) {
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  }
  if (!live) return;
  const int64_t page = slot >> a.page_shift;
  const int64_t s_in = slot & ((1 << a.page_shift) - 1);
  const int64_t off = page * a.kv_sp + (int64_t)h * a.kv_sh + s_in * a.kv_ss + (int64_t)part * EPL;
  if constexpr (MODE == 0) {
    uint16_t* dst = static_cast<uint16_t*>(is_v ? a.v_cache : a.k_cache) + off;
#pragma unroll
    for (int c = 0; c < EPL / 8; ++c) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (__bf16)x[8 * c + e];   // exact for bf16, RNE for fp32
      *reinterpret_cast<bf16x8*>(dst + 8 * c) = v;
    }
  } else {
    float sc;
    if constexpr (MODE == 1) sc = *(is_v ? a.v_scale : a.k_scale);
    else sc = scale_of(amax);
    const float inv = 1.0f / sc;
    uint8_t* dst = static_cast<uint8_t*>(is_v ? a.v_cache : a.k_cache) + off;
#pragma unroll
    for (int c = 0; c < EPL / 8; ++c) *reinterpret_cast<uint2*>(dst + 8 * c) = encode8(x + 8 * c, sc, inv);
    if constexpr (MODE == 2) {
      if (part == 0)
        (is_v ? a.v_scale : a.k_scale)[page * a.sc_sp + (int64_t)h * a.sc_sh + s_in * a.sc_ss] = sc;
    }
  }
}

template <bool BF16SRC, int MODE>
static int launch_append_mode(const AppendArgs& a, int head_dim, hipStream_t s) {
  const int64_t rows = 2 * a.n_tokens * a.hkv;
  auto blocks = [&](int d) {
    const int rpw = 64 / (d / (d >= 512 ? d / 64 : 8));
    return (unsigned)((rows + 4 * rpw - 1) / (4 * rpw));
  };
  switch (head_dim) {
    case 64: hipLaunchKernelGGL((append_kernel<BF16SRC, 64, MODE>), dim3(blocks(64)), dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL((append_kernel<BF16SRC, 128, MODE>), dim3(blocks(128)), dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL((append_kernel<BF16SRC, 256, MODE>), dim3(blocks(256)), dim3(256), 0, s, a); break;
    case 512: hipLaunchKernelGGL((append_kernel<BF16SRC, 512, MODE>), dim3(blocks(512)), dim3(256), 0, s, a); break;
    case 1024: hipLaunchKernelGGL((append_kernel<BF16SRC, 1024, MODE>), dim3(blocks(1024)), dim3(256), 0, s, a); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_append(const AppendArgs& a, int src_bf16, int head_dim, int mode, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.n_tokens <= 0) return 0;
  if (src_bf16) {
    if (mode == 0) return launch_append_mode<true, 0>(a, head_dim, s);
    if (mode == 1) return launch_append_mode<true, 1>(a, head_dim, s);
    return launch_append_mode<true, 2>(a, head_dim, s);
  }
  if (mode == 0) return launch_append_mode<false, 0>(a, head_dim, s);
  if (mode == 1) return launch_append_mode<false, 1>(a, head_dim, s);
  return launch_append_mode<false, 2>(a, head_dim, s);
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
