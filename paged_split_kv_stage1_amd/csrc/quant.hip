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
// Memory access: a row of D elements is LPR lanes x EPL consecutive elements (EPL = 8,
// or D/64 for D >= 512): 16-byte loads of bf16 (two of fp32) and 8-byte code stores.  A
// wave takes U groups of 64/LPR consecutive rows and issues the loads of all of them
// before it encodes the first, so that enough bytes are in flight per CU to stream at
// HBM rate.  Every row is read once and every code written once, so loads and stores
// carry the non-temporal hint (with dirty lines left in L2 by earlier writes, plain
// loads stream at about two thirds of the rate).
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kv_append.hpp"

namespace pa {

template <bool BF16SRC>
__device__ __forceinline__ void load8(const void* src, int64_t i, float* x) {
  if constexpr (BF16SRC) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(src) + i));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(static_cast<const float*>(src) + i));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(static_cast<const float*>(src) + i + 4));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = a[k];
      x[4 + k] = b[k];
    }
  }
}

// BIG: U = 4 row groups per wave (2 for D = 1024) on inputs that fill the chip several
// times over; otherwise U = 1, so that small inputs still spread over many workgroups.
template <int D, bool BIG>
struct RowShape {
  static constexpr int EPL = D >= 512 ? D / 64 : 8;   // elements per lane
  static constexpr int LPR = D / EPL;                 // lanes per row
  static constexpr int RPW = 64 / LPR;                // rows per wave and group
  static constexpr int U = BIG ? (EPL == 8 ? 4 : 2) : 1;
  static constexpr int ROWS_PER_BLOCK = 4 * RPW * U;
};

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

// INT8 codes: scale = amax / 127, code = round-half-even(clamp(x / scale, -127, 127))
// with the same correctly rounded quotient.
__device__ __forceinline__ float scale_of_i8(float amax) { return amax == 0.f ? 1.0f : amax / 127.0f; }
__device__ __forceinline__ uint2 encode8_i8(const float* x, float sc, float inv) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float q = fminf(fmaxf(div_rn(x[k], sc, inv), -127.0f), 127.0f);
    w[k >> 2] |= ((uint32_t)(int)__builtin_rintf(q) & 0xFFu) << (8 * (k & 3));
  }
  return uint2{w[0], w[1]};
}
template <bool I8>
__device__ __forceinline__ float scale_fmt(float amax) {
  if constexpr (I8) return scale_of_i8(amax);
  else return scale_of(amax);
}
template <bool I8>
__device__ __forceinline__ uint2 encode_fmt(const float* x, float sc, float inv) {
  if constexpr (I8) return encode8_i8(x, sc, inv);
  else return encode8(x, sc, inv);
}

// Streaming stores: 8 codes, 8 bf16.
__device__ __forceinline__ void store_codes(uint8_t* p, uint2 c) {
  __builtin_nontemporal_store((uint64_t)c.x | ((uint64_t)c.y << 32), reinterpret_cast<uint64_t*>(p));
}
__device__ __forceinline__ void store_bf16x8(uint16_t* p, bf16x8 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(p));
}

// Per-row scales.  Rows past the end load the last row (branch-free loads) and store
// nothing.
template <bool BF16SRC, int D, bool BIG, bool I8 = false>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* src, int64_t n_rows, uint8_t* dst,
                                                         float* scale) {
  using S = RowShape<D, BIG>;
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (S::RPW * S::U) + lane / S::LPR;
  const int part = lane % S::LPR;
  float x[S::U][S::EPL];
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    const int64_t row = min(row0 + u * S::RPW, n_rows - 1);
#pragma unroll
    for (int c = 0; c < S::EPL / 8; ++c)
      load8<BF16SRC>(src, row * D + (int64_t)part * S::EPL + 8 * c, x[u] + 8 * c);
  }
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) amax = fmaxf(amax, fabsf(x[u][e]));
#pragma unroll
    for (int off = S::LPR / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const int64_t row = row0 + u * S::RPW;
    if (row >= n_rows) continue;
    const float sc = scale_fmt<I8>(amax);
    const float inv = 1.0f / sc;                          // IEEE divide, once per row
#pragma unroll
    for (int c = 0; c < S::EPL / 8; ++c)
      store_codes(dst + row * D + (int64_t)part * S::EPL + 8 * c, encode_fmt<I8>(x[u] + 8 * c, sc, inv));
    if (part == 0) scale[row] = sc;
  }
}

__global__ void zero_word_kernel(float* p) { *p = 0.f; }

// Per-tensor amax over n elements (n a multiple of 8), TENSOR_U 8-element groups in flight
// per lane over a grid-stride loop.  The four wave maxima of a workgroup meet in LDS and
// one atomic max per workgroup goes to the word (atomics on one address serialise, so
// one per wave would cost more than the streaming at the end of the pass).
constexpr int TENSOR_U = 4;

template <bool BF16SRC>
__global__ __launch_bounds__(256) void amax_kernel(const void* src, int64_t n, float* amax_word) {
  const int64_t groups = n / 8;
  const int64_t stride = (int64_t)gridDim.x * 256;
  float m = 0.f;
  int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; gi + (TENSOR_U - 1) * stride < groups; gi += TENSOR_U * stride) {
    float x[TENSOR_U][8];
#pragma unroll
    for (int u = 0; u < TENSOR_U; ++u) load8<BF16SRC>(src, (gi + u * stride) * 8, x[u]);
#pragma unroll
    for (int u = 0; u < TENSOR_U; ++u)
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
  __shared__ float wave_max[4];
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
    // non-negative floats order like their bit patterns
    atomicMax(reinterpret_cast<unsigned int*>(amax_word), __float_as_uint(m));
  }
}

template <bool BF16SRC, bool I8 = false>
__global__ __launch_bounds__(256) void quant_tensor_kernel(const void* src, int64_t n, uint8_t* dst,
                                                           const float* amax_word) {
  const float sc = scale_fmt<I8>(*amax_word);
  const float inv = 1.0f / sc;
  const int64_t groups = n / 8;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; gi + (TENSOR_U - 1) * stride < groups; gi += TENSOR_U * stride) {
    float x[TENSOR_U][8];
#pragma unroll
    for (int u = 0; u < TENSOR_U; ++u) load8<BF16SRC>(src, (gi + u * stride) * 8, x[u]);
#pragma unroll
    for (int u = 0; u < TENSOR_U; ++u) store_codes(dst + (gi + u * stride) * 8, encode_fmt<I8>(x[u], sc, inv));
  }
  for (; gi < groups; gi += stride) {
    float x[8];
    load8<BF16SRC>(src, gi * 8, x);
    store_codes(dst + gi * 8, encode_fmt<I8>(x, sc, inv));
  }
}

template <bool I8 = false>
__global__ void finish_scale_kernel(float* scale) { scale[0] = scale_fmt<I8>(scale[0]); }

constexpr unsigned kBigGrid = 2048;      // 8 workgroups per CU: enough to take U = 4

template <int D, bool BIG>
static unsigned grid_of(int64_t n_rows) {
  constexpr int per = RowShape<D, BIG>::ROWS_PER_BLOCK;
  return (unsigned)((n_rows + per - 1) / per);
}

template <bool BF16SRC, int D, bool I8 = false>
static void launch_rows_d(const void* src, int64_t n_rows, uint8_t* dst, float* scale, hipStream_t s) {
  const unsigned big = grid_of<D, true>(n_rows);
  if (big >= kBigGrid)
    hipLaunchKernelGGL((quant_rows_kernel<BF16SRC, D, true, I8>), dim3(big), dim3(256), 0, s, src, n_rows, dst, scale);
  else
    hipLaunchKernelGGL((quant_rows_kernel<BF16SRC, D, false, I8>), dim3(grid_of<D, false>(n_rows)), dim3(256), 0, s,
                       src, n_rows, dst, scale);
}

template <bool BF16SRC, bool I8 = false>
static int launch_rows(const void* src, int64_t n_rows, int head_dim, uint8_t* dst, float* scale, hipStream_t s) {
  switch (head_dim) {
    case 64: launch_rows_d<BF16SRC, 64, I8>(src, n_rows, dst, scale, s); break;
    case 128: launch_rows_d<BF16SRC, 128, I8>(src, n_rows, dst, scale, s); break;
    case 256: launch_rows_d<BF16SRC, 256, I8>(src, n_rows, dst, scale, s); break;
    case 512: launch_rows_d<BF16SRC, 512, I8>(src, n_rows, dst, scale, s); break;
    case 1024: launch_rows_d<BF16SRC, 1024, I8>(src, n_rows, dst, scale, s); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

template <bool BF16SRC, bool I8 = false>
static int launch_tensor(const void* src, int64_t n, uint8_t* dst, float* scale, hipStream_t s) {
  const int64_t want = (n / 8 + 255) / 256;
  const unsigned blocks = (unsigned)(want < 1024 ? (want > 0 ? want : 1) : 1024);   // 4 per CU
  hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(1), 0, s, scale);
  hipLaunchKernelGGL((amax_kernel<BF16SRC>), dim3(blocks), dim3(256), 0, s, src, n, scale);
  hipLaunchKernelGGL((quant_tensor_kernel<BF16SRC, I8>), dim3(blocks), dim3(256), 0, s, src, n, dst, scale);
  hipLaunchKernelGGL(finish_scale_kernel<I8>, dim3(1), dim3(1), 0, s, scale);
  return (int)hipGetLastError();
}

// ---- per-head scales ---------------------------------------------------------------------
// Rows of [n_tokens, H, D]; row r belongs to head r % H, and head h's scale is the amax over
// all of its rows / 448 (FlashInfer PR #869, per-head quantization).  Three launches: the
// per-head amax (a fixed grid striding over the rows; row maxima meet per head in LDS and
// one atomic per head and workgroup goes to global memory), the encode (the per-row
// quantiser with the row's head scale), and the finish that turns the amax words into
// scales.  H <= kMaxHeads.
constexpr int kMaxHeads = 1024;

__global__ void zero_words_kernel(float* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0.f;
}

template <bool BF16SRC, int D>
__global__ __launch_bounds__(256) void amax_heads_kernel(const void* src, int64_t n_rows, int H, float* amax_words) {
  using S = RowShape<D, true>;
  __shared__ unsigned int hmax[kMaxHeads];
  for (int t = threadIdx.x; t < H; t += 256) hmax[t] = 0u;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int part = lane % S::LPR;
  for (int64_t base = (int64_t)blockIdx.x * S::ROWS_PER_BLOCK; base < n_rows;
       base += (int64_t)gridDim.x * S::ROWS_PER_BLOCK) {
    const int64_t row0 = base + (threadIdx.x >> 6) * (S::RPW * S::U) + lane / S::LPR;
    float x[S::U][S::EPL];
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      const int64_t row = min(row0 + u * S::RPW, n_rows - 1);
#pragma unroll
      for (int c = 0; c < S::EPL / 8; ++c)
        load8<BF16SRC>(src, row * D + (int64_t)part * S::EPL + 8 * c, x[u] + 8 * c);
    }
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < S::EPL; ++e) amax = fmaxf(amax, fabsf(x[u][e]));
#pragma unroll
      for (int off = S::LPR / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
      const int64_t row = row0 + u * S::RPW;
      // non-negative floats order like their bit patterns
      if (part == 0 && row < n_rows) atomicMax(&hmax[row % H], __float_as_uint(amax));
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < H; t += 256)
    if (hmax[t] != 0u) atomicMax(reinterpret_cast<unsigned int*>(amax_words) + t, hmax[t]);
}

template <bool BF16SRC, int D, bool BIG>
__global__ __launch_bounds__(256) void encode_heads_kernel(const void* src, int64_t n_rows, int H, uint8_t* dst,
                                                           const float* amax_words) {
  using S = RowShape<D, BIG>;
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (S::RPW * S::U) + lane / S::LPR;
  const int part = lane % S::LPR;
  float x[S::U][S::EPL];
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    const int64_t row = min(row0 + u * S::RPW, n_rows - 1);
#pragma unroll
    for (int c = 0; c < S::EPL / 8; ++c)
      load8<BF16SRC>(src, row * D + (int64_t)part * S::EPL + 8 * c, x[u] + 8 * c);
  }
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    const int64_t row = row0 + u * S::RPW;
    if (row >= n_rows) continue;
    const float sc = scale_of(amax_words[row % H]);
    const float inv = 1.0f / sc;
#pragma unroll
    for (int c = 0; c < S::EPL / 8; ++c)
      store_codes(dst + row * D + (int64_t)part * S::EPL + 8 * c, encode8(x[u] + 8 * c, sc, inv));
  }
}

__global__ void finish_scales_kernel(float* scale, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) scale[i] = scale_of(scale[i]);
}

template <bool BF16SRC, int D>
static void launch_heads_d(const void* src, int64_t n_rows, int H, uint8_t* dst, float* scale, hipStream_t s) {
  const unsigned amax_blocks = std::min(grid_of<D, true>(n_rows), 1024u);   // 4 per CU
  hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(1024), 0, s, scale, H);
  hipLaunchKernelGGL((amax_heads_kernel<BF16SRC, D>), dim3(amax_blocks), dim3(256), 0, s, src, n_rows, H, scale);
  const unsigned big = grid_of<D, true>(n_rows);
  if (big >= kBigGrid)
    hipLaunchKernelGGL((encode_heads_kernel<BF16SRC, D, true>), dim3(big), dim3(256), 0, s, src, n_rows, H, dst,
                       scale);
  else
    hipLaunchKernelGGL((encode_heads_kernel<BF16SRC, D, false>), dim3(grid_of<D, false>(n_rows)), dim3(256), 0, s,
                       src, n_rows, H, dst, scale);
  hipLaunchKernelGGL(finish_scales_kernel, dim3(1), dim3(1024), 0, s, scale, H);
}

int launch_quant_heads(const void* src, int src_bf16, int64_t n_tokens, int num_heads, int head_dim, uint8_t* dst,
                       float* scale, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (n_tokens <= 0) return 0;
  const int64_t n_rows = n_tokens * num_heads;
  auto go = [&](auto bf16_c) {
    constexpr bool B = decltype(bf16_c)::value;
    switch (head_dim) {
      case 64: launch_heads_d<B, 64>(src, n_rows, num_heads, dst, scale, s); break;
      case 128: launch_heads_d<B, 128>(src, n_rows, num_heads, dst, scale, s); break;
      case 256: launch_heads_d<B, 256>(src, n_rows, num_heads, dst, scale, s); break;
      case 512: launch_heads_d<B, 512>(src, n_rows, num_heads, dst, scale, s); break;
      case 1024: launch_heads_d<B, 1024>(src, n_rows, num_heads, dst, scale, s); break;
      default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
  };
  return src_bf16 ? go(std::true_type{}) : go(std::false_type{});
}

// ---- KV append -------------------------------------------------------------------------
// Rows of the new tokens' K (first n_tokens * hkv rows) then V, laid out like the
// quantiser's rows, each written to its token's slot in the paged cache.  MODE: 0 bf16
// cache, 1 FP8 with the caches' per-tensor scales (per-head: indexed by the KV head),
// 2 FP8 with per-token-head scales.
// Row indices fit in 32 bits (the host checks 2 * n_tokens * hkv < 2^31).  Rows of
// skipped tokens (negative slot) and rows past the end still load a row (the last one,
// past the end) so that the loads stay branch-free, and store nothing.
template <bool BF16SRC, int D, int MODE, bool BIG, bool I8 = false>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  using S = RowShape<D, BIG>;
  const int lane = threadIdx.x & 63;
  const uint32_t hkv = (uint32_t)a.hkv;
  const uint32_t per = (uint32_t)a.n_tokens * hkv;
  const uint32_t row0 = ((uint32_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (S::RPW * S::U) + lane / S::LPR;
  const int part = lane % S::LPR;
  float x[S::U][S::EPL];
  int64_t slot[S::U];
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    const uint32_t row = min(row0 + u * S::RPW, 2 * per - 1);
    const bool is_v = row >= per;
    const uint32_t rr = is_v ? row - per : row;          // token * hkv + head
    slot[u] = row0 + u * S::RPW < 2 * per ? a.slots[rr / hkv] : -1;
    const void* src = is_v ? a.v_new : a.k_new;
#pragma unroll
    for (int c = 0; c < S::EPL / 8; ++c)
      load8<BF16SRC>(src, (int64_t)rr * D + part * S::EPL + 8 * c, x[u] + 8 * c);
  }
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    float amax = 0.f;
    if constexpr (MODE == 2) {
#pragma unroll
      for (int e = 0; e < S::EPL; ++e) amax = fmaxf(amax, fabsf(x[u][e]));
#pragma unroll
      for (int off = S::LPR / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    }
    if (slot[u] < 0) continue;
    const uint32_t row = row0 + u * S::RPW;
    const bool is_v = row >= per;
    const uint32_t rr = is_v ? row - per : row;
    const uint32_t h = rr % hkv;
    const int64_t page = slot[u] >> a.page_shift;
    const int64_t s_in = slot[u] & ((1 << a.page_shift) - 1);
    const int64_t off = page * a.kv_sp + (int64_t)h * a.kv_sh + s_in * a.kv_ss + part * S::EPL;
    if constexpr (MODE == 0) {
      uint16_t* dst = static_cast<uint16_t*>(is_v ? a.v_cache : a.k_cache) + off;
#pragma unroll
      for (int c = 0; c < S::EPL / 8; ++c) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)x[u][8 * c + e];   // exact for bf16, RNE for fp32
        store_bf16x8(dst + 8 * c, v);
      }
    } else {
      float sc;
      if constexpr (MODE == 1) sc = (is_v ? a.v_scale : a.k_scale)[h * a.scale_hstride];
      else sc = scale_fmt<I8>(amax);
      const float inv = 1.0f / sc;
      uint8_t* dst = static_cast<uint8_t*>(is_v ? a.v_cache : a.k_cache) + off;
#pragma unroll
      for (int c = 0; c < S::EPL / 8; ++c) store_codes(dst + 8 * c, encode_fmt<I8>(x[u] + 8 * c, sc, inv));
      if constexpr (MODE == 2) {
        if (part == 0)
          (is_v ? a.v_scale : a.k_scale)[page * a.sc_sp + (int64_t)h * a.sc_sh + s_in * a.sc_ss] = sc;
      }
    }
  }
}

template <bool BF16SRC, int D, int MODE, bool I8>
static void launch_append_d(const AppendArgs& a, hipStream_t s) {
  const int64_t rows = 2 * a.n_tokens * a.hkv;
  const unsigned big = grid_of<D, true>(rows);
  if (big >= kBigGrid)
    hipLaunchKernelGGL((append_kernel<BF16SRC, D, MODE, true, I8>), dim3(big), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((append_kernel<BF16SRC, D, MODE, false, I8>), dim3(grid_of<D, false>(rows)), dim3(256), 0, s, a);
}

template <bool BF16SRC, int MODE, bool I8>
static int launch_append_mode(const AppendArgs& a, int head_dim, hipStream_t s) {
  switch (head_dim) {
    case 64: launch_append_d<BF16SRC, 64, MODE, I8>(a, s); break;
    case 128: launch_append_d<BF16SRC, 128, MODE, I8>(a, s); break;
    case 256: launch_append_d<BF16SRC, 256, MODE, I8>(a, s); break;
    case 512: launch_append_d<BF16SRC, 512, MODE, I8>(a, s); break;
    case 1024: launch_append_d<BF16SRC, 1024, MODE, I8>(a, s); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_append(const AppendArgs& a, int src_bf16, int head_dim, int mode, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.n_tokens <= 0) return 0;
  auto go = [&](auto bf16_c, auto i8_c) {
    constexpr bool B = decltype(bf16_c)::value, I = decltype(i8_c)::value;
    if (mode == 0) return launch_append_mode<B, 0, false>(a, head_dim, s);
    if (mode == 1) return launch_append_mode<B, 1, I>(a, head_dim, s);
    return launch_append_mode<B, 2, I>(a, head_dim, s);
  };
  if (src_bf16) return a.i8 ? go(std::true_type{}, std::true_type{}) : go(std::true_type{}, std::false_type{});
  return a.i8 ? go(std::false_type{}, std::true_type{}) : go(std::false_type{}, std::false_type{});
}

int launch_quant(const void* src, int src_bf16, int64_t n_rows, int head_dim, int per_tensor, int i8, uint8_t* dst,
                 float* scale, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (n_rows <= 0) return 0;
  auto go = [&](auto bf16_c, auto i8_c) {
    constexpr bool B = decltype(bf16_c)::value, I = decltype(i8_c)::value;
    if (per_tensor) return launch_tensor<B, I>(src, n_rows * head_dim, dst, scale, s);
    return launch_rows<B, I>(src, n_rows, head_dim, dst, scale, s);
  };
  if (src_bf16) return i8 ? go(std::true_type{}, std::true_type{}) : go(std::true_type{}, std::false_type{});
  return i8 ? go(std::false_type{}, std::true_type{}) : go(std::false_type{}, std::false_type{});
}

}  // namespace pa
