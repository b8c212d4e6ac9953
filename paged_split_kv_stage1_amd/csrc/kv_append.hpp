// Device launches of the cache-side operations that the host API and the kernel file
// share: the KV append (new tokens' K/V rows into their paged-cache slots) and the
// per-head quantiser.
#pragma once

#include <cstdint>

namespace pa {

struct AppendArgs {
  const void* k_new; const void* v_new; const int64_t* slots;
  void* k_cache; void* v_cache; float* k_scale; float* v_scale;
  int64_t n_tokens; int hkv; int page_shift;
  int64_t kv_sp, kv_sh, kv_ss;        // cache element strides (page, head, slot)
  int64_t sc_sp, sc_sh, sc_ss;        // scale element strides (per-token-head)
  int scale_hstride;                  // mode 1: 1 = per-head scales [Hkv], 0 = one scale
  int i8;                             // modes 1, 2: INT8 codes instead of e4m3
};
// mode: 0 bf16 cache, 1 FP8 with per-tensor scales, 2 FP8 with per-token-head scales
int launch_append(const AppendArgs& a, int src_bf16, int head_dim, int mode, void* stream);
// Per-head FP8 quantiser: src [n_tokens, num_heads, head_dim] -> codes, scale[num_heads].
int launch_quant_heads(const void* src, int src_bf16, int64_t n_tokens, int num_heads, int head_dim, uint8_t* dst,
                       float* scale, void* stream);

}  // namespace pa
