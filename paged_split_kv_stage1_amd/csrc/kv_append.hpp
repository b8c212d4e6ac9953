// Device launch of the KV append (new tokens' K/V rows into their paged-cache slots),
// shared by the host API and the kernel file.
#pragma once

#include <cstdint>

namespace pa {

struct AppendArgs {
  const void* k_new; const void* v_new; const int64_t* slots;
  void* k_cache; void* v_cache; float* k_scale; float* v_scale;
  int64_t n_tokens; int hkv; int page_shift;
  int64_t kv_sp, kv_sh, kv_ss;        // cache element strides (page, head, slot)
  int64_t sc_sp, sc_sh, sc_ss;        // scale element strides (per-token-head)
};
// mode: 0 bf16 cache, 1 FP8 with per-tensor scales, 2 FP8 with per-token-head scales
int launch_append(const AppendArgs& a, int src_bf16, int head_dim, int mode, void* stream);

}  // namespace pa
