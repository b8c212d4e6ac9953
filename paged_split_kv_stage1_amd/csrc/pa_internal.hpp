// Internal definitions shared by the host planner/dispatcher and the gfx950 kernels.
#pragma once
#include <stdint.h>

namespace pa {

// One stage-1 work item: (request, KV head, split).  64 bytes, int32 fields.
struct PaItem {
  int32_t row0;       // first query row of the request (qo_indptr[b])
  int32_t nrows;      // query rows of the request
  int32_t kv_len;     // tokens of the request
  int32_t page_base;  // kv_indptr[b]
  int32_t window;     // sliding window (0 = none)
  int32_t kvh;        // KV head
  int32_t split;      // split index within the request
  int32_t nsplit;     // splits of the request (1 => write the final output)
  int32_t tok_begin;  // token range [tok_begin, tok_end) of this split
  int32_t tok_end;
  int32_t req;        // request index
  int32_t qblk0;      // first 16-row query block (of the request's rows x heads) this item runs
  int32_t pad[4];
};
static_assert(sizeof(PaItem) == 64, "PaItem must be 64 bytes");

// Plan buffer layout: PaItem items[num_items]; int32 row_nsplit[total_rows].
inline int64_t plan_bytes_for(int64_t items, int64_t rows) { return items * 64 + rows * 4; }

// Tile configuration of a stage-1 launch (packed into pa_plan_info.variant).
struct KernelCfg {
  int dh;        // key width: 128, 256 or 512; with kr, dv + 64
  int qf8;       // q is e4m3 (fp8 MFMA for q.k)
  int kvf8;      // KV holds one-byte codes (e4m3, or int8 with i8)
  int i8;        // KV codes are int8
  int pt;        // per-(token, KV head) scales
  int wq;        // waves splitting the 16-row query blocks (1, 2, 4); 4/wq waves split tokens
  int nqb;       // 16-row query blocks per wave
  int kr = 0;    // keys of dv + 64 channels with a 64-channel rotary part (stage1_kr.hip)
  int mla = 0;   // with kr: MLA-style latent cache (value = latent, e4m3 per 128 channels)
  int dv = 0;    // value width (= dh unless kr)
  int qm = 0;    // query rows on the MFMA M axis (S = Q K^T) instead of the key tokens
};
inline int32_t pack_cfg(const KernelCfg& c) {
  return (c.dh == 256 ? 1 : 0) | (c.qf8 << 1) | (c.kvf8 << 2) | (c.pt << 3) | (c.wq << 4) | (c.nqb << 8) |
         (c.i8 << 12) | ((c.dh == 512 ? 1 : 0) << 13) | (c.kr << 14) | (c.mla << 15) | (c.qm << 16);
}
inline KernelCfg unpack_cfg(int32_t v) {
  KernelCfg c;
  c.dh = ((v >> 13) & 1) ? 512 : ((v & 1) ? 256 : 128); c.qf8 = (v >> 1) & 1; c.kvf8 = (v >> 2) & 1; c.pt = (v >> 3) & 1;
  c.wq = (v >> 4) & 15; c.nqb = (v >> 8) & 15; c.i8 = (v >> 12) & 1;
  c.kr = (v >> 14) & 1; c.mla = (v >> 15) & 1; c.qm = (v >> 16) & 1;
  c.dv = c.dh;
  if (c.kr) {
    c.dv = c.mla ? 512 : 128;
    c.dh = c.dv + 64;
  }
  return c;
}

constexpr int kSplitAlign = 64;     // split boundaries are multiples of this many tokens
constexpr int kMaxSplits = 1024;

struct Stage1Args {
  const PaItem* items;
  const void* q; const float* q_scale;
  const void* k; const void* v;
  int64_t kv_sp, kv_sh, kv_ss;          // element strides (page, head, slot)
  const float* k_scale; const float* v_scale;
  int64_t sc_sp, sc_sh, sc_ss;
  int scale_per_head;                   // 1: k/v_scale[Hkv] and, for FP8 Q, q_scale[Hq]; 0: scalars
  const int32_t* page_indices;
  float sm_scale;
  void* partial_o; float* partial_lse;  // partial O: float32, or bf16 when part_bf16
  void* out; int out_bf16;
  float* out_lse;                       // LSE of rows whose request has one split, or NULL
  int hq, group, page_shift, s_max;
  int part_bf16;
  int fair;                             // every item runs at once (at most two per CU)
};

// Stage 1 of keys with a 64-channel rotary part (stage1_kr.hip).
struct KrArgs {
  const PaItem* items;
  const void* q;                        // bf16 [T, Hq, dv + 64]; MLA: e4m3 latent codes [T, Hq, dv]
  const float* q_scale;                 // MLA: [T, Hq, dv / 128]
  const void* q_rope;                   // MLA: bf16 [T, Hq, 64]
  const void* k_main;                   // bf16 key rows (dv + 64 channels); MLA: latent codes
  int64_t m_sp, m_sh, m_ss;             // element strides (page, head, slot) of k_main
  const void* k_rope;                   // rotary channels: k_main + dv elements, or MLA's bf16 cache
  int64_t r_sp, r_sh, r_ss;
  const void* v;                        // bf16 value rows (dv channels); MLA: unused (value = latent)
  int64_t v_sp, v_sh, v_ss;
  const float* k_scale;                 // MLA: latent scales, dv / 128 per (page, head, slot)
  int64_t s_sp, s_sh, s_ss;
  const int32_t* page_indices;
  float sm_scale;
  void* partial_o; float* partial_lse;  // partial O: float32, or bf16 when part_bf16
  void* out; float* out_lse;
  int out_bf16, part_bf16;
  int hq, group, page_shift, s_max;
  int fair;                             // every item runs at once (at most two per CU)
};

struct MergeArgs {
  const int32_t* row_nsplit;
  const void* partial_o; const float* partial_lse;   // partial O: float32, or bf16 when part_bf16
  void* out; int out_bf16; float* out_lse;
  int total_rows, hq, dh, s_max;
  int part_bf16;
};

struct GatherArgs {
  const PaItem* items; const int32_t* page_indices;
  int64_t kv_sp, kv_sh, kv_ss;          // KV element strides (page, head, slot)
  int64_t sc_sp, sc_sh, sc_ss;          // per-token-head scale strides
  int64_t* kv_off;                      // [items, max_tok, chunks per token]: byte offsets
  int64_t* sc_off;                      // [items, max_tok, 2]: k / v scale element offsets, or NULL
  int64_t max_tok;                      // longest token range of an item
  int page_shift;
};

struct GatherRopeArgs {
  const PaItem* items; const int32_t* page_indices;
  int64_t m_sp, m_sh, m_ss;             // K main rows / latent codes
  int64_t r_sp, r_sh, r_ss;             // rotary rows
  int64_t v_sp, v_sh, v_ss;             // V rows (192/128)
  int64_t s_sp, s_sh, s_ss;             // latent block scales
  int64_t* off;                         // [items, max_tok, columns]
  int64_t max_tok;
  int page_shift;
};
int launch_gather_rope(const KernelCfg& c, const GatherRopeArgs& a, int num_items, void* stream);

// Sets the message pa_last_error returns and returns st (defined in api.cpp).
int report_error(int st, const char* msg);

// Launchers (defined in the .hip files); return a hipError_t as int.
int launch_stage1(const KernelCfg& cfg, const Stage1Args& a, int num_items, void* stream);
int launch_merge(const MergeArgs& a, void* stream);
int launch_gather(const KernelCfg& cfg, const GatherArgs& a, int num_items, void* stream);
int launch_quant(const void* src, int src_bf16, int64_t n_rows, int head_dim, int per_tensor, int i8,
                 uint8_t* dst, float* scale, void* stream);
bool stage1_cfg_supported(const KernelCfg& cfg);
int launch_stage1_kr(int dv, int wq, const KrArgs& a, int num_items, void* stream);
int launch_stage1_mla(int wq, const KrArgs& a, int num_items, void* stream);

}  // namespace pa
