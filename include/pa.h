/*
 * pa.h -- C ABI of a gfx950 (MI355X) library for paged split-KV decode attention.
 *
 * The operation (FreeToken PR #900 "perf(attention): run up to 8 query rows per
 * request in the triton decode kernel", section "Changes"): decode attention over a
 * paged KV cache where each request carries up to 8 causal query rows described by
 * qo_indptr / max_q_len; stage 1 keeps the KV split and packs query rows x GQA
 * heads of one KV head into one matrix tile, limiting each row to its own position
 * and window; stage 2 merges the splits of each row.  KV may be bf16 or FP8
 * (OCP E4M3FN) with a per-tensor scale (FlashMLA PR #54 "Functionality") or one
 * scale per (token, KV head) (FreeToken PR #900, "fp8_per_token_head").
 * Dequantisation is folded into the score scale and the final normaliser
 * (FlashInfer PR #869, item 3).  Requests with more rows than supported are
 * rejected with an error rather than silently mishandled (hpc-ops issue #4: its
 * FP8 decode entry point raises a runtime error for any q_len other than 1).
 *
 * Conventions for every entry point
 *  - Every pointer is caller-owned.  Pointers documented as "device" must be
 *    device memory of the current HIP device; "host" pointers are plain host
 *    memory.  The library never allocates or frees memory, never synchronises,
 *    and launches work only on the stream passed in (a hipStream_t; NULL = the
 *    default stream).  stage1/merge launches are hipGraph-capturable.
 *  - Every call returns a pa_status.  On failure nothing has been launched and
 *    pa_last_error() returns a message (thread-local, valid until the next call
 *    on the same thread).  Errors of kernels that already ran asynchronously
 *    surface through the HIP runtime (hipStreamSynchronize), not here.
 *  - FP8 means OCP E4M3FN: bias 7, max finite 448, S.1111.111 = NaN, no Inf.
 *  - Q is [T, Hq, d] contiguous (T = total query rows = qo_indptr[B]); the output
 *    is [T, Hq, d] contiguous.  Query head h reads KV head h / (Hq / Hkv).
 *  - Row r (0-based) of request b sits at position p = kv_len[b] - n_b + r, with
 *    n_b = qo_indptr[b+1] - qo_indptr[b]; kv_len counts the new rows' own keys.
 *    It attends to keys j with lo <= j <= p, lo = max(0, p - W + 1) when the
 *    request's window W > 0 (W keys including itself), lo = 0 otherwise.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARGUMENT = 1,     /* malformed input: the call can never succeed as given */
  PA_ERR_UNSUPPORTED = 2,          /* well-formed but outside what the kernels implement   */
  PA_ERR_INSUFFICIENT_WORKSPACE = 3,/* a caller buffer is smaller than required             */
  PA_ERR_HIP = 4                   /* a HIP runtime call failed (message has the HIP error) */
} pa_status;

/* INT8 (KV caches only): symmetric codes in [-127, 127], value = code * scale, scale =
 * amax / 127 over the scaled group (FreeToken PR #900, "Tested on", names int8 KV
 * kernels; the format is this library's reading). */
typedef enum { PA_DTYPE_BF16 = 0, PA_DTYPE_FP32 = 1, PA_DTYPE_FP8_E4M3 = 2, PA_DTYPE_INT8 = 3 } pa_dtype;

typedef enum {
  PA_SCALE_NONE = 0,           /* bf16 KV                                               */
  PA_SCALE_PER_TENSOR = 1,     /* one float32 scale for the whole K (and one for V)     */
  PA_SCALE_PER_TOKEN_HEAD = 2, /* one float32 scale per (token slot, KV head)           */
  PA_SCALE_PER_HEAD = 3,       /* one float32 scale per KV head for K and for V, and per */
                               /* query head for FP8 Q (FlashInfer PR #869, title:       */
                               /* per-head quantization)                                 */
  PA_SCALE_PER_TOKEN_BLOCK128 = 4 /* MLA-style latent cache: one float32 scale per        */
                               /* (token, KV head, 128 latent channels) (FlashMLA PR #54, */
                               /* review thread); see pa_decode_stage1_rope              */
} pa_scale_mode;

/* Element strides of a paged cache: element (page, kv_head, slot, c) lives at
 * base[page*page + kv_head*head + slot*slot + c] (the head_dim axis is contiguous).
 * [pages, Hkv, P, d] has {Hkv*P*d, P*d, d}; [pages, P, Hkv, d] has {P*Hkv*d, d, Hkv*d}.
 * Every stride times the element size must be a multiple of 16 bytes. */
typedef struct { int64_t page, head, slot; } pa_kv_layout;

/* Element strides of per-(token, KV head) float32 scales: scale(page, kv_head, slot)
 * = base[page*page + kv_head*head + slot*slot]. */
typedef struct { int64_t page, head, slot; } pa_scale_layout;

/* Planner input.  All array pointers are HOST memory. */
typedef struct {
  int32_t batch;               /* B >= 1 requests                                          */
  const int32_t* qo_indptr;    /* [B+1] query-row CSR; 1 <= n_b <= max_q_len                */
  const int32_t* kv_indptr;    /* [B+1] CSR into page_indices; must equal ceil(kv_len/P)    */
  const int32_t* kv_len;       /* [B] tokens in the cache, including the new rows; >= n_b   */
  const int32_t* window;       /* [B] sliding window in keys (0 = none), or NULL (none)      */
  int32_t max_q_len;           /* upper bound of n_b; must be <= 8                          */
  int32_t page_size;           /* tokens per page: a power of two in [16, 1024]             */
  int32_t num_q_heads;         /* Hq                                                        */
  int32_t num_kv_heads;        /* Hkv; Hq % Hkv == 0                                        */
  int32_t head_dim;            /* 128 or 256; 512 with bf16 queries and bf16 or            */
                               /*   PER_TOKEN_HEAD FP8 KV (a request's rows x heads per KV  */
                               /*   head run in work items of at most 64)                   */
  pa_dtype q_dtype;            /* BF16, or FP8_E4M3 (then kv must be FP8 as well)           */
  pa_dtype kv_dtype;           /* BF16, FP8_E4M3 or INT8 (INT8: PER_TENSOR or PER_TOKEN_HEAD */
                               /*   scales, bf16 queries)                                   */
  pa_scale_mode kv_scale_mode; /* NONE for bf16 KV; PER_TENSOR, PER_HEAD or PER_TOKEN_HEAD   */
                               /*   for FP8 KV                                              */
  int32_t num_cus;             /* compute units to plan for; 0 = query the current device   */
  int32_t max_splits;          /* cap on splits per request (fixes scratch size for graph   */
                               /*   capture); 0 = no cap beyond the library's limit (1024)  */
  int32_t force_splits;        /* > 0: every request gets exactly this many splits           */
  int32_t head_dim_v;          /* value width when it differs from head_dim (0 = head_dim):   */
                               /*   192/128 (bf16) or 576/512 (latent cache, PER_TOKEN_BLOCK128 */
                               /*   scales, FP8 queries); such plans run pa_decode_stage1_rope */
  int32_t orientation;         /* pa_orientation of stage 1's matrix products (0 = default)  */
} pa_plan_args;

/* Which axis of stage 1's 16x16 MFMA tiles the key tokens take.  KV_ON_M (the default)
 * computes S^T = K Q^T and O^T = V^T P^T: the score accumulator already has the layout
 * of P^T as an operand, so P stays in registers.  Q_ON_M computes S = Q K^T and O = P V
 * with the packed query rows on M (FreeToken PR #900, "Changes"), transposing P through
 * LDS every tile; it is kept as the measured alternative (the swapped form is what
 * hpc-ops issue #4 asks about) for bf16 KV and for PER_TOKEN_HEAD FP8 KV with bf16
 * queries at head_dim 128 and 256, except bf16 KV at head_dim 256 with 9-16 query rows
 * per KV head and bf16 KV at head_dim 128 with more than 128 (UNSUPPORTED there). */
typedef enum { PA_ORIENT_KV_ON_M = 0, PA_ORIENT_Q_ON_M = 1 } pa_orientation;

/* Planner output, consumed by stage1/merge.  Sizes are in bytes. */
typedef struct {
  int32_t batch, total_rows, num_q_heads, num_kv_heads, head_dim, page_size, max_q_len;
  int32_t q_dtype, kv_dtype, kv_scale_mode;
  int32_t num_items;           /* stage-1 work items (one workgroup each)                   */
  int32_t max_splits;          /* S_max: the split axis of the scratch buffers               */
  int32_t needs_merge;         /* 0 when every request has a single split                   */
  int32_t num_cus;
  int32_t variant;             /* kernel tile configuration (library internal)              */
  int32_t head_dim_v;          /* value width (output and partial-O rows)                    */
  int64_t plan_bytes;          /* bytes of the plan buffer (host copy and device copy)       */
  int64_t partial_o_bytes;     /* [T, Hq, S_max, dv]: float32 (bf16 KV) or bf16 (FP8/INT8 KV) */
  int64_t partial_lse_bytes;   /* float32 [T, Hq, S_max]                                    */
  int64_t max_item_tokens;     /* longest KV token range of one work item                   */
  int64_t reserved[3];
} pa_plan_info;

/* Split planner (host only; no device work, no allocation).
 * Defined by: FreeToken PR #900, "Changes" (the kernel takes qo_indptr and max_q_len,
 * keeps the split-KV grid for multi-row requests, and sizes per-row scratch so that a
 * captured graph keeps working) and its motivation section (one program per whole
 * context is many times slower than splitting the KV sequence); hpc-ops issue #4, request
 * section (unsupported query lengths are refused with an error).
 * Reads the host index arrays, validates them, chooses the number of KV splits of
 * every request for the device's compute units, and writes the work list into
 * plan_host (plan_capacity bytes).  With plan_host == NULL only *info is filled,
 * which tells the caller how large the plan and scratch buffers must be.  The caller
 * copies plan_host to a device buffer of info->plan_bytes bytes before stage 1.
 * Split boundaries are 64-token aligned but not necessarily equal: when every item gets
 * its own workgroup slot, the splits of a memory-bound range are sized for the XCD their
 * position in the work list runs on (workgroup p on XCD p mod 8; the odd XCDs were
 * measured ~10% slower at streaming); info->max_item_tokens is the longest item.
 * Errors: INVALID_ARGUMENT (non-monotone CSR, n_b > kv_len, kv_indptr inconsistent
 * with kv_len, Hq % Hkv != 0, bad enum), UNSUPPORTED (max_q_len > 8, head_dim not
 * 128/256/512, page size not a power of two in [16, 1024], rows x group too large for one
 * tile, dtype combination), INSUFFICIENT_WORKSPACE (plan_capacity < info->plan_bytes). */
pa_status pa_plan_splits(const pa_plan_args* args, void* plan_host, size_t plan_capacity,
                         pa_plan_info* info);

/* Stage 1 (device).  Defined by: FreeToken PR #900, "Changes" (rows x GQA heads of one KV
 * head share one tile, each row limited to its own position, partial output and LSE per
 * split); FlashInfer PR #869, summary items 1-3 (V transposed for FP8 operands, P
 * requantised for the FP8 P.V product, dequantisation folded into sm_scale and the
 * final normaliser); hpc-ops issue #4, "why K x Q^T" question (the swapped product).
 * For every work item (request, KV head, split) stream the split's
 * pages and write, for each of its query rows x heads, the split's normalised
 * partial output and natural-log LSE; requests planned with a single split write
 * the final output directly.
 *   plan_dev     device copy of the plan (info->plan_bytes)
 *   q            device [T, Hq, d]: bf16, or e4m3 codes with *q_scale (device float)
 *   q_scale      device float32 when q is FP8 (a scalar, or [Hq] per query head with
 *                PER_HEAD), else NULL
 *   k_cache, v_cache  device paged caches (bf16 or e4m3 codes) with strides kv
 *   k_scale, v_scale  device float32: a scalar (PER_TENSOR), [Hkv] (PER_HEAD), or a
 *                per-token-head array with strides sc (PER_TOKEN_HEAD); NULL for bf16 KV
 *   page_indices device int32, indexed through kv_indptr
 *   sm_scale     softmax scale applied to q.k (typically 1/sqrt(d) in float32)
 *   partial_o    device [T, Hq, S_max, d], info->partial_o_bytes: float32 for bf16 KV,
 *                bf16 for FP8 / INT8 KV (unused if !info->needs_merge)
 *   partial_lse  device float32 [T, Hq, S_max]
 *   out          device [T, Hq, d] in out_dtype (BF16 or FP32)
 *   out_lse      device float32 [T, Hq] or NULL: rows of requests planned with a single
 *                split receive their natural-log LSE here (pa_decode_merge writes the
 *                rows of split requests, so the two together fill every row)
 * Tokens past kv_len (the tail of the last page) are never read.
 * Accuracy (softmax(s q.k) v over the same quantised K/V): bf16 KV keeps P in two bf16
 * terms (~2^-16 relative); per-tensor FP8 V carries P as two e4m3 terms; per-token-head
 * FP8 and INT8 V carry P as one bf16 term with v_scale folded in.  With FP8 or INT8 K
 * and four one-block waves per work item, bf16 queries are carried as two 8-bit terms
 * under a per-row scale (~2^-8 relative for e4m3, ~2^-16 of the row's largest element
 * for int8).  Measured against an fp64 evaluation: <= 2e-3 (bf16 KV) and <= 2e-2
 * (FP8 / INT8 KV) max relative error per (row, head). */
pa_status pa_decode_stage1(const pa_plan_info* info, const void* plan_dev,
                           const void* q, const float* q_scale,
                           const void* k_cache, const void* v_cache, const pa_kv_layout* kv,
                           const float* k_scale, const float* v_scale, const pa_scale_layout* sc,
                           const int32_t* page_indices, float sm_scale,
                           void* partial_o, float* partial_lse,
                           void* out, pa_dtype out_dtype, float* out_lse, void* stream);

/* Stage 1 for keys wider than values (device; a plan with head_dim != head_dim_v).
 * Defined by: FlashInfer PR #869, "Remaining Work" (separate head_dim_qk and head_dim_v);
 * the latent form by FlashMLA PR #54, review thread (keys' and queries' no-position part in
 * 8 bits with one scale per token and 128 channels, their 64 rotary channels in 16 bits).
 * Keys have head_dim = head_dim_v + 64 channels, the last 64 of which are rotary; the
 * output and the partials have head_dim_v channels.  Otherwise as pa_decode_stage1 (same
 * plan items, partial layout, LSE, out_lse and merge).
 *   192/128, bf16 (kv_scale_mode NONE):
 *     q        device bf16 [T, Hq, 192];  q_scale, q_rope, k_rope, k_scale: NULL
 *     k_cache  bf16 key rows of 192 channels, element strides k_layout
 *     v_cache  bf16 value rows of 128 channels, element strides v_layout
 *   576/512 latent cache (kv_scale_mode PER_TOKEN_BLOCK128, q_dtype and kv_dtype FP8):
 *     q        device e4m3 codes [T, Hq, 512] of the queries' latent part
 *     q_scale  device float32 [T, Hq, 4]: the scale of each 128-channel block
 *     q_rope   device bf16 [T, Hq, 64]: the queries' rotary part
 *     k_cache  e4m3 latent codes, 512 per (page, KV head, slot), element strides k_layout
 *     k_scale  float32 latent scales, 4 consecutive per (page, KV head, slot) (one per 128
 *              channels; k_scale_layout gives the strides of the first)
 *     k_rope   bf16 rotary rows of 64 channels, element strides k_rope_layout
 *     v_cache, v_layout: NULL (the value is the latent: code times its block's scale)
 * Accuracy: 192/128 runs bf16 MFMA and keeps P in two bf16 terms.  The latent form computes
 * the latent q.k on the FP8 MFMA over the raw e4m3 codes of keys and queries (exact
 * products, fp32 sums, then the two block scales), the rotary part on bf16 MFMA, and P.V as
 * one bf16 term of P times the token's block scale against exactly upconverted codes.  Pointers
 * 16-byte aligned, cache strides multiples of 16 bytes.  Errors: INVALID_ARGUMENT (a plan
 * of equal widths, missing or misaligned arguments). */
pa_status pa_decode_stage1_rope(const pa_plan_info* info, const void* plan_dev,
                                const void* q, const float* q_scale, const void* q_rope,
                                const void* k_cache, const pa_kv_layout* k_layout,
                                const void* k_rope, const pa_kv_layout* k_rope_layout,
                                const float* k_scale, const pa_kv_layout* k_scale_layout,
                                const void* v_cache, const pa_kv_layout* v_layout,
                                const int32_t* page_indices, float sm_scale,
                                void* partial_o, float* partial_lse,
                                void* out, pa_dtype out_dtype, float* out_lse, void* stream);

/* Stage 2 (device).  Defined by: FreeToken PR #900, "Changes" (stage 2 merges the splits
 * of each row).  Per (row, query head) with more than one split,
 * out = sum_s e^{lse_s - M} o_s / sum_s e^{lse_s - M}, M = max_s lse_s, written
 * in out_dtype; out_lse (device float32 [T, Hq], nullable) receives the merged
 * natural-log LSE of those rows (stage 1 writes the LSE of single-split rows).  A no-op launch-free success when
 * info->needs_merge == 0.  out and partial_o must be 16-byte aligned (as for stage 1). */
pa_status pa_decode_merge(const pa_plan_info* info, const void* plan_dev,
                          const void* partial_o, const float* partial_lse,
                          void* out, pa_dtype out_dtype, float* out_lse, void* stream);

/* FP8 quantiser (device).  Defined by: FlashMLA PR #54, "Functionality" (symmetric
 * per-tensor FP8 scales for the KV cache); FreeToken PR #900, end-to-end A/B section (the
 * fp8_per_token_head KV cache: one scale per token and KV head); the scale amax / 448 is
 * the FP8 maximum FlashInfer PR #869 (summary item 2) scales by.
 * src holds n_rows rows of head_dim contiguous values
 * (bf16 or float32; e.g. a [pages, Hkv, P, d] cache is pages*Hkv*P rows).
 *   PER_TOKEN_HEAD: scale[i] = amax_i / 448 (1 if amax_i == 0) per row i;
 *   PER_TENSOR:     one scale = amax / 448 over all rows, written to scale[0].
 * dst[i, c] = RNE_e4m3(clamp(src[i, c] / scale, -448, 448)) with an IEEE float32
 * divide.  dst: device uint8 [n_rows, head_dim]; scale: device float32 (n_rows, or 1).
 * head_dim must be a multiple of 64 and <= 1024.  (PER_HEAD scales need the head
 * count: pa_kv_quantize_fp8_per_head.) */
pa_status pa_kv_quantize_fp8(const void* src, pa_dtype src_dtype, int64_t n_rows, int32_t head_dim,
                             pa_scale_mode mode, uint8_t* dst, float* scale, void* stream);

/* Per-head FP8 quantiser (device; FlashInfer PR #869, per-head quantization): src is
 * [n_tokens, num_heads, head_dim] (bf16 or float32, contiguous); head h's scale is
 * amax over all of its n_tokens * head_dim values / 448 (1 if that amax is 0), written
 * to scale[h] (device float32 [num_heads]); dst[t, h, c] = RNE_e4m3(clamp(src[t, h, c] /
 * scale[h], -448, 448)) with an IEEE float32 divide (device uint8, src's shape).  A
 * paged cache [pages, P, Hkv, d] is n_tokens = pages * P tokens of Hkv heads; use it for
 * FP8 queries [T, Hq, d] too.  The caller owns every buffer.  Errors: INVALID_ARGUMENT
 * (NULL pointer, src not 16-byte or dst not 8-byte aligned, src dtype, n_tokens < 0),
 * UNSUPPORTED (num_heads outside [1, 1024], head_dim not 64 times a power of two up to
 * 1024). */
pa_status pa_kv_quantize_fp8_per_head(const void* src, pa_dtype src_dtype, int64_t n_tokens, int32_t num_heads,
                                      int32_t head_dim, uint8_t* dst, float* scale, void* stream);

/* INT8 quantiser (device): as pa_kv_quantize_fp8 with int8 codes: scale = amax / 127
 * (1 if amax == 0) per row (PER_TOKEN_HEAD) or over all rows (PER_TENSOR, scale[0]);
 * dst[i, c] = round-half-even(clamp(src[i, c] / scale, -127, 127)) with an IEEE float32
 * divide (-128 is never written).  dst: device int8 [n_rows, head_dim], 8-byte
 * aligned; src 16-byte aligned.  Errors as pa_kv_quantize_fp8. */
pa_status pa_kv_quantize_int8(const void* src, pa_dtype src_dtype, int64_t n_rows, int32_t head_dim,
                              pa_scale_mode mode, int8_t* dst, float* scale, void* stream);

/* KV append (device): writes the keys and values of n_tokens new tokens into the paged
 * caches, as a serving step does before decode attention reads them (the per-token-head
 * FP8 KV cache of FreeToken PR #900, end-to-end table; per-tensor scales as in FlashMLA
 * PR #54, "Functionality").  The row of token t for KV head h goes to cache element
 * (page, h, slot, :) with page = slot_mapping[t] / page_size, slot = slot_mapping[t] %
 * page_size, addressed through kv.
 *   k_new, v_new   device [n_tokens, num_kv_heads, head_dim], src_dtype BF16 or FP32,
 *                  contiguous, 16-byte aligned
 *   slot_mapping   device int64 [n_tokens]; a negative entry skips the token (padding)
 *   kv_dtype BF16, mode NONE: rows stored as bf16 (FP32 sources rounded to nearest even);
 *   kv_dtype FP8_E4M3, mode PER_TENSOR: codes RNE_e4m3(clamp(x / s, -448, 448)) with the
 *                  caches' scales s = *k_scale, *v_scale (device scalars, only read);
 *   kv_dtype FP8_E4M3, mode PER_HEAD: the same with s = k_scale[h], v_scale[h] for KV
 *                  head h (device float32 [num_kv_heads], only read);
 *   kv_dtype INT8, mode PER_TENSOR or PER_TOKEN_HEAD: as FP8 with the codes and scales
 *                  of pa_kv_quantize_int8;
 *   kv_dtype FP8_E4M3, mode PER_TOKEN_HEAD: each row's scale amax/448 (1 if amax == 0)
 *                  is written to k_scale / v_scale at (page, h, slot) through sc and the
 *                  codes are those of pa_kv_quantize_fp8.
 * The caller owns every buffer; slots must be distinct and inside the caches.  Cache
 * pointers and strides must be 16-byte aligned (as for stage 1).  Errors:
 * INVALID_ARGUMENT (NULL pointer, misalignment, dtype/mode combination), UNSUPPORTED
 * (head_dim not 64 times a power of two up to 1024, page_size not a power of two,
 * 2 * n_tokens * num_kv_heads >= 2^31). */
pa_status pa_kv_append(const void* k_new, const void* v_new, pa_dtype src_dtype, int64_t n_tokens,
                       int32_t num_kv_heads, int32_t head_dim, int32_t page_size, const int64_t* slot_mapping,
                       void* k_cache, void* v_cache, pa_dtype kv_dtype, pa_scale_mode mode,
                       const pa_kv_layout* kv, float* k_scale, float* v_scale, const pa_scale_layout* sc,
                       void* stream);

/* Test hook (device), for the bit-exact page-gather check: runs stage 1's KV address code
 * (the same device functions stage 1 loads through, with the tile geometry of the plan's
 * kernel configuration) over every tile of every work item and records what it returns:
 *   kv_off_out[(i * M + (t - b_i)) * C + c] = byte offset from the K (and V) cache base of
 *     16-byte chunk c of token t of item i's KV head, for every token t of the item's range
 *     [b_i, e_i), with M = info->max_item_tokens and C = head_dim * element size / 16
 *     (device int64, caller-filled beforehand; entries past e_i - b_i stay untouched);
 *   scale_off_out[(i * M + (t - b_i)) * 2 + {0: k, 1: v}] = element offset of that token's
 *     per-token-head scale (device int64; required for PER_TOKEN_HEAD and INT8 KV, else
 *     ignored and may be NULL; INT8 with a PER_TENSOR scale reads it through zero strides,
 *     so its offsets are 0 and sc may be NULL).
 * Item i is the i-th 64-byte record of the plan (fields in the library's plan layout).
 * Errors: INVALID_ARGUMENT (NULL pointer, plan info not from pa_plan_splits, missing
 * scale arguments). */
pa_status pa_debug_gather(const pa_plan_info* info, const void* plan_dev, const int32_t* page_indices,
                          const pa_kv_layout* kv, const pa_scale_layout* sc, int64_t* kv_off_out,
                          int64_t* scale_off_out, void* stream);

/* Test hook (device), the same for plans whose keys are wider than their values: runs the
 * load enumerators of the two wider-key stage-1 kernels (the 192/128 kernel's 32-token
 * quarters, the latent kernel's 16-token spans, each with its own page lookup and clamp)
 * over every tile of every work item and records
 *   off_out[(i * M + (t - b_i)) * N + col] (device int64, caller-filled beforehand; entries
 *   past e_i - b_i stay untouched), M = info->max_item_tokens, with columns
 *   192/128 (N = 40): 0..15 byte offsets of the 16-byte chunks of token t's 128 main K
 *     channels from the K cache base, 16..23 of its 64 rotary channels from the rotary
 *     base (K base + 256 bytes, K strides), 24..39 of its V row from the V cache base;
 *   latent (N = 44): 0..31 latent chunks from the latent base, 32..39 rotary chunks from the
 *     rotary base, 40..43 element offsets of its four block scales from the scale base.
 * Layouts: k_layout always; v_layout for 192/128; k_rope_layout and k_scale_layout for the
 * latent cache (others may be NULL).  Errors: INVALID_ARGUMENT (NULL pointer, plan info not
 * from pa_plan_splits, a layout the plan's form needs is missing), UNSUPPORTED (a plan of
 * equal widths: pa_debug_gather covers it). */
pa_status pa_debug_gather_rope(const pa_plan_info* info, const void* plan_dev, const int32_t* page_indices,
                               const pa_kv_layout* k_layout, const pa_kv_layout* k_rope_layout,
                               const pa_kv_layout* v_layout, const pa_scale_layout* k_scale_layout, int64_t* off_out,
                               void* stream);

/* Debug check (device; synchronises the stream): every page-table entry that the plan's
 * work items read (page_indices[kv_indptr[b] + t / P] for the tokens t of each item) must
 * lie in [0, num_pages), num_pages being the number of pages the K and V caches hold.
 * Stage 1 never checks page numbers, so an entry outside the caches would make it read
 * outside them; run this check first where the page table is not trusted (the Python
 * binding runs it before every stage 1 when the environment sets PA_VALIDATE=1).
 * Returns INVALID_ARGUMENT naming the count of offending reads (an entry read by the items
 * of several KV heads or splits counts once per item) and the first offending position, PA_OK
 * otherwise, or PA_ERR_HIP.  Not graph-capturable (it waits for its result). */
pa_status pa_validate_page_indices(const pa_plan_info* info, const void* plan_dev, const int32_t* page_indices,
                                   int64_t num_pages, void* stream);

/* Allocation-free decode step (device), for callers that cannot allocate device memory:
 * code under graph capture, tight serving loops, harnesses that forbid hipMalloc.  Runs
 * pa_decode_stage1 followed by pa_decode_merge with the same arguments, except that the
 * split partials live in a scratch array inside the library (128 MiB per GPU, held
 * from the library's first use on that GPU until the process ends) instead of caller
 * workspace.  The caller still passes every input and output.  Calls no allocating
 * routine.  Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (two streams, or two threads) race and give wrong results; calls on one stream are
 * ordered and safe.  Errors: those of stage 1 and the merge, and
 * INSUFFICIENT_WORKSPACE when info->partial_o_bytes (rounded up to 256) plus
 * info->partial_lse_bytes exceed the array (plan with a lower max_splits). */
pa_status pa_decode_noalloc(const pa_plan_info* info, const void* plan_dev,
                            const void* q, const float* q_scale,
                            const void* k_cache, const void* v_cache, const pa_kv_layout* kv,
                            const float* k_scale, const float* v_scale, const pa_scale_layout* sc,
                            const int32_t* page_indices, float sm_scale,
                            void* out, pa_dtype out_dtype, float* out_lse, void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* pa_last_error(void);

/* Library version string. */
const char* pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
