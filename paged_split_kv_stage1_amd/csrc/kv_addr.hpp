// Address code of the paged KV loads of stage 1.
//
// Stage 1 computes the address of every 16-byte K/V chunk and every per-token-head
// scale it loads through these functions, and the gather test hook (gather.hip) calls
// the same functions over the same tiles and records what they return, so the bit-exact
// page-gather check covers the code stage 1 loads with.
//
// Page gather (the paged KV layout the pages describe, e.g. the block-size-64 FP8 cache of
// hpc-ops issue #4): logical token j of a request lives in page
// page_indices[page_base + j / P] at slot j % P (P = 1 << page_shift); element c of KV head
// g of that token sits at page * kv_sp + g * kv_sh + slot * kv_ss + c (element strides).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// The page table is read-only while a kernel runs: reading it through the constant
// address space lets the compiler use scalar loads for wave-uniform indices.
typedef const int32_t __attribute__((address_space(4))) cint32;

// Tiles of BN tokens whose rows are CPR 16-byte chunks in HBM.  One wave's 64 lanes cover
// 64 / CPR consecutive tokens per load group (lane = token lt, chunk cpos), and a tile
// takes CPT load groups per thread.  Groups start on multiples of 64 / CPR tokens and
// pages hold >= 16 tokens, so a group never straddles a page: its page and slot are
// wave-uniform, and a lane's address is a uniform row offset plus a per-lane offset that
// does not change between tiles.  Tokens past the split's last one (te - 1) are clamped
// to it (finite data, masked later).
template <int CPR, int BN, int KVB>
struct KvTileAddr {
  static constexpr int CPT = BN * CPR / 256;
  int lt;          // token of this lane within its wave's load group
  int cpos;        // 16-byte chunk of the token row this lane loads
  uint32_t goff;   // byte offset of (lt, cpos) from the group's first row (no clamp)

  __device__ __forceinline__ KvTileAddr(int lane, int64_t kv_ss)
      : lt(lane / CPR), cpos(lane % CPR), goff((uint32_t)(lane / CPR * kv_ss * KVB) + ((lane % CPR) << 4)) {}

  // First token of load group i of wave w in the tile starting at tile0 (wave-uniform).
  static __device__ __forceinline__ int group_token(int tile0, int wave, int i, int te) {
    return min(tile0 + (wave * 64 + 256 * i) / CPR, te - 1);
  }
  // Physical page of the group whose first token is jb (a scalar load).
  static __device__ __forceinline__ int32_t group_page(const cint32* pidx, int jb, int page_shift) {
    return pidx[jb >> page_shift];
  }
  // Byte offset of the group's first token row of KV head head_off / kv_sh (wave-uniform).
  static __device__ __forceinline__ int64_t row_offset(int32_t page, int jb, int64_t kv_sp, int64_t head_off,
                                                       int64_t kv_ss, int pmask) {
    return ((int64_t)page * kv_sp + head_off + (int64_t)(jb & pmask) * kv_ss) * KVB;
  }
  // Per-lane byte offset from the group's row; lanes past te - 1 read the last token.
  __device__ __forceinline__ uint32_t lane_offset(int jb, int te, int64_t kv_ss) const {
    const int ltc = min(lt, te - 1 - jb);
    return goff - (uint32_t)((lt - ltc) * kv_ss * KVB);
  }
  // Token whose chunk cpos this lane loads.
  __device__ __forceinline__ int lane_token(int jb, int te) const { return jb + min(lt, te - 1 - jb); }
};

// Per-(token, KV head) scales of a tile: thread tid < 2 * BN loads the k_scale (tid < BN) or
// the v_scale (tid >= BN) of token min(tile0 + tid % BN, te - 1).  The NP pages a tile can
// touch are looked up first (all scalar loads), then each thread picks its token's page.
template <int BN, int NP>
struct ScaleTileAddr {
  int64_t off;     // element offset of the scale
  int token;       // token it belongs to
  bool is_v;       // v_scale (else k_scale)
  __device__ __forceinline__ ScaleTileAddr(const cint32* pidx, int tile0, int te, int page_shift, int tid, int kvh,
                                           int64_t sc_sp, int64_t sc_sh, int64_t sc_ss) {
    int pages[NP];
    const int pg0 = tile0 >> page_shift;
    const int pgl = (te - 1) >> page_shift;
#pragma unroll
    for (int k = 0; k < NP; ++k) pages[k] = pidx[min(pg0 + k, pgl)];
    is_v = tid >= BN;
    token = min(tile0 + (is_v ? tid - BN : tid), te - 1);
    const int sel = (token >> page_shift) - pg0;
    int page = pages[0];
#pragma unroll
    for (int k = 1; k < NP; ++k) page = sel == k ? pages[k] : page;
    off = (int64_t)page * sc_sp + (int64_t)kvh * sc_sh + (int64_t)(token & ((1 << page_shift) - 1)) * sc_ss;
  }
};

// Spans of SPAN consecutive tokens of a tile, one per wave, for rows of CPR 16-byte chunks:
// load group i (i < SPAN * CPR / 64) covers the 64 / CPR tokens from q0 + i * 64 / CPR of the
// span starting at q0 (lane = token lt, chunk cpos).  Spans start on multiples of SPAN
// tokens (SPAN = 16 or 32) and pages hold >= 16 tokens, so a span touches at most two
// pages: their two page-table entries are the only scalar loads, and each group picks its
// row base from them.  Tokens past the split's last one (te - 1) are clamped to it, as in
// KvTileAddr.
template <int CPR, int KVB, int SPAN = 32>
struct KvSpanAddr {
  static constexpr int NG = SPAN * CPR / 64;  // load groups per span
  static constexpr int GT = 64 / CPR;         // tokens per group
  int lt, cpos;
  uint32_t goff;
  __device__ __forceinline__ KvSpanAddr(int lane, int64_t kv_ss)
      : lt(lane / CPR), cpos(lane % CPR), goff((uint32_t)(lane / CPR * kv_ss * KVB) + ((lane % CPR) << 4)) {}
  // First token of group i (wave-uniform).
  static __device__ __forceinline__ int group_token(int q0, int i, int te) { return min(q0 + GT * i, te - 1); }
  // Byte offset of group i's first row: page base A (the page of the span's first
  // clamped token) or B (that of its last), plus the slot.
  static __device__ __forceinline__ int64_t row_offset(int jb, int pgA_first, int64_t baseA, int64_t baseB,
                                                       int page_shift, int64_t kv_ss) {
    const int64_t base = (jb >> page_shift) == pgA_first ? baseA : baseB;
    return base + (int64_t)(jb & ((1 << page_shift) - 1)) * kv_ss * KVB;
  }
  __device__ __forceinline__ uint32_t lane_offset(int jb, int te, int64_t kv_ss) const {
    const int ltc = min(lt, te - 1 - jb);
    return goff - (uint32_t)((lt - ltc) * kv_ss * KVB);
  }
};

// The two page-table entries a span of `span` tokens from q0 can touch (see KvSpanAddr).
struct SpanPages {
  int first;       // logical page of the span's first clamped token
  int32_t pA, pB;  // physical pages of its first and last clamped tokens
  __device__ __forceinline__ SpanPages(const cint32* pidx, int q0, int span, int te, int page_shift) {
    first = min(q0, te - 1) >> page_shift;
    pA = pidx[first];
    pB = pidx[min(q0 + span - 1, te - 1) >> page_shift];
  }
  // Byte offset of the page's row block of one head, for pages A and B.
  __device__ __forceinline__ int64_t base(bool b, int64_t kv_sp, int64_t head_off, int kvb) const {
    return ((int64_t)(b ? pB : pA) * kv_sp + head_off) * kvb;
  }
};

}  // namespace pa
