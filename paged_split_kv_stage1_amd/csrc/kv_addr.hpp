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

#include <type_traits>

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
  // Token whose chunk cpos this lane loads in group i (clamped like lane_offset).
  __device__ __forceinline__ int lane_token(int jb, int te) const { return jb + min(lt, te - 1 - jb); }

  // A span that lies wholly before te and starts on a multiple of 16 tokens sits in one
  // page: its first row's byte offset is one scalar (span_row), group i adds a scalar
  // step, and each lane adds its constant goff -- no clamp, no page choice.
  static __device__ __forceinline__ bool span_full(int q0, int te) { return q0 + SPAN <= te; }
  static __device__ __forceinline__ int64_t span_row(const cint32* pidx, int q0, int page_shift, int64_t kv_sp,
                                                     int64_t head_off, int64_t kv_ss) {
    return ((int64_t)pidx[q0 >> page_shift] * kv_sp + head_off +
            (int64_t)(q0 & ((1 << page_shift) - 1)) * kv_ss) * KVB;
  }
  static __device__ __forceinline__ int64_t group_step(int i, int64_t kv_ss) { return (int64_t)GT * i * kv_ss * KVB; }
};

// Float32 scales of 128-channel blocks, four per (page, KV head, slot) with element strides
// (sc_sp, sc_sh, sc_ss), for a 16-token span from u0: lane e reads the scale of block e % 4
// of token u0 + e / 4 (clamped to te - 1), an element offset.
struct BlockScaleAddr {
  static __device__ __forceinline__ int64_t lane_term(int lane, int64_t sc_ss) {
    return (int64_t)(lane >> 2) * sc_ss + (lane & 3);
  }
  // the span lies wholly before te: one page, lane_term precomputed
  static __device__ __forceinline__ int64_t full(const cint32* pidx, int u0, int page_shift, int kvh, int64_t sc_sp,
                                                 int64_t sc_sh, int64_t sc_ss, int64_t lane_term) {
    return (int64_t)pidx[u0 >> page_shift] * sc_sp + (int64_t)kvh * sc_sh +
           (int64_t)(u0 & ((1 << page_shift) - 1)) * sc_ss + lane_term;
  }
  // the last span of a split: clamped token, page A or B of the span
  template <typename Pages>
  static __device__ __forceinline__ int64_t clamped(const Pages& sp, int u0, int te, int page_shift, int lane, int kvh,
                                                    int64_t sc_sp, int64_t sc_sh, int64_t sc_ss) {
    const int j = min(u0 + (lane >> 2), te - 1);
    const int32_t pg = (j >> page_shift) == sp.first ? sp.pA : sp.pB;
    return (int64_t)pg * sc_sp + (int64_t)kvh * sc_sh + (int64_t)(j & ((1 << page_shift) - 1)) * sc_ss + (lane & 3);
  }
  static __device__ __forceinline__ int token(int u0, int te, int lane) { return min(u0 + (lane >> 2), te - 1); }
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

template <int V>
using kv_part = std::integral_constant<int, V>;

// Every load of one wave for one tile of the 192/128 kernel (stage1_kr.hip): the wave's
// 32-token quarter from q0 of K main rows (DV bf16 channels), K rotary rows (64 bf16
// channels at byte offset 2 DV of the K row) and V rows (DV bf16 channels).
// emit(kv_part<p>, i, byte offset, token, chunk) once per 16-byte load, in load order:
// part 0 K main (offset from the K base), 1 K rotary (from the K base + 2 DV bytes),
// 2 V (from the V base); i the load group, token the (clamped) token, chunk the 16-byte
// chunk of that part's row.  The gather test hook runs the same function.
template <int DV>
struct RopeQuarterLoads {
  using AM = KvSpanAddr<DV * 2 / 16, 2>;
  using AR = KvSpanAddr<8, 2>;
  using AV = KvSpanAddr<DV * 2 / 16, 2>;
  AM am; AR ar; AV av;
  int64_t m_sp, m_ss, r_sp, r_ss, v_sp, v_ss, mhead, rhead, vhead;
  __device__ __forceinline__ RopeQuarterLoads(int lane, int kvh, int64_t msp, int64_t msh, int64_t mss, int64_t rsp,
                                              int64_t rsh, int64_t rss, int64_t vsp, int64_t vsh, int64_t vss)
      : am(lane, mss), ar(lane, rss), av(lane, vss), m_sp(msp), m_ss(mss), r_sp(rsp), r_ss(rss), v_sp(vsp), v_ss(vss),
        mhead((int64_t)kvh * msh), rhead((int64_t)kvh * rsh), vhead((int64_t)kvh * vsh) {}
  template <class Emit>
  __device__ __forceinline__ void tile(const cint32* pidx, int q0, int te, int shift, Emit&& emit) const {
    const SpanPages qp(pidx, q0, 32, te, shift);
    {
      const int64_t bA = qp.base(false, m_sp, mhead, 2), bB = qp.base(true, m_sp, mhead, 2);
#pragma unroll
      for (int i = 0; i < AM::NG; ++i) {
        const int jb = AM::group_token(q0, i, te);
        emit(kv_part<0>{}, i, AM::row_offset(jb, qp.first, bA, bB, shift, m_ss) + am.lane_offset(jb, te, m_ss),
             am.lane_token(jb, te), am.cpos);
      }
    }
    {
      const int64_t bA = qp.base(false, r_sp, rhead, 2), bB = qp.base(true, r_sp, rhead, 2);
#pragma unroll
      for (int i = 0; i < AR::NG; ++i) {
        const int jb = AR::group_token(q0, i, te);
        emit(kv_part<1>{}, i, AR::row_offset(jb, qp.first, bA, bB, shift, r_ss) + ar.lane_offset(jb, te, r_ss),
             ar.lane_token(jb, te), ar.cpos);
      }
    }
    {
      const int64_t bA = qp.base(false, v_sp, vhead, 2), bB = qp.base(true, v_sp, vhead, 2);
#pragma unroll
      for (int i = 0; i < AV::NG; ++i) {
        const int jb = AV::group_token(q0, i, te);
        emit(kv_part<2>{}, i, AV::row_offset(jb, qp.first, bA, bB, shift, v_ss) + av.lane_offset(jb, te, v_ss),
             av.lane_token(jb, te), av.cpos);
      }
    }
  }
};

// Every load of one wave for one tile of the latent-cache kernel (stage1_mla.hip): the
// wave's 16-token span from u0 of latent codes (DV bytes per row), bf16 rotary rows (64
// channels) and the DV / 128 = 4 block scales per token.  emit(kv_part<p>, i, offset,
// token, chunk) per load: part 0 latent (byte offset), 1 rotary (byte offset), 2 scale
// (element offset; chunk = the 128-channel block).  Spans wholly before te take one page
// and no clamp (scalar rows, constant lane offsets); the split's last span clamps tokens
// past te - 1 to it.  The gather test hook runs the same function.
template <int DV>
struct LatentSpanLoads {
  using AL = KvSpanAddr<DV / 16, 1, 16>;
  using AR = KvSpanAddr<8, 2, 16>;
  static_assert(DV == 512, "four 128-channel scale blocks per token: one scale load per lane");
  AL al; AR ar;
  int lane, kvh;
  int64_t m_sp, m_ss, r_sp, r_ss, s_sp, s_sh, s_ss, mhead, rhead, sl_lane;
  __device__ __forceinline__ LatentSpanLoads(int ln, int kh, int64_t msp, int64_t msh, int64_t mss, int64_t rsp,
                                             int64_t rsh, int64_t rss, int64_t ssp, int64_t ssh, int64_t sss)
      : al(ln, mss), ar(ln, rss), lane(ln), kvh(kh), m_sp(msp), m_ss(mss), r_sp(rsp), r_ss(rss), s_sp(ssp),
        s_sh(ssh), s_ss(sss), mhead((int64_t)kh * msh), rhead((int64_t)kh * rsh),
        sl_lane(BlockScaleAddr::lane_term(ln, sss)) {}
  template <class Emit>
  __device__ __forceinline__ void tile(const cint32* pidx, int u0, int te, int shift, Emit&& emit) const {
    if (AL::span_full(u0, te)) {
      const int64_t lrow = AL::span_row(pidx, u0, shift, m_sp, mhead, m_ss);
      const int64_t rrow = AR::span_row(pidx, u0, shift, r_sp, rhead, r_ss);
#pragma unroll
      for (int i = 0; i < AL::NG; ++i)
        emit(kv_part<0>{}, i, lrow + AL::group_step(i, m_ss) + al.goff, u0 + AL::GT * i + al.lt, al.cpos);
#pragma unroll
      for (int i = 0; i < AR::NG; ++i)
        emit(kv_part<1>{}, i, rrow + AR::group_step(i, r_ss) + ar.goff, u0 + AR::GT * i + ar.lt, ar.cpos);
      emit(kv_part<2>{}, 0, BlockScaleAddr::full(pidx, u0, shift, kvh, s_sp, s_sh, s_ss, sl_lane),
           u0 + (lane >> 2), lane & 3);
      return;
    }
    const SpanPages sp(pidx, u0, 16, te, shift);
    {
      const int64_t bA = sp.base(false, m_sp, mhead, 1), bB = sp.base(true, m_sp, mhead, 1);
#pragma unroll
      for (int i = 0; i < AL::NG; ++i) {
        const int jb = AL::group_token(u0, i, te);
        emit(kv_part<0>{}, i, AL::row_offset(jb, sp.first, bA, bB, shift, m_ss) + al.lane_offset(jb, te, m_ss),
             al.lane_token(jb, te), al.cpos);
      }
    }
    {
      const int64_t bA = sp.base(false, r_sp, rhead, 2), bB = sp.base(true, r_sp, rhead, 2);
#pragma unroll
      for (int i = 0; i < AR::NG; ++i) {
        const int jb = AR::group_token(u0, i, te);
        emit(kv_part<1>{}, i, AR::row_offset(jb, sp.first, bA, bB, shift, r_ss) + ar.lane_offset(jb, te, r_ss),
             ar.lane_token(jb, te), ar.cpos);
      }
    }
    emit(kv_part<2>{}, 0, BlockScaleAddr::clamped(sp, u0, te, shift, lane, kvh, s_sp, s_sh, s_ss),
         BlockScaleAddr::token(u0, te, lane), lane & 3);
  }
};

}  // namespace pa
