// Stage 1 of paged split-KV decode attention for gfx950.
//
// One workgroup (4 waves) per work item (request, KV head, KV split).  The query
// rows x GQA heads of the item's KV head form the "query-row" axis m = r*G + h
// (FreeToken PR #900, "Changes": rows x heads share one tile and keep the KV split),
// padded to 16-row blocks that never mix KV heads (the same PR's group-divisibility
// fix).  Scores are computed transposed, S^T = K Q^T (tokens on the MFMA M axis, as
// in the hpc-ops issue #4 discussion of its split-K FP8 kernel): on MFMA the
// accumulator layout of S^T (lane <-> query row, 4 consecutive tokens per lane) is
// exactly the B-operand layout P^T needs for O^T = V^T P^T, so the probabilities
// never leave registers.  V^T is read from LDS with the gfx950 transpose loads
// (ds_read_b64_tr_b16 / _tr_b8), the LDS-side counterpart of the in-kernel V
// transpose FP8 tensor cores need (FlashInfer PR #869, item 1).
//
// KV tiles stream HBM -> VGPRs (16-byte non-temporal loads, PD tiles ahead) -> LDS
// (NS stages); the LDS footprint is kept small enough for two workgroups per CU, so
// that one workgroup's prologue and tail overlap the other's streaming.
//
// Per tile, each wave owns 32 tokens x (its query blocks):
//   QK:  bf16 MFMA 16x16x32 (bf16 Q; FP8 K upconverted exactly, once when the tile is
//        stored if several query blocks per wave read it, else as it is read), or fp8
//        MFMA 16x16x32 when Q is FP8 (exact products), or -- per-token-head FP8 K read
//        by four one-block waves -- the 16x16x128 FP8 MFMA on the raw K codes with the
//        bf16 query split into two e4m3 terms under a per-row scale;
//   softmax: scores scaled into the log2 domain with the dequant scales folded in
//        (FlashInfer PR #869 item 3), per-row causal/window masks, online max/sum,
//        the O rescale skipped while no row maximum moves;
//   PV:  bf16 KV -> P split in two bf16 terms (hi + lo), so that P carries ~16
//        significant bits; per-token-head FP8 V -> v_scale folded into P, V
//        upconverted, one bf16 term (its 2^-9 rounding is far below the e4m3
//        resolution of V itself); per-tensor FP8 V ->
//        P requantised to e4m3 after scaling by the format maximum 448 (FlashInfer
//        PR #869 item 2), as a hi term plus a lo term of the residual x16, with the
//        per-tensor v_scale applied in the final normaliser.
// Waves that split the tokens of a tile merge their (max, sum, O) in LDS at the end.
//
// The other orientation, S = Q K^T and O = P V with the query rows on the MFMA M axis,
// is instantiated beside it (template flag QM, chosen per plan): the score accumulator
// then holds four rows of one token per lane, so P goes through a per-wave LDS scratch
// to become an A operand, and row maxima take DPP reductions across 16 lanes.  It is
// the measured alternative, slower on the compute-bound shapes.
#include <type_traits>

#include "common.hpp"
#include "fair_share.hpp"
#include "row_store.hpp"
#include "kv_addr.hpp"

namespace pa {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// 16x16x128 with e4m3 A and B (32 bytes per lane): A lane l holds row l%16 and B lane l
// column l%16, both over the same 32 K positions of lane group l/16; C as for 16x16x32.
// SCALE_B is an E8M0 exponent (127 = x1) applied to B.
template <int SCALE_B>
__device__ __forceinline__ f32x4 mfma_fp8_k128(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, SCALE_B);
}
// The same with the E8M0 exponent applied to A.
template <int SCALE_A>
__device__ __forceinline__ f32x4 mfma_fp8_k128_sa(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, SCALE_A, 0, 127);
}

// q.k products with the key tokens on the MFMA M axis (S^T = K Q^T, QM false) or the
// query rows on it (S = Q K^T, QM true): the A and B operands have the same per-lane
// layout, so the orientation is the order of the two operands.
template <bool QM>
__device__ __forceinline__ f32x4 mfma_bf16_o(bf16x8 k, bf16x8 q, f32x4 c) {
  return QM ? mfma_bf16(q, k, c) : mfma_bf16(k, q, c);
}
template <bool QM>
__device__ __forceinline__ f32x4 mfma_fp8_o(long k, long q, f32x4 c) {
  return QM ? mfma_fp8(q, k, c) : mfma_fp8(k, q, c);
}
template <bool QM>
__device__ __forceinline__ i32x4 mfma_i8(i32x4 k, i32x4 q, i32x4 c) {
  return QM ? __builtin_amdgcn_mfma_i32_16x16x64_i8(q, k, c, 0, 0, 0)
            : __builtin_amdgcn_mfma_i32_16x16x64_i8(k, q, c, 0, 0, 0);
}

// Maximum and sum over the 16 lanes of each lane group (DPP within a row of 16 lanes:
// swap neighbours, swap pairs, mirror halves of 8, mirror the 16).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane16_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));      // quad_perm 1,0,3,2
  x = fmaxf(x, dpp_f<0x4E>(x));      // quad_perm 2,3,0,1
  x = fmaxf(x, dpp_f<0x141>(x));     // row_half_mirror
  return fmaxf(x, dpp_f<0x140>(x));  // row_mirror
}
// Value of lane 4 (l / 4) + r (DPP quad_perm r,r,r,r); r must be a constant.
__device__ __forceinline__ float quad_bcast(float x, int r) {
  switch (r) {
    case 0: return dpp_f<0x00>(x);
    case 1: return dpp_f<0x55>(x);
    case 2: return dpp_f<0xAA>(x);
    default: return dpp_f<0xFF>(x);
  }
}
__device__ __forceinline__ int quad_bcast_i(int x, int r) { return __float_as_int(quad_bcast(__int_as_float(x), r)); }
__device__ __forceinline__ float lane16_sum(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  return x + dpp_f<0x140>(x);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// KV: 0 bf16 cache, 1 e4m3 codes, 2 int8 codes (both one byte per element).
template <int DH, bool QF8, int KV, bool PT, int WQ, int NQB, int NS, int PD, bool QM = false>
struct S1Cfg {
  static constexpr bool KVF8 = KV != 0;             // one-byte codes (e4m3 or int8)
  static constexpr bool I8 = KV == 2;
  static constexpr int WT = 4 / WQ;                 // waves splitting the tokens of a tile
  static constexpr int BN = 32 * WT;                // tokens per tile
  static constexpr int KVB = KVF8 ? 1 : 2;          // bytes per cached element in HBM
  // LDS holds bf16 tiles for bf16 caches.  For per-token-head FP8 caches read with
  // bf16 queries by four query-block waves, K is upconverted once when a tile is stored
  // (instead of once by every wave that reads it) while V stays FP8, which halves the
  // bytes of the transposing V reads that bound this shape.  INT8 codes have no packed
  // conversion to bf16 (two to three VALU operations per value), so both K and V are
  // converted once, when the tile is stored.
  // With four query-block waves reading every per-token-head FP8 tile (one block each),
  // bf16 queries are carried as two e4m3 terms with a per-row scale,
  // q ~ s_r (hi + lo / 16), so that q.k runs on the double-rate 16x16x128 FP8 MFMA
  // straight from the e4m3 K tile: no K upconversion, and K occupies half the LDS
  // bytes (and read instructions) of a bf16 tile.  Measured 4% faster there; with one
  // or two query-block waves (K upconverted as it is read) and with three blocks per
  // wave it measured 2-5% slower, so those keep bf16 MFMA on upconverted K.
  static constexpr bool QX2 = KV == 1 && !QF8 && PT && WQ == 4 && NQB == 1;
  // The INT8 counterpart: two int8 query terms (q ~ s_r (hi + lo / 254), s_r =
  // amax_row / 127) on the 16x16x64 integer MFMA against the raw K codes, exact int32
  // sums, K kept in INT8 in LDS.
  static constexpr bool QI2 = I8 && !QF8 && PT && WQ == 4 && NQB == 1;
  // FP8 V of four one-block waves: the tile's V fragments are read before the softmax
  // (VPRE, all of them), or at head_dim 512, where all of them would take 64 registers,
  // the first VRA of them, the rest VRA steps ahead of their MFMAs (VRING).
  static constexpr bool VPRE = QX2 && !QM && DH < 512;
  static constexpr bool VRING = QX2 && !QM && DH == 512;
  static constexpr int VRA = 4;
  static constexpr bool LBF = !KVF8 || (I8 && !QI2) || (PT && !QF8 && WQ == 4 && !QX2 && !I8);   // K tile in bf16
  static constexpr bool LBFV = !KVF8 || I8;                               // V tile in bf16
  static constexpr int LKB = LBF ? 2 : 1;           // bytes per K element in LDS
  static constexpr int LVB = LBFV ? 2 : 1;          // bytes per V element in LDS
  static constexpr int CPR = DH * KVB / 16;         // 16-byte chunks per token row in HBM
  static constexpr int LCPR = DH * LKB / 16;        // 16-byte chunks per K token row in LDS
  static constexpr int VCPR = DH * LVB / 16;        // 16-byte chunks per V token row in LDS
  static constexpr int XPC = LKB / KVB;             // LDS K chunks stored per loaded chunk
  static constexpr int VXPC = LVB / KVB;            // LDS V chunks stored per loaded chunk
  static constexpr int TPI = 64 / CPR;              // tokens one wave covers per load step
  static constexpr int KTB = BN * DH * LKB;         // LDS bytes of one K tile
  static constexpr int VTB = BN * DH * LVB;         // LDS bytes of one V tile
  static constexpr int CPT = BN * CPR / 256;        // 16-byte chunks per thread per K (or V) tile
  static constexpr int SCB = PT ? 2 * BN * 4 : 0;   // scale bytes per stage: k_scale[BN], v_scale[BN]
  static constexpr int STAGEB = KTB + VTB + SCB;
  static constexpr int NPMAX = BN / 16 + 1;         // pages a tile can touch (page size >= 16)
  static constexpr int KC = DH / 32;                // K-steps of q.k (16x16x32 MFMA)
  static constexpr int KC2 = DH / 128;              // K-steps of q.k (16x16x128 FP8 MFMA, QX2)
  static constexpr int KC4 = DH / 64;               // K-steps of q.k (16x16x64 INT8 MFMA, QI2)
  static constexpr int DB = DH / 16;                // 16-wide d blocks of P.V
  static constexpr bool PV_FP8 = KVF8 && !PT;       // per-tensor FP8 V: fp8 MFMA for P.V
  // bf16 K and V operand fragments read this many steps ahead of their MFMAs (0: as the
  // compiler schedules them, one step ahead).  With one wave per SIMD (head_dim 512)
  // nothing else covers an LDS read's latency; two steps measured slightly faster than
  // four (eight spills).  With two waves per SIMD it gains nothing on the bf16 head_dim
  // 256 kernels and 1-2% on the compute-bound INT8 four-wave kernel (bf16 V in LDS).
  static constexpr int RA = QM ? 0 : DH == 512 ? 2 : (DH == 256 && KV == 2 && WQ == 4) ? 4 : 0;
  static constexpr int EPIB = (WT > 1) ? (4 * NQB * DB * 256 * 4 + 4 * NQB * 64 * 2 * 4) : 0;
  // Query blocks whose operand stays in registers.  Three blocks of bf16 queries against
  // per-token-head FP8 would need more than 256 VGPRs: the third block's operand lives in
  // LDS instead (16 B per lane and K-step, re-read every tile).  A spilled register
  // would be reloaded from scratch every tile, and the wait for that load also waits for
  // every tile load still in flight, which undoes the prefetch.
  static constexpr int QREG = (NQB == 3 && KVF8 && PT && !QF8) ? 2 : NQB;
  static constexpr int QLB = (NQB - QREG) * KC * 1024;   // LDS bytes per wave
  // Query rows on the MFMA M axis (the alternative orientation): P is transposed through
  // a per-wave LDS scratch of 32 tokens x 16 rows in bf16 (two terms for bf16 V), which
  // also carries the final change of accumulator layout (1 KB per 16 x 16 block).
  static constexpr int PSB = QM ? (KVF8 ? 1024 : 2048) : 0;
  static constexpr int MAINB = NS * STAGEB + 4 * QLB + 4 * PSB;
  static constexpr int LDSB = MAINB > EPIB ? MAINB : EPIB;
  static_assert(CPT >= 1 && (BN * CPR) % 256 == 0, "tile must split evenly over 256 threads");
  static_assert(WT == 1 || NQB == 1, "query blocks per wave > 1 only without token split");
  static_assert(NS == 1 || NS == 2, "one or two LDS stages");
  static_assert(PD >= 1 && PD <= 3, "prefetch one to three tiles ahead");
  static_assert(2 * BN <= 256, "scale loads use one thread per token");
  static_assert(!QM || (!PV_FP8 && DH <= 256), "query rows on M: bf16 P.V, head_dim <= 256");
};

// XOR swizzles of the 16-byte chunk index inside a token row, chosen so the MFMA
// operand reads hit distinct LDS banks: K rows are read 16 tokens x one chunk; bf16
// V rows by ds_read_b64_tr_b16 (4 tokens x 2 chunks per 16 lanes); fp8 V rows by
// ds_read_b64_tr_b8 (tokens {0..7, 16..23} + 4g, one chunk).
template <int CPR>
__device__ __forceinline__ int swz_k(int t) {
  if constexpr (CPR >= 16) return t & 15;
  else return (t >> 1) & 7;
}
template <int CPR, bool FP8V>
__device__ __forceinline__ int swz_v(int t) {
  if constexpr (!FP8V) return 2 * (t & 7);
  else if constexpr (CPR == 8) return ((t >> 1) + 4 * ((t >> 4) & 1)) & 7;
  else return (t & 7) + 8 * ((t >> 4) & 1);
}

template <bool QF8>
struct QOperand;
template <>
struct QOperand<false> { using T = bf16x8; };
template <>
struct QOperand<true> { using T = long; };

template <int V>
using ic = std::integral_constant<int, V>;

template <int DH, bool QF8, int KV, bool PT, int WQ, int NQB, int NS, int PD, bool QM = false>
__global__ __launch_bounds__(256, DH == 512 ? 1 : 2) void stage1_kernel(Stage1Args a) {
  using C = S1Cfg<DH, QF8, KV, PT, WQ, NQB, NS, PD, QM>;
  constexpr bool KVF8 = C::KVF8;
  using QT = typename QOperand<QF8>::T;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDSB];

  const PaItem it = a.items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wq = wave % WQ;
  const int wt = wave / WQ;
  const int L16 = lane & 15;
  const int g = lane >> 4;
  const int G = a.group;
  const int Hq = a.hq;
  const int Mq = it.nrows * G;
  const int tb0 = it.tok_begin;
  const int te = it.tok_end;
  const int shift = a.page_shift;
  const int pmask = (1 << shift) - 1;

  // ---- query operand (registers, or LDS past QREG blocks), per-row limits -----------------
  QT qop[NQB][C::KC];                                    // blocks >= QREG are never touched
  uint8_t* const qlds = smem + NS * C::STAGEB + wave * C::QLB + lane * 16;
  auto qget = [&](int i, int kc) __attribute__((always_inline)) -> QT {
    if (i < C::QREG) return qop[i][kc];
    return *reinterpret_cast<const QT*>(qlds + ((i - C::QREG) * C::KC + kc) * 1024);
  };
  int lim_lo[NQB], lim_hi[NQB];
  bool qvalid[NQB];
  float qsc[NQB];                     // FP8 query scale of this lane's row (per tensor or per head)
  const int hstep = a.scale_per_head; // 1: scales indexed by head, 0: one scale
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    const int qb = it.qblk0 + wq + WQ * i;
    qvalid[i] = 16 * qb < Mq;
    const int m = 16 * qb + L16;
    const int mr = m < Mq ? m : Mq - 1;
    const int r = mr / G;
    const int hl = mr - r * G;
    const int p = it.kv_len - it.nrows + r;
    const int lo = it.window > 0 ? max(0, p - it.window + 1) : 0;
    lim_lo[i] = max(lo, tb0);
    lim_hi[i] = min(p, te - 1);
    qsc[i] = QF8 ? a.q_scale[(it.kvh * G + hl) * hstep] : 1.0f;
  }
  int qpos[NQB];                      // query rows on M: position of row 4g + (L16 & 3)
  if constexpr (QM) {
#pragma unroll
    for (int i = 0; i < NQB; ++i)
      qpos[i] = it.kv_len - it.nrows + min(16 * (it.qblk0 + wq + WQ * i) + 4 * g + (L16 & 3), Mq - 1) / G;
  }
  // Tokens every real row of the item sees (fast path: no masking inside).
  const int p_first = it.kv_len - it.nrows;
  const int lo_last = it.window > 0 ? max(0, it.kv_len - 1 - it.window + 1) : 0;
  const int vis_lo_all = max(lo_last, tb0);
  const int vis_hi_all = min(p_first, te - 1);

  // Score scale into the log2 domain.  Per-tensor / per-head K and Q scales are folded
  // into xsb (one value per query block and lane: with per-head Q scales each row of the
  // block has its head's); per-token-head K scales are applied per token in the tile.
  float qk_scale = a.sm_scale * kLog2e;
  if constexpr (KVF8 && !PT) qk_scale *= a.k_scale[it.kvh * hstep];
  float xsb[NQB];
#pragma unroll
  for (int i = 0; i < NQB; ++i) xsb[i] = PT ? qsc[i] : qk_scale * qsc[i];
  float out_scale = 1.0f;
  if constexpr (C::PV_FP8) out_scale = a.v_scale[it.kvh * hstep];   // P carried x448, and so does l

  f32x4 o[NQB][C::DB];
  f32x4 olo[C::PV_FP8 ? NQB : 1][C::PV_FP8 ? C::DB : 1];
  float mrun[NQB], lrun[NQB];
  // With the query rows on M a lane holds rows 4g .. 4g+3 of each block: their partial
  // sums (over the lane's tokens) and score scales, and, packed one row per lane (row
  // 4g + (L16 & 3), read by the other lanes of the quad through DPP), their running
  // maxima.
  float lq[NQB][4], xq[NQB][4], mqp[NQB];
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    mrun[i] = -INFINITY;
    lrun[i] = 0.f;
    mqp[i] = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) lq[i][r] = 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[i][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  uint8_t* const pscr = smem + NS * C::STAGEB + 4 * C::QLB + wave * C::PSB;   // P transpose (QM)
  if constexpr (C::PV_FP8) {
#pragma unroll
    for (int i = 0; i < NQB; ++i)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) olo[i][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- KV tile loads: HBM -> registers -> LDS ------------------------------------------
  // Thread chunk i of a tile is 16-byte chunk cpos of token tb_i + lt (the page-gather
  // addressing of kv_addr.hpp: wave-uniform page and row, loop-invariant lane offset).
  // In LDS, position p (16-byte unit) of a K tile holds chunk (p % CPR) ^ swz_k(t) of
  // token t = p / CPR; V likewise with swz_v.
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k);
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v);
  using KA = KvTileAddr<C::CPR, C::BN, C::KVB>;
  const KA ka(lane, a.kv_ss);
  const cint32* pidx = (const cint32*)(a.page_indices) + it.page_base;
  const int64_t head_off = (int64_t)it.kvh * a.kv_sh;
  const int lt = ka.lt;
  const int cpos = ka.cpos;
  uint32_t kpos[C::CPT][C::XPC], vpos[C::CPT][C::VXPC];
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) {
    const int t = (wave * 64 + 256 * i) / C::CPR + lt;
#pragma unroll
    for (int x = 0; x < C::XPC; ++x) {
      const int c = cpos * C::XPC + x;
      kpos[i][x] = (t * C::LCPR + (c ^ swz_k<C::LCPR>(t))) << 4;
    }
#pragma unroll
    for (int x = 0; x < C::VXPC; ++x) {
      const int c = cpos * C::VXPC + x;
      vpos[i][x] = (t * C::VCPR + (c ^ swz_v<C::VCPR, !C::LBFV>(t))) << 4;
    }
  }
  u32x4 kreg[PD][C::CPT], vreg[PD][C::CPT];
  float sreg[PD];
  auto load_tile = [&](auto slot_c, int tile0) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
    // Page numbers of all load groups first, so that their scalar loads share one wait.
    // The clamps to the last token of the split are no-ops inside full tiles; keeping
    // them unconditional leaves the whole load sequence in one basic block.
    int jbs[C::CPT];
    int32_t pages[C::CPT];
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      jbs[i] = KA::group_token(tile0, wave, i, te);   // first token of this load (uniform)
      pages[i] = KA::group_page(pidx, jbs[i], shift);
    }
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int jb = jbs[i];
      const uint32_t off = ka.lane_offset(jb, te, a.kv_ss);
      const int64_t row = KA::row_offset(pages[i], jb, a.kv_sp, head_off, a.kv_ss, pmask);
      // Streaming loads: every KV byte is read once, so keep it out of the caches;
      // normal loads must first evict (and write back) whatever dirty lines the
      // preceding kernels left in L2/MALL, which halves the achieved HBM rate.
      kreg[SL][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + row + off));
      vreg[SL][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + row + off));
    }
    if constexpr (PT) {
      if (tid < 2 * C::BN) {
        const ScaleTileAddr<C::BN, C::NPMAX> sa(pidx, tile0, te, shift, tid, it.kvh, a.sc_sp, a.sc_sh, a.sc_ss);
        sreg[SL] = __builtin_nontemporal_load((sa.is_v ? a.v_scale : a.k_scale) + sa.off);
      }
    }
  };
  auto store_tile = [&](auto slot_c, uint8_t* stage) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      if constexpr (C::XPC == 1) {
        *reinterpret_cast<u32x4*>(stage + kpos[i][0]) = kreg[SL][i];
      } else {                 // 16 one-byte codes -> two chunks of 8 bf16 (exact)
        const u32x4 kq = kreg[SL][i];
        *reinterpret_cast<bf16x8*>(stage + kpos[i][0]) = codes8_to_bf16x8<C::I8>(kq[0], kq[1]);
        *reinterpret_cast<bf16x8*>(stage + kpos[i][1]) = codes8_to_bf16x8<C::I8>(kq[2], kq[3]);
      }
      if constexpr (C::VXPC == 1) {
        *reinterpret_cast<u32x4*>(stage + C::KTB + vpos[i][0]) = vreg[SL][i];
      } else {
        const u32x4 vq = vreg[SL][i];
        *reinterpret_cast<bf16x8*>(stage + C::KTB + vpos[i][0]) = codes8_to_bf16x8<C::I8>(vq[0], vq[1]);
        *reinterpret_cast<bf16x8*>(stage + C::KTB + vpos[i][1]) = codes8_to_bf16x8<C::I8>(vq[2], vq[3]);
      }
    }
    if constexpr (PT) {
      if (tid < 2 * C::BN) reinterpret_cast<float*>(stage + C::KTB + C::VTB)[tid] = sreg[SL];
    }
  };

  const int ntiles = te > tb0 ? (te - tb0 + C::BN - 1) / C::BN : 0;

  // Loop-invariant LDS offsets of this lane's operand reads.
  const int tk0 = wt * 32 + L16;                         // K rows: tokens tk0 and tk0 + 16
  uint32_t kro[2][C::KC];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      const int t = tk0 + 16 * tb;
      if constexpr (C::LBF) kro[tb][kc] = t * (C::LCPR * 16) + (((4 * kc + g) ^ swz_k<C::LCPR>(t)) << 4);
      else kro[tb][kc] = t * (C::LCPR * 16) + (((2 * kc + (g >> 1)) ^ swz_k<C::LCPR>(t)) << 4) + 8 * (g & 1);
    }
  // QX2: lane group g reads the two 16-byte chunks 8*ks + 2g, +1 of tokens tk0, tk0 + 16.
  uint32_t kro2[2][C::KC2][2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int ks = 0; ks < C::KC2; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = tk0 + 16 * tb;
        kro2[tb][ks][h] = t * (C::LCPR * 16) + (((8 * ks + 2 * g + h) ^ swz_k<C::LCPR>(t)) << 4);
      }
  // QI2: lane group g reads 16-byte chunk 4*ks + g of tokens tk0, tk0 + 16.
  uint32_t kro4[2][C::KC4];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int ks = 0; ks < C::KC4; ++ks) {
      const int t = tk0 + 16 * tb;
      kro4[tb][ks] = t * (C::LCPR * 16) + (((4 * ks + g) ^ swz_k<C::LCPR>(t)) << 4);
    }
  // V rows read transposed: bf16 -> two 4-token reads (tokens 4g+j and 16+4g+j);
  // fp8 -> one 8-token read (tokens {4g..4g+3, 16+4g..16+4g+3}).
  auto vaddr = [&](int db, int half) __attribute__((always_inline)) -> uint32_t {
    if constexpr (C::LBFV) {
      const int t1 = wt * 32 + 4 * g + (L16 >> 2) + 16 * half;
      const int c = 2 * db + ((L16 & 3) >> 1);
      return t1 * (C::VCPR * 16) + ((c ^ swz_v<C::VCPR, false>(t1)) << 4) + 8 * (L16 & 1);
    } else {
      const int jr = L16 >> 1;
      const int tv = wt * 32 + (jr < 4 ? 4 * g + jr : 16 + 4 * g + (jr - 4));
      return tv * (C::VCPR * 16) + ((db ^ swz_v<C::VCPR, true>(tv)) << 4) + 8 * (L16 & 1);
    }
  };
  // V operand of one 16-channel block for 32 tokens, bf16 (k order {4g..4g+3,
  // 16+4g..16+4g+3}; lane L16 = channel): A operand of O^T += V^T P^T, B operand of
  // O += P V.
  auto vfrag = [&](const uint8_t* Vl, int db) __attribute__((always_inline)) -> bf16x8 {
    bf16x8 va;
    if constexpr (C::LBFV) {
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4*)(Vl + vaddr(db, 0)));
      const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4*)(Vl + vaddr(db, 1)));
      const __bf16* p1 = reinterpret_cast<const __bf16*>(&v1);
      const __bf16* p2 = reinterpret_cast<const __bf16*>(&v2);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        va[k] = p1[k];
        va[4 + k] = p2[k];
      }
    } else {
      const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((PA_LDS i32x2*)(Vl + vaddr(db, 0)));
      va = fp8x8_to_bf16x8((uint32_t)w[0], (uint32_t)w[1]);
    }
    return va;
  };
  const bool wave_has_rows = qvalid[0];
  // exponent offset: per-tensor FP8 V scales P into [0, 448] inside exp2 (the final
  // normaliser divides the 448 out again because l accumulates the scaled P)
  constexpr float kPoff = C::PV_FP8 ? 8.807354922057604f : 0.0f;   // log2(448)

  // One tile of this wave, query block by query block: S^T, online softmax, O^T += V^T P^T.
  // (The compiler overlaps one block's MFMAs with the previous block's softmax; reading
  // each K/V fragment once for all blocks instead serialises those phases.)
  auto compute_tile = [&](int tile0, const uint8_t* stage) __attribute__((always_inline)) {
    const uint8_t* Kl = stage;
    const uint8_t* Vl = stage + C::KTB;
    const float* ksl = reinterpret_cast<const float*>(stage + C::KTB + C::VTB);
    const float* vsl = ksl + C::BN;
    const int c0 = tile0 + wt * 32;          // first token of this wave's 32-token chunk
    if (!(c0 < te && wave_has_rows)) return;
    const bool need_mask = !(c0 >= vis_lo_all && c0 + 31 <= vis_hi_all);
    // Per-token-head scales of the lane's tokens: with K on M, tokens {4g..4g+3,
    // 16+4g..16+4g+3} of the chunk; with Q on M, tokens L16 and 16 + L16.
    constexpr int NT = QM ? 2 : 8;
    float ks[NT], vs[NT];
    if constexpr (PT) {
      if constexpr (QM) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          ks[h] = ksl[wt * 32 + 16 * h + L16] * qk_scale;
          vs[h] = vsl[wt * 32 + 16 * h + L16];
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          ks[k] = ksl[wt * 32 + 4 * g + k] * qk_scale;
          ks[4 + k] = ksl[wt * 32 + 16 + 4 * g + k] * qk_scale;
          vs[k] = vsl[wt * 32 + 4 * g + k];
          vs[4 + k] = vsl[wt * 32 + 16 + 4 * g + k];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NQB; ++i) {
      if (!qvalid[i]) continue;
      // ---- S^T = K Q^T (or S = Q K^T) for 2 x 16 tokens ---------------------------------
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (C::QX2) {
#pragma unroll
        for (int ks = 0; ks < C::KC2; ++ks) {
          auto kld = [&](int tb) __attribute__((always_inline)) -> i32x8 {
            const i32x4 c0 = *reinterpret_cast<const i32x4*>(Kl + kro2[tb][ks][0]);
            const i32x4 c1 = *reinterpret_cast<const i32x4*>(Kl + kro2[tb][ks][1]);
            return __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
          };
          auto qld = [&](int u) __attribute__((always_inline)) -> i32x4 {
            return __builtin_bit_cast(i32x4, qget(i, 4 * ks + u));
          };
          const i32x8 qh = __builtin_shufflevector(qld(0), qld(1), 0, 1, 2, 3, 4, 5, 6, 7);
          const i32x8 ql = __builtin_shufflevector(qld(2), qld(3), 0, 1, 2, 3, 4, 5, 6, 7);
          const i32x8 k0 = kld(0), k1 = kld(1);
          if constexpr (QM) {
            s0 = mfma_fp8_k128_sa<127>(qh, k0, s0);
            s1 = mfma_fp8_k128_sa<127>(qh, k1, s1);
            s0 = mfma_fp8_k128_sa<123>(ql, k0, s0);
            s1 = mfma_fp8_k128_sa<123>(ql, k1, s1);
          } else {
            s0 = mfma_fp8_k128<127>(k0, qh, s0);
            s1 = mfma_fp8_k128<127>(k1, qh, s1);
            s0 = mfma_fp8_k128<123>(k0, ql, s0);     // lo term carries x16: scale 2^-4
            s1 = mfma_fp8_k128<123>(k1, ql, s1);
          }
        }
      }
      if constexpr (C::QI2) {
        i32x4 h0 = {0, 0, 0, 0}, l0 = {0, 0, 0, 0}, h1 = {0, 0, 0, 0}, l1 = {0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < C::KC4; ++ks) {
          const i32x4 k0 = *reinterpret_cast<const i32x4*>(Kl + kro4[0][ks]);
          const i32x4 k1 = *reinterpret_cast<const i32x4*>(Kl + kro4[1][ks]);
          const i32x4 qh = __builtin_bit_cast(i32x4, qget(i, 2 * ks));
          const i32x4 ql = __builtin_bit_cast(i32x4, qget(i, 2 * ks + 1));
          h0 = mfma_i8<QM>(k0, qh, h0);
          h1 = mfma_i8<QM>(k1, qh, h1);
          l0 = mfma_i8<QM>(k0, ql, l0);
          l1 = mfma_i8<QM>(k1, ql, l1);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {        // exact int32 sums (|sum| < 2^24) -> fp32
          s0[k] = fmaf((float)l0[k], 1.f / 254.f, (float)h0[k]);
          s1[k] = fmaf((float)l1[k], 1.f / 254.f, (float)h1[k]);
        }
      }
      if constexpr (C::LBF && C::RA > 0 && !C::QX2 && !C::QI2) {
        // ring of RA K-step fragment pairs: the reads for step kc + RA go out before the
        // MFMAs of step kc
        bf16x8 kr[C::RA][2];
        auto kread = [&](int kc, int tb) __attribute__((always_inline)) -> bf16x8 {
          return *reinterpret_cast<const bf16x8*>(Kl + kro[tb][kc]);
        };
#pragma unroll
        for (int p = 0; p < C::RA; ++p) {
          kr[p][0] = kread(p, 0);
          kr[p][1] = kread(p, 1);
        }
#pragma unroll
        for (int kc = 0; kc < C::KC; ++kc) {
          const bf16x8 k0 = kr[kc % C::RA][0], k1 = kr[kc % C::RA][1];
          if (kc + C::RA < C::KC) {
            kr[kc % C::RA][0] = kread(kc + C::RA, 0);
            kr[kc % C::RA][1] = kread(kc + C::RA, 1);
          }
          const QT qv = qget(i, kc);
          s0 = mfma_bf16(k0, qv, s0);
          s1 = mfma_bf16(k1, qv, s1);
          __builtin_amdgcn_sched_barrier(0);   // keep the read-ahead in this step
        }
      }
#pragma unroll
      for (int kc = 0; kc < ((C::QX2 || C::QI2 || (C::LBF && C::RA > 0)) ? 0 : C::KC); ++kc) {
        if constexpr (C::LBF) {
          const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(Kl + kro[0][kc]);
          const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(Kl + kro[1][kc]);
          const QT qv = qget(i, kc);
          s0 = mfma_bf16_o<QM>(k0, qv, s0);
          s1 = mfma_bf16_o<QM>(k1, qv, s1);
        } else {
          const uint2 r0 = *reinterpret_cast<const uint2*>(Kl + kro[0][kc]);
          const uint2 r1 = *reinterpret_cast<const uint2*>(Kl + kro[1][kc]);
          if constexpr (QF8) {
            s0 = mfma_fp8_o<QM>((long)r0.x | ((long)r0.y << 32), qop[i][kc], s0);
            s1 = mfma_fp8_o<QM>((long)r1.x | ((long)r1.y << 32), qop[i][kc], s1);
          } else {
            s0 = mfma_bf16_o<QM>(fp8x8_to_bf16x8(r0.x, r0.y), qop[i][kc], s0);
            s1 = mfma_bf16_o<QM>(fp8x8_to_bf16x8(r1.x, r1.y), qop[i][kc], s1);
          }
        }
      }
      // ---- scale, mask, online softmax -----------------------------------------------
      float x[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[k] = s0[k];
        x[4 + k] = s1[k];
      }
      if constexpr (QM) {
        // Lane (L16, g) holds S[row 4g + r][token L16] in x[r] and S[row 4g + r][token
        // 16 + L16] in x[4 + r]: four rows per lane, each row spread over 16 lanes.
        if constexpr (PT) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x[r] *= ks[0];
            x[4 + r] *= ks[1];
          }
        }
        if (need_mask) {
          // visible range of row 4g + (L16 & 3) (as lim_lo / lim_hi), then of each row r
          const int lop = max(it.window > 0 ? max(0, qpos[i] - it.window + 1) : 0, tb0);
          const int hip = min(qpos[i], te - 1);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int lo = quad_bcast_i(lop, r), hi = quad_bcast_i(hip, r);
            x[r] = (c0 + L16 >= lo && c0 + L16 <= hi) ? x[r] : -INFINITY;
            x[4 + r] = (c0 + 16 + L16 >= lo && c0 + 16 + L16 <= hi) ? x[4 + r] : -INFINITY;
          }
        }
        float mx[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) mx[r] = lane16_max(fmaxf(x[r], x[4 + r])) * xq[i][r];
        const int sel = L16 & 3;
        const float mxp = sel == 0 ? mx[0] : sel == 1 ? mx[1] : sel == 2 ? mx[2] : mx[3];
        const float mnew = fmaxf(mqp[i], mxp);
        const float musep = (mnew == -INFINITY) ? 0.f : mnew;
        if (__builtin_amdgcn_ballot_w64(mnew != mqp[i]) != 0) {     // lazy rescale
          const float alpha = fast_exp2(mqp[i] - musep);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float ar = quad_bcast(alpha, r);
            lq[i][r] *= ar;
#pragma unroll
            for (int db = 0; db < C::DB; ++db) o[i][db][r] *= ar;
          }
          mqp[i] = mnew;
        }
        // P, transposed through this wave's LDS scratch: P^T[token][row] (32 tokens x
        // 16 rows, bf16), read back as the A operand P[row][tokens {4g..4g+3,
        // 16+4g..16+4g+3}] with ds_read_b64_tr_b16 (the k order of the V operand below).
        uint8_t* pw = pscr + L16 * 32 + 8 * g;
        const uint8_t* pr = pscr + (4 * g + (L16 >> 2)) * 32 + 8 * (L16 & 3);
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x4 hv4, lv4;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = fast_exp2(fmaf(x[4 * h + r], xq[i][r], kPoff - quad_bcast(musep, r)));
            lq[i][r] += p;
            const float y = PT ? p * vs[h] : p;
            const __bf16 hb = (__bf16)y;
            hv4[r] = hb;
            if constexpr (!KVF8) lv4[r] = (__bf16)(y - (float)hb);
          }
          *reinterpret_cast<bf16x4*>(pw + 512 * h) = hv4;
          if constexpr (!KVF8) *reinterpret_cast<bf16x4*>(pw + 1024 + 512 * h) = lv4;
        }
        auto pread = [&](int term) __attribute__((always_inline)) -> bf16x8 {
          const i16x4 u1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4*)(pr + 1024 * term));
          const i16x4 u2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4*)(pr + 1024 * term + 512));
          bf16x8 r8;
          const __bf16* p1 = reinterpret_cast<const __bf16*>(&u1);
          const __bf16* p2 = reinterpret_cast<const __bf16*>(&u2);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            r8[k] = p1[k];
            r8[4 + k] = p2[k];
          }
          return r8;
        };
        const bf16x8 ph = pread(0);
        bf16x8 pl;
        if constexpr (!KVF8) pl = pread(1);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const bf16x8 vb = vfrag(Vl, db);
          o[i][db] = mfma_bf16(ph, vb, o[i][db]);
          if constexpr (!KVF8) o[i][db] = mfma_bf16(pl, vb, o[i][db]);
        }
        continue;
      }
      // Four one-block waves on FP8 V: the tile's V fragments (at head_dim 512 the first
      // VRA of them) are requested here, before the softmax, so that their LDS latency
      // hides behind it (in the P.V loop each read would otherwise be waited for on its own).
      i32x2 vraw[C::VPRE ? C::DB : C::VRING ? C::VRA : 1];
      if constexpr (C::VPRE || C::VRING) {
#pragma unroll
        for (int db = 0; db < (C::VPRE ? C::DB : C::VRA); ++db)
          vraw[db] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((PA_LDS i32x2*)(Vl + vaddr(db, 0)));
      }
      const float xs = xsb[i];               // score scale still to apply
      if constexpr (PT) {
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] *= ks[k];
      }
      if (need_mask) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int j = c0 + (k < 4 ? 4 * g + k : 16 + 4 * g + (k - 4));
          x[k] = (j >= lim_lo[i] && j <= lim_hi[i]) ? x[k] : -INFINITY;
        }
      }
      float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      mx = wave_max_xor_16_32(mx) * xs;
      const float mnew = fmaxf(mrun[i], mx);
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      if (__builtin_amdgcn_ballot_w64(mnew != mrun[i]) != 0) {     // lazy rescale
        const float alpha = fast_exp2(mrun[i] - muse);
        lrun[i] *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) o[i][db] *= alpha;
        if constexpr (C::PV_FP8) {
#pragma unroll
          for (int db = 0; db < C::DB; ++db) olo[i][db] *= alpha;
        }
        mrun[i] = mnew;
      }
      const float nb = kPoff - muse;
      float pv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        pv[k] = fast_exp2(fmaf(x[k], xs, nb));
        lrun[i] += pv[k];
      }
      // ---- P operand and O^T += V^T P^T --------------------------------------------------
      if constexpr (C::PV_FP8) {
        const uint32_t h0 = f32x4_to_fp8x4(pv[0], pv[1], pv[2], pv[3]);
        const uint32_t h1 = f32x4_to_fp8x4(pv[4], pv[5], pv[6], pv[7]);
        const f32x2 d0 = fp8x2_to_f32x2<false>(h0), d1 = fp8x2_to_f32x2<true>(h0);
        const f32x2 d2 = fp8x2_to_f32x2<false>(h1), d3 = fp8x2_to_f32x2<true>(h1);
        const uint32_t l0 = f32x4_to_fp8x4((pv[0] - d0[0]) * 16.f, (pv[1] - d0[1]) * 16.f,
                                           (pv[2] - d1[0]) * 16.f, (pv[3] - d1[1]) * 16.f);
        const uint32_t l1 = f32x4_to_fp8x4((pv[4] - d2[0]) * 16.f, (pv[5] - d2[1]) * 16.f,
                                           (pv[6] - d3[0]) * 16.f, (pv[7] - d3[1]) * 16.f);
        const long phi = (long)h0 | ((long)h1 << 32);
        const long plo = (long)l0 | ((long)l1 << 32);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((PA_LDS i32x2*)(Vl + vaddr(db, 0)));
          const long va = (long)(uint32_t)w[0] | ((long)(uint32_t)w[1] << 32);
          o[i][db] = mfma_fp8(va, phi, o[i][db]);
          olo[i][db] = mfma_fp8(va, plo, olo[i][db]);
        }
      } else {
        bf16x8 hv, lv;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float y = PT ? pv[k] * vs[k] : pv[k];
          const __bf16 h = (__bf16)y;
          hv[k] = h;
          if constexpr (!KVF8) lv[k] = (__bf16)(y - (float)h);
        }
        if constexpr (C::LBFV && C::RA > 0) {
          // ring of RA d-block fragments (two transposing reads each), as for K
          i16x4 vr[C::RA][2];
#pragma unroll
          for (int p = 0; p < C::RA; ++p) {
            vr[p][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4*)(Vl + vaddr(p, 0)));
            vr[p][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4*)(Vl + vaddr(p, 1)));
          }
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const i16x4 v1 = vr[db % C::RA][0], v2 = vr[db % C::RA][1];
            if (db + C::RA < C::DB) {
              vr[db % C::RA][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4*)(Vl + vaddr(db + C::RA, 0)));
              vr[db % C::RA][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4*)(Vl + vaddr(db + C::RA, 1)));
            }
            const auto w = __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7);
            const bf16x8 va = __builtin_bit_cast(bf16x8, w);
            o[i][db] = mfma_bf16(va, hv, o[i][db]);
            if constexpr (!KVF8) o[i][db] = mfma_bf16(va, lv, o[i][db]);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else if constexpr (C::VRING) {
          // fragment db + 1 is converted while the MFMA of db runs; slot r of vraw holds
          // fragments r, r + VRA, ... in turn, each refilled when its fragment is converted
          auto vread = [&](int db) __attribute__((always_inline)) -> i32x2 {
            return __builtin_amdgcn_ds_read_tr8_b64_v2i32((PA_LDS i32x2*)(Vl + vaddr(db, 0)));
          };
          bf16x8 vnext = fp8x8_to_bf16x8((uint32_t)vraw[0][0], (uint32_t)vraw[0][1]);
          if (C::VRA < C::DB) vraw[0] = vread(C::VRA);
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const bf16x8 va = vnext;
            if (db + 1 < C::DB) {
              const int r = (db + 1) % C::VRA;
              vnext = fp8x8_to_bf16x8((uint32_t)vraw[r][0], (uint32_t)vraw[r][1]);
              if (db + 1 + C::VRA < C::DB) vraw[r] = vread(db + 1 + C::VRA);
            }
            o[i][db] = mfma_bf16(va, hv, o[i][db]);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            bf16x8 va;
            if constexpr (C::VPRE) va = fp8x8_to_bf16x8((uint32_t)vraw[db][0], (uint32_t)vraw[db][1]);
            else va = vfrag(Vl, db);
            o[i][db] = mfma_bf16(va, hv, o[i][db]);
            if constexpr (!KVF8) o[i][db] = mfma_bf16(va, lv, o[i][db]);
          }
        }
      }
    }
  };

  // One tile: refill the register slot that held it PD tiles ahead, compute it, then
  // move the next tile from registers to LDS.  FULL steps do this unconditionally,
  // which keeps the compiler's load-counter bookkeeping exact in the steady state
  // (a conditional load there makes it wait for every outstanding tile).
  auto step = [&](auto slot_c, auto full_c, int ti) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
    constexpr bool FULL = decltype(full_c)::value != 0;
    const int tile0 = tb0 + ti * C::BN;
    if (FULL || ti + PD < ntiles) load_tile(ic<SL>{}, tile0 + PD * C::BN);
    compute_tile(tile0, smem + (ti % NS) * C::STAGEB);
    if (FULL || ti + 1 < ntiles) {
      if constexpr (NS == 1) __syncthreads();
      store_tile(ic<(SL + 1) % PD>{}, smem + ((ti + 1) % NS) * C::STAGEB);
      __syncthreads();
    }
  };

  // Two-term FP8 query: the bf16 row is requested before the first tiles, so that its
  // conversion below waits for it alone and runs while the tiles are in flight.
  bf16x8 qraw[C::QX2 ? C::KC2 : 1][4];
  if constexpr (C::QX2) {
    static_assert(NQB == 1, "two-term query: one block per wave");
    const int m = 16 * (it.qblk0 + wq) + L16;
    const int mr = m < Mq ? m : Mq - 1;
    const int r = mr / G;
    const int hl = mr - r * G;
    const __bf16* qp = static_cast<const __bf16*>(a.q) + ((int64_t)(it.row0 + r) * Hq + (int64_t)it.kvh * G + hl) * DH;
#pragma unroll
    for (int ks = 0; ks < C::KC2; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j) qraw[ks][j] = *reinterpret_cast<const bf16x8*>(qp + 128 * ks + 32 * g + 8 * j);
  }
  if (ntiles > 0) {
    load_tile(ic<0>{}, tb0);
    if constexpr (PD >= 2) {
      if (ntiles > 1) load_tile(ic<1>{}, tb0 + C::BN);
    }
    if constexpr (PD >= 3) {
      if (ntiles > 2) load_tile(ic<2>{}, tb0 + 2 * C::BN);
    }
  }
  // Query operand, loaded after the first tiles and waited for completely here: a
  // load still pending at the loop entry would make every iteration wait for all
  // outstanding tile loads before its first MFMA.
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    const int m = 16 * (it.qblk0 + wq + WQ * i) + L16;
    const int mr = m < Mq ? m : Mq - 1;                // rows past Mq repeat the last real row
    const int r = mr / G;
    const int hl = mr - r * G;
    const int64_t qrow = ((int64_t)(it.row0 + r) * Hq + (int64_t)it.kvh * G + hl) * DH;
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      if constexpr (C::QX2 || C::QI2) break;
      QT v;
      if constexpr (QF8)
        v = *reinterpret_cast<const long*>(static_cast<const uint8_t*>(a.q) + qrow + kc * 32 + 8 * g);
      else
        v = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.q) + qrow + kc * 32 + 8 * g);
      if (i < C::QREG) qop[i][kc] = v;
      else *reinterpret_cast<QT*>(qlds + ((i - C::QREG) * C::KC + kc) * 1024) = v;   // read back by this lane only
    }
    if constexpr (C::QI2) {
      // Lane group g holds d = 64*ks + 16*g .. +15 of its row for every K-step ks.  The
      // row is scaled so that its largest magnitude maps to 127 and rounded to integers
      // (hi); the residual in [-1/2, 1/2], x254, is rounded again (lo): q = s_r (hi +
      // lo/254) to ~2^-16 of amax.  16-byte unit 2*ks + term holds 16 codes of term.
      const __bf16* qp = static_cast<const __bf16*>(a.q) + qrow;
      bf16x8 raw[C::KC4][2];
      float amax = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KC4; ++ks)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          raw[ks][j] = *reinterpret_cast<const bf16x8*>(qp + 64 * ks + 16 * g + 8 * j);
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)raw[ks][j][e]));
        }
      amax = wave_max_xor_16_32(amax);
      const float inv = amax > 0.f ? 127.f / amax : 1.f;
      xsb[i] *= amax > 0.f ? amax * (1.f / 127.f) : 1.f;
#pragma unroll
      for (int ks = 0; ks < C::KC4; ++ks) {
        u32x4 hi, lo;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t h = 0, l = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = fminf(fmaxf((float)raw[ks][w >> 1][4 * (w & 1) + e] * inv, -127.f), 127.f);
            const float xh = __builtin_rintf(x);
            const float xl = fminf(fmaxf(__builtin_rintf((x - xh) * 254.f), -127.f), 127.f);
            h |= ((uint32_t)(int)xh & 0xFFu) << (8 * e);
            l |= ((uint32_t)(int)xl & 0xFFu) << (8 * e);
          }
          hi[w] = h;
          lo[w] = l;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const QT v = __builtin_bit_cast(QT, u == 0 ? hi : lo);
          if (i < C::QREG) qop[i][2 * ks + u] = v;
          else *reinterpret_cast<QT*>(qlds + ((i - C::QREG) * C::KC + 2 * ks + u) * 1024) = v;
        }
      }
    }
    if constexpr (C::QX2) {
      // Lane group g holds d = 128*ks + 32*g .. +31 of its row for every K-step ks.  The
      // row is scaled so that its largest magnitude maps to 448, rounded to e4m3 (hi),
      // and the residual, x16, rounded again (lo): q = s_r (hi + lo/16) to ~2^-8
      // relative, and s_r joins the row's score scale.  16-byte unit 4*ks + 2*term + half
      // of the operand store holds 16 codes of term (0 hi, 1 lo).
      bf16x8 (&raw)[C::KC2][4] = qraw;
      float amax = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KC2; ++ks)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)raw[ks][j][e]));
        }
      amax = wave_max_xor_16_32(amax);
      const float inv = amax > 0.f ? 448.f / amax : 1.f;
      xsb[i] *= amax > 0.f ? amax * (1.f / 448.f) : 1.f;
#pragma unroll
      for (int ks = 0; ks < C::KC2; ++ks) {
        u32x4 hi[2], lo[2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (float)raw[ks][j][4 * w + e] * inv;
            const uint32_t h = f32x4_to_fp8x4(x[0], x[1], x[2], x[3]);
            const f32x2 d0 = fp8x2_to_f32x2<false>(h), d1 = fp8x2_to_f32x2<true>(h);
            hi[j >> 1][2 * (j & 1) + w] = h;
            lo[j >> 1][2 * (j & 1) + w] = f32x4_to_fp8x4((x[0] - d0[0]) * 16.f, (x[1] - d0[1]) * 16.f,
                                                         (x[2] - d1[0]) * 16.f, (x[3] - d1[1]) * 16.f);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const QT v = __builtin_bit_cast(QT, u < 2 ? hi[u] : lo[u - 2]);
          if (i < C::QREG) qop[i][4 * ks + u] = v;
          else *reinterpret_cast<QT*>(qlds + ((i - C::QREG) * C::KC + 4 * ks + u) * 1024) = v;
        }
      }
    }
  }
  if constexpr (QM) {
    // score scale of row 4g + r: that of lane L16 = 4g + r (the same in every lane group;
    // one value for all rows unless the query carries per-head or per-row scales)
#pragma unroll
    for (int i = 0; i < NQB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        xq[i][r] = (!QF8 && !C::QX2 && !C::QI2) ? xsb[i] : __shfl(xsb[i], 4 * g + r);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F & ~0xC00F);          // vmcnt(0) lgkmcnt(0)
  if (ntiles > 0) {
    store_tile(ic<0>{}, smem);
    __syncthreads();
  }
  int ti = 0;
  // Issue-priority balance with the other workgroup of the CU (FairShare), for one-block
  // waves: with several blocks per wave the added loop check measured 2% slower on the
  // ragged mix, whose plans run in more than one round anyway.
  constexpr bool FAIRK = !QM && NQB == 1;
  const FairShare fs(FAIRK && a.fair, ntiles, PD);
  for (; ti + 2 * PD - 1 < ntiles; ti += PD) {         // steady state
    if constexpr (FAIRK) fs.at(ti);
    step(ic<0>{}, ic<1>{}, ti);
    if constexpr (PD >= 2) step(ic<1>{}, ic<1>{}, ti + 1);
    if constexpr (PD >= 3) step(ic<2>{}, ic<1>{}, ti + 2);
  }
  for (; ti < ntiles; ti += PD) {                      // drain the last tiles
    step(ic<0>{}, ic<0>{}, ti);
    if constexpr (PD >= 2) {
      if (ti + 1 < ntiles) step(ic<1>{}, ic<0>{}, ti + 1);
    }
    if constexpr (PD >= 3) {
      if (ti + 2 < ntiles) step(ic<2>{}, ic<0>{}, ti + 2);
    }
  }
  if constexpr (QM) {
    // Back to the K-on-M accumulator layout the epilogue takes: lane (L16, g) gets row
    // L16's maximum, its sum (in lane group 0; the epilogue sums the four groups) and
    // O^T[16 db + 4g + r][row L16], through this wave's scratch.
    float* pf = reinterpret_cast<float*>(pscr);
#pragma unroll
    for (int i = 0; i < NQB; ++i) {
      float lt[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) lt[r] = lane16_sum(lq[i][r]);
      if (L16 == 0) *reinterpret_cast<f32x4*>(pf + 4 * g) = f32x4{lt[0], lt[1], lt[2], lt[3]};
      // row L16 = 4 (L16 >> 2) + (L16 & 3): packed in lane 16 (L16 >> 2) + (L16 & 3)
      mrun[i] = __shfl(mqp[i], 16 * (L16 >> 2) + (L16 & 3));
      lrun[i] = g == 0 ? pf[L16] : 0.f;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        *reinterpret_cast<f32x4*>(pf + L16 * 16 + 4 * g) = o[i][db];    // [channel][row]
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = pf[(4 * g + r) * 16 + L16];
        o[i][db] = v;
      }
    }
  }
  __syncthreads();

  // ---- epilogue ------------------------------------------------------------------------
  float ltot[NQB];
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    ltot[i] = wave_sum_xor_16_32(lrun[i]);
    if constexpr (C::PV_FP8) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db) o[i][db] += olo[i][db] * (1.0f / 16.0f);
    }
  }
  if constexpr (C::WT > 1) {
    // waves that split the tokens of a tile combine (max, sum, O) through LDS
    float* eo = reinterpret_cast<float*>(smem);
    float* em = eo + 4 * NQB * C::DB * 256;
    float* el = em + 4 * NQB * 64;
    if (wt > 0) {
#pragma unroll
      for (int i = 0; i < NQB; ++i) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
          *reinterpret_cast<f32x4*>(eo + ((wave * NQB + i) * C::DB + db) * 256 + lane * 4) = o[i][db];
        em[(wave * NQB + i) * 64 + lane] = mrun[i];
        el[(wave * NQB + i) * 64 + lane] = ltot[i];
      }
    }
    __syncthreads();
    if (wt == 0) {
#pragma unroll
      for (int i = 0; i < NQB; ++i) {
        float mall = mrun[i];
        for (int w2 = 1; w2 < C::WT; ++w2) mall = fmaxf(mall, em[((wq + WQ * w2) * NQB + i) * 64 + lane]);
        const float muse = (mall == -INFINITY) ? 0.f : mall;
        const float f0 = fast_exp2(mrun[i] - muse);
        float lsum = ltot[i] * f0;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) o[i][db] *= f0;
        for (int w2 = 1; w2 < C::WT; ++w2) {
          const int wv = wq + WQ * w2;
          const float f = fast_exp2(em[(wv * NQB + i) * 64 + lane] - muse);
          lsum += el[(wv * NQB + i) * 64 + lane] * f;
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
            o[i][db] += *reinterpret_cast<const f32x4*>(eo + ((wv * NQB + i) * C::DB + db) * 256 + lane * 4) * f;
        }
        mrun[i] = mall;
        ltot[i] = lsum;
      }
    }
  }
  if (wt != 0) return;

#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    if (!qvalid[i]) continue;
    const int m = 16 * (it.qblk0 + wq + WQ * i) + L16;
    if (m >= Mq) continue;
    const int r = m / G;
    const int hl = m - r * G;
    const int64_t th = (int64_t)(it.row0 + r) * Hq + (int64_t)it.kvh * G + hl;
    const bool empty = !(ltot[i] > 0.f);
    const float sc = empty ? 0.f : out_scale / ltot[i];
    const float lse = empty ? -INFINITY : (mrun[i] + __log2f(ltot[i]) - kPoff) * kLn2;
    if (it.nsplit == 1) {
      if (a.out_lse && g == 0) a.out_lse[th] = lse;
      if (a.out_bf16) {
        store_row_bf16_x16(static_cast<__bf16*>(a.out) + th * DH, o[i], sc, g);
      } else {
        float* dst = static_cast<float*>(a.out) + th * DH;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * g) = o[i][db] * sc;
      }
    } else if (a.part_bf16) {
      store_row_bf16_x16(static_cast<__bf16*>(a.partial_o) + (th * a.s_max + it.split) * DH, o[i], sc, g);
      if (g == 0) a.partial_lse[th * a.s_max + it.split] = lse;
    } else {
      float* dst = static_cast<float*>(a.partial_o) + (th * a.s_max + it.split) * DH;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * g) = o[i][db] * sc;
      if (g == 0) a.partial_lse[th * a.s_max + it.split] = lse;
    }
  }
}

// LDS stages and register prefetch depth: two stages when two workgroups still fit
// in the CU's 160 KiB of LDS, else one; two tiles of register prefetch when a tile
// costs at most 32 VGPRs per thread, else one.
template <int DH, bool QF8, int KV, bool PT, int WQ, int NQB>
struct Pipe {
  static constexpr bool KVF8 = KV != 0;
  static constexpr int BN = 32 * (4 / WQ);
  static constexpr bool QX2 = KV == 1 && !QF8 && PT && WQ == 4 && NQB == 1;   // as S1Cfg::QX2
  static constexpr bool QI2 = KV == 2 && !QF8 && PT && WQ == 4 && NQB == 1;   // as S1Cfg::QI2
  static constexpr bool LBF = !KVF8 || (KV == 2 && !QI2) || (PT && !QF8 && WQ == 4 && !QX2 && KV != 2);
  static constexpr bool LBFV = !KVF8 || KV == 2;                              // as S1Cfg::LBFV
  static constexpr int stage = BN * DH * ((LBF ? 2 : 1) + (LBFV ? 2 : 1)) + (PT ? 2 * BN * 4 : 0);
  // LDS per workgroup: 80 KB (two workgroups per CU), 160 KB for head_dim 512 (one)
  static constexpr int LDS_CAP = (DH == 512 ? 160 : 80) * 1024;
  static constexpr int NS = 2 * stage <= LDS_CAP ? 2 : 1;
  static constexpr int CPT = BN * DH * (KVF8 ? 1 : 2) / 16 / 256;
  // tiles in flight in registers (8 VGPRs per 16-byte chunk of K and V).  A third tile
  // measured slower on the d256 per-token-head shape (register pressure; also without
  // spills once K stays FP8), so at most two; head_dim 512 runs one wave per SIMD, whose
  // register file holds two of its 64 KB tiles (four FP8 tiles measured slower too).
  // head_dim 256 with per-tensor FP8 V (a second, lo-term accumulator) or with INT8 tiles
  // split over two token groups keeps one tile in flight: two would not fit beside the
  // accumulators in the 256 registers a wave has at two workgroups per CU.  bf16 KV at
  // head_dim 256 with four row-block waves keeps one too: measured c3 R8 177 -> 175 us
  // and c3 B1 R8 26.4 -> 24.8 us (32 KB tiles: with two in flight, the first compute of
  // a batch-1 launch waits for 32 MB requested by all workgroups at once); so does FP8
  // KV with two row-block waves (c4 R1 331.5 -> 327.5 us, c4 B1 R1 30.4 -> 30.0).  The
  // FP8 four-wave shape lost 4.5% with one and keeps two, as does head_dim 512 (c6 74.2
  // -> 75.3 us with one).
  static constexpr bool PV_FP8 = KV == 1 && !PT;
  static constexpr int PD = DH == 512 ? 2 : (DH == 256 && (PV_FP8 || (KV == 2 && WQ == 2) || (WQ == 4 && KV == 0) || (WQ == 2 && KV == 1))) ? 1 : (CPT <= 4 ? 2 : 1);
};

template <int DH, bool QF8, int KV, bool PT, int WQ, int NQB, bool QM = false>
static int launch_one(const Stage1Args& a, int num_items, void* stream) {
  using Pp = Pipe<DH, QF8, KV, PT, WQ, NQB>;
  using C = S1Cfg<DH, QF8, KV, PT, WQ, NQB, Pp::NS, Pp::PD, QM>;
  static_assert(Pp::stage == C::STAGEB, "host and kernel disagree on the LDS stage size");
  static_assert(C::LDSB <= Pp::LDS_CAP, "the workgroups of a CU must fit in its 160 KB of LDS");
  hipLaunchKernelGGL((stage1_kernel<DH, QF8, KV, PT, WQ, NQB, Pp::NS, Pp::PD, QM>), dim3(num_items), dim3(256), 0,
                     (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

// The query-rows-on-M orientation, for bf16 KV and per-token-head FP8 KV with bf16
// queries at head_dim 128 and 256, in the tile shapes listed by stage1_cfg_supported
// (bf16 KV at head_dim 256 with two query-block waves and at head_dim 128 with three
// blocks per wave would need more than 256 registers).
template <int DH, int KV>
static int dispatch_qm(const KernelCfg& c, const Stage1Args& a, int n, void* s) {
  constexpr bool PT = KV == 1;
  if constexpr (DH == 128) {
    if (c.wq == 1 && c.nqb == 1) return launch_one<DH, false, KV, PT, 1, 1, true>(a, n, s);
  }
  if constexpr (DH == 128 || PT) {
    if (c.wq == 2 && c.nqb == 1) return launch_one<DH, false, KV, PT, 2, 1, true>(a, n, s);
  }
  if (c.wq == 4 && c.nqb == 1) return launch_one<DH, false, KV, PT, 4, 1, true>(a, n, s);
  if constexpr (DH == 128) {
    if (c.wq == 4 && c.nqb == 2) return launch_one<DH, false, KV, PT, 4, 2, true>(a, n, s);
  }
  if constexpr (DH == 128 && PT) {
    if (c.wq == 4 && c.nqb == 3) return launch_one<DH, false, KV, PT, 4, 3, true>(a, n, s);
  }
  return (int)hipErrorInvalidValue;
}

// Largest query-block count per wave instantiated for a mode: per-tensor FP8 V keeps
// a second (lo) accumulator, which does not fit in registers for more blocks; at head_dim
// 256 a wave's accumulators for one block already take 64 registers, so more than four
// blocks per KV head run as query-block groups (one work item per run of four blocks).
template <int DH, int KV, bool PT>
constexpr int max_nqb() {
  constexpr bool pv_fp8 = KV == 1 && !PT;
  if constexpr (DH == 128) return pv_fp8 ? 2 : 3;
  else return 1;
}

template <int DH, bool QF8, int KV, bool PT>
static int dispatch_tiles(const KernelCfg& c, const Stage1Args& a, int n, void* s) {
  constexpr int NMAX = max_nqb<DH, KV, PT>();
  if constexpr (DH == 128) {      // d256 always runs >= 2 query-block waves (64-token tiles)
    if (c.wq == 1 && c.nqb == 1) return launch_one<DH, QF8, KV, PT, 1, 1>(a, n, s);
  }
  // (head_dim 256, bf16 queries against per-tensor FP8: the upconverted query operand,
  // two accumulator sets and a 64-token tile in flight exceed 256 registers with two
  // query-block waves, so such requests run on four one-block waves)
  if constexpr (!(DH == 256 && KV == 1 && !PT && !QF8)) {
    if (c.wq == 2 && c.nqb == 1) return launch_one<DH, QF8, KV, PT, 2, 1>(a, n, s);
  }
  if (c.wq == 4 && c.nqb == 1) return launch_one<DH, QF8, KV, PT, 4, 1>(a, n, s);
  if constexpr (NMAX >= 2) {
    if (c.wq == 4 && c.nqb == 2) return launch_one<DH, QF8, KV, PT, 4, 2>(a, n, s);
  }
  if constexpr (NMAX >= 3) {
    if (c.wq == 4 && c.nqb == 3) return launch_one<DH, QF8, KV, PT, 4, 3>(a, n, s);
  }
  return (int)hipErrorInvalidValue;
}

template <int DH>
static int dispatch_modes(const KernelCfg& c, const Stage1Args& a, int n, void* s) {
  if (c.qm) {
    if (c.qf8 || c.i8 || c.kvf8 != c.pt) return (int)hipErrorInvalidValue;
    return c.kvf8 ? dispatch_qm<DH, 1>(c, a, n, s) : dispatch_qm<DH, 0>(c, a, n, s);
  }
  if (c.i8) return !c.qf8 && c.pt ? dispatch_tiles<DH, false, 2, true>(c, a, n, s) : (int)hipErrorInvalidValue;
  if (!c.qf8 && !c.kvf8) return dispatch_tiles<DH, false, 0, false>(c, a, n, s);
  if (c.qf8 && c.kvf8 && !c.pt) return dispatch_tiles<DH, true, 1, false>(c, a, n, s);
  if (c.qf8 && c.kvf8 && c.pt) return dispatch_tiles<DH, true, 1, true>(c, a, n, s);
  if (!c.qf8 && c.kvf8 && !c.pt) return dispatch_tiles<DH, false, 1, false>(c, a, n, s);
  if (!c.qf8 && c.kvf8 && c.pt) return dispatch_tiles<DH, false, 1, true>(c, a, n, s);
  return (int)hipErrorInvalidValue;
}

int launch_stage1(const KernelCfg& c, const Stage1Args& a, int num_items, void* stream) {
  if (num_items <= 0) return 0;
  if (c.dh == 128) return dispatch_modes<128>(c, a, num_items, stream);
  if (c.dh == 256) return dispatch_modes<256>(c, a, num_items, stream);
  if (c.dh == 512 && stage1_cfg_supported(c)) {
    if (!c.kvf8) return launch_one<512, false, 0, false, 4, 1>(a, num_items, stream);
    return launch_one<512, false, 1, true, 4, 1>(a, num_items, stream);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace pa
