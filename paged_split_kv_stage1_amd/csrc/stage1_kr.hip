// Stage 1 for keys wider than values: bf16 K rows of DV + 64 channels (a 64-channel rotary
// part after DV channels) in one cache and bf16 V rows of DV channels in another
// (head_dim_qk 192, head_dim_v 128; FlashInfer PR #869, "Remaining Work": separate
// head_dim_qk and head_dim_v).  The latent cache of multi-head latent attention, whose keys
// are also wider than its values, has a kernel of its own (stage1_mla.hip).
//
// One workgroup (4 waves) per work item (request, KV head, split, group of one, two or four
// 16-row query blocks): the waves split the tokens of each 128-token tile between them as
// far as the blocks leave waves free, and combine their (max, sum, O) at the end.  Scores
// are computed transposed, S^T = K Q^T (tokens on the MFMA M axis), so that their
// accumulator is the P^T operand of O^T = V^T P^T, as in the main stage-1 kernel.  K/V
// tiles stream HBM -> registers -> LDS (one stage, the next tile's loads in flight in
// registers) with the page-gather address code of kv_addr.hpp.
//   QK: bf16 MFMA 16x16x32 over the DV main channels and the rotary channels.
//   softmax: log2 domain, per-row causal / window masks, lazy rescale.
//   PV: P as two bf16 terms (hi + lo) against bf16 V.
#include "common.hpp"
#include "fair_share.hpp"
#include "kv_addr.hpp"

namespace pa {

namespace {

constexpr float kLog2eKr = 1.4426950408889634f;
constexpr float kLn2Kr = 0.6931471805599453f;

// XOR swizzle of the 16-byte chunk index within a token row in LDS (row-wise reads of 16
// tokens x one chunk, and transposing reads of 4 or 8 tokens x one chunk, spread over banks).
template <int CPR>
__device__ __forceinline__ int swz(int t) {
  if constexpr (CPR >= 16) return t & 15;
  else return (t >> 1) & (CPR - 1);
}

template <int DV>
struct KrCfg {
  static constexpr int BN = 128;                      // tokens per tile: four 32-token quarters
  static constexpr int DR = 64;                       // rotary channels
  static constexpr int CPR_M = DV * 2 / 16;           // 16-byte chunks per main-part row
  static constexpr int CPR_R = DR * 2 / 16;           // ... per rotary row
  static constexpr int CPR_V = DV * 2 / 16;           // ... per value row
  static constexpr int CPT_M = BN * CPR_M / 256;      // chunks per thread per tile
  static constexpr int CPT_R = BN * CPR_R / 256;
  static constexpr int CPT_V = BN * CPR_V / 256;
  static constexpr int MTB = BN * DV * 2;             // LDS bytes of the main tile
  static constexpr int RTB = BN * DR * 2;
  static constexpr int VTB = BN * DV * 2;
  static constexpr int STAGEB = MTB + RTB + VTB;
  static constexpr int KCM = DV / 32;                 // K-steps of q.k over the main part
  static constexpr int KCR = DR / 32;                 // ... over the rotary part
  static constexpr int DB = DV / 16;                  // 16-wide output blocks
  static constexpr int OWB = 64 * 4 * DB * 4;         // bytes of one wave's O in the combine
  static_assert(CPT_M >= 1 && CPT_R >= 1 && CPT_V >= 1, "tile must split over 256 threads");
};

// One work item is (request, KV head, split, group of WQ 16-row query blocks).  The four
// waves form WQ teams of WT = 4 / WQ waves, one team per block; the WT waves of a team
// take every WT-th 32-token quarter of each 128-token tile, keep their own (max, sum, O)
// and combine them through LDS at the end.  A tile is loaded once for all blocks.
template <int DV, int WQ>
__global__ __launch_bounds__(256, 2) void stage1_kr_kernel(KrArgs a) {
  using C = KrCfg<DV>;
  constexpr int WT = 4 / WQ;
  static_assert(WQ == 1 || WQ == 2 || WQ == 4, "one, two or four query blocks per item");
  static_assert(WT == 1 || C::STAGEB >= WQ * (C::OWB + 2 * 64 * 4), "the combine reuses the tile's LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::STAGEB];

  const PaItem it = a.items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int L16 = lane & 15;
  const int g = lane >> 4;
  const int G = a.group;
  const int Hq = a.hq;
  const int Mq = it.nrows * G;
  const int tb0 = it.tok_begin;
  const int te = it.tok_end;
  const int shift = a.page_shift;
  const int team = wave / WT;                          // the query block this wave works on
  const int wave_in = wave % WT;                       // its place among the team's waves

  // ---- this team's query block: rows, limits, operand ------------------------------------
  const int qb = it.qblk0 + team;
  const bool has_rows = 16 * qb < Mq;
  const int m = 16 * qb + L16;
  const int mr = m < Mq ? m : Mq - 1;                  // rows past Mq repeat the last real row
  const int r = mr / G;
  const int hl = mr - r * G;
  const int p = it.kv_len - it.nrows + r;
  const int lo = it.window > 0 ? max(0, p - it.window + 1) : 0;
  const int lim_lo = max(lo, tb0);
  const int lim_hi = min(p, te - 1);
  const int p_first = it.kv_len - it.nrows;
  const int lo_last = it.window > 0 ? max(0, it.kv_len - 1 - it.window + 1) : 0;
  const int vis_lo_all = max(lo_last, tb0);
  const int vis_hi_all = min(p_first, te - 1);
  const int64_t th = (int64_t)(it.row0 + r) * Hq + (int64_t)it.kvh * G + hl;    // (row, query head)

  bf16x8 qm[C::KCM], qr[C::KCR];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + th * (DV + C::DR);
#pragma unroll
    for (int kc = 0; kc < C::KCM; ++kc) qm[kc] = *reinterpret_cast<const bf16x8*>(qp + kc * 32 + 8 * g);
#pragma unroll
    for (int kc = 0; kc < C::KCR; ++kc) qr[kc] = *reinterpret_cast<const bf16x8*>(qp + DV + kc * 32 + 8 * g);
  }
  const float qk_scale = a.sm_scale * kLog2eKr;

  f32x4 o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;

  // ---- tile loads: HBM -> registers -> LDS -------------------------------------------------
  // Wave w loads quarter w of every tile (tokens 32 w .. 32 w + 31): main, rotary and
  // value rows.
  const RopeQuarterLoads<DV> ld(lane, it.kvh, a.m_sp, a.m_sh, a.m_ss, a.r_sp, a.r_sh, a.r_ss, a.v_sp, a.v_sh,
                                a.v_ss);
  using LD = RopeQuarterLoads<DV>;
  const typename LD::AM& am = ld.am;
  const typename LD::AR& ar = ld.ar;
  const typename LD::AV& av = ld.av;
  using AM = typename LD::AM;
  using AR = typename LD::AR;
  using AV = typename LD::AV;
  const cint32* pidx = (const cint32*)(a.page_indices) + it.page_base;
  const uint8_t* mbase = static_cast<const uint8_t*>(a.k_main);
  const uint8_t* rbase = static_cast<const uint8_t*>(a.k_rope);
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v);
  static_assert(C::CPT_M == AM::NG && C::CPT_R == AR::NG && C::CPT_V == AV::NG, "one quarter per wave");
  u32x4 mreg[C::CPT_M], rreg[C::CPT_R], vreg[C::CPT_V];
  auto load_tile = [&](int tile0) __attribute__((always_inline)) {
    ld.tile(pidx, tile0 + 32 * wave, te, shift,
            [&](auto part, int i, int64_t off, int, int) __attribute__((always_inline)) {
              constexpr int PART = decltype(part)::value;
              if constexpr (PART == 0) mreg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(mbase + off));
              else if constexpr (PART == 1) rreg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rbase + off));
              else vreg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + off));
            });
  };
  // LDS: chunk c of token t of a tile sits at 16-byte unit t * CPR + (c ^ swz(t)).
  auto store_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < AM::NG; ++i) {
      const int t = 32 * wave + AM::GT * i + am.lt;
      *reinterpret_cast<u32x4*>(smem + ((t * C::CPR_M + (am.cpos ^ swz<C::CPR_M>(t))) << 4)) = mreg[i];
    }
#pragma unroll
    for (int i = 0; i < AR::NG; ++i) {
      const int t = 32 * wave + AR::GT * i + ar.lt;
      *reinterpret_cast<u32x4*>(smem + C::MTB + ((t * C::CPR_R + (ar.cpos ^ swz<C::CPR_R>(t))) << 4)) = rreg[i];
    }
#pragma unroll
    for (int i = 0; i < AV::NG; ++i) {
      const int t = 32 * wave + AV::GT * i + av.lt;
      *reinterpret_cast<u32x4*>(smem + C::MTB + C::RTB + ((t * C::CPR_V + (av.cpos ^ swz<C::CPR_V>(t))) << 4)) = vreg[i];
    }
  };

  // ---- 32 tokens of a tile (from wt0 on): S^T, softmax, O^T += V^T P^T ------------------
  auto compute_quarter = [&](int tile0, int wt0) __attribute__((always_inline)) {
    const int c0 = tile0 + wt0;
    if (c0 >= te) return;
    const uint8_t* Ml = smem;
    const uint8_t* Rl = smem + C::MTB;
    float x[8];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int t = wt0 + 16 * tb + L16;               // K row (token) of this lane in the tile
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < C::KCR; ++kc) {
        const bf16x8 kv = *reinterpret_cast<const bf16x8*>(Rl + ((t * C::CPR_R + ((4 * kc + g) ^ swz<C::CPR_R>(t))) << 4));
        acc = mfma_bf16(kv, qr[kc], acc);
      }
#pragma unroll
      for (int kc = 0; kc < C::KCM; ++kc) {
        const bf16x8 kv = *reinterpret_cast<const bf16x8*>(Ml + ((t * C::CPR_M + ((4 * kc + g) ^ swz<C::CPR_M>(t))) << 4));
        acc = mfma_bf16(kv, qm[kc], acc);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) x[4 * tb + k] = acc[k];
    }
    // ---- scale, mask, online softmax
    const bool need_mask = !(c0 >= vis_lo_all && c0 + 31 <= vis_hi_all);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x[k] *= qk_scale;
      if (need_mask) {
        const int j = c0 + (k < 4 ? 4 * g + k : 16 + 4 * g + (k - 4));
        x[k] = (j >= lim_lo && j <= lim_hi) ? x[k] : -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mx = wave_max_xor_16_32(mx);
    const float mnew = fmaxf(mrun, mx);
    const float muse = (mnew == -INFINITY) ? 0.f : mnew;
    if (__builtin_amdgcn_ballot_w64(mnew != mrun) != 0) {
      const float alpha = fast_exp2(mrun - muse);
      lrun *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
      mrun = mnew;
    }
    float pv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      pv[k] = fast_exp2(x[k] - muse);
      lrun += pv[k];
    }
    // ---- O^T += V^T P^T
    const uint8_t* Vl = smem + C::MTB + C::RTB;
    bf16x8 hv, lv;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const __bf16 h = (__bf16)pv[k];
      hv[k] = h;
      lv[k] = (__bf16)(pv[k] - (float)h);
    }
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      bf16x8 va;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int t1 = wt0 + 4 * g + (L16 >> 2) + 16 * half;
        const int c = 2 * db + ((L16 & 3) >> 1);
        const uint32_t addr = ((t1 * C::CPR_V + (c ^ swz<C::CPR_V>(t1))) << 4) + 8 * (L16 & 1);
        const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4*)(Vl + addr));
        const __bf16* pvv = reinterpret_cast<const __bf16*>(&v);
#pragma unroll
        for (int k = 0; k < 4; ++k) va[4 * half + k] = pvv[k];
      }
      o[db] = mfma_bf16(va, hv, o[db]);
      o[db] = mfma_bf16(va, lv, o[db]);
    }
  };
  auto compute_tile = [&](int tile0) __attribute__((always_inline)) {
    if (!has_rows) return;
#pragma unroll
    for (int k = 0; k < WQ; ++k) compute_quarter(tile0, 32 * (wave_in + WT * k));
  };

  // One LDS stage: the next tile's loads are in flight in registers while this one is
  // computed, and are stored once every wave is done reading the stage.
  const int ntiles = te > tb0 ? (te - tb0 + C::BN - 1) / C::BN : 0;
  if (ntiles > 0) {
    load_tile(tb0);
    __builtin_amdgcn_s_waitcnt(0xC07F & ~0xC00F);      // vmcnt(0) lgkmcnt(0)
    store_tile();
    __syncthreads();
  }
  const FairShare fs(a.fair != 0, ntiles);     // issue-priority balance within the CU
  for (int ti = 0; ti < ntiles; ++ti) {
    fs.at(ti);
    const int tile0 = tb0 + ti * C::BN;
    const bool more = ti + 1 < ntiles;
    if (more) load_tile(tile0 + C::BN);
    compute_tile(tile0);
    __syncthreads();
    if (more) {
      store_tile();
      __syncthreads();
    }
  }

  // ---- combine each team's (max, sum, O) through LDS, one wave at a time -------------------
  const float ltot = wave_sum_xor_16_32(lrun);
  float* eo = reinterpret_cast<float*>(smem + team * (C::OWB + 2 * 64 * 4));
  float* em = eo + 64 * 4 * C::DB;
  float* el = em + 64;
  float mall = mrun, lsum = ltot;
  for (int w2 = 1; w2 < WT; ++w2) {
    if (wave_in == w2) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db) *reinterpret_cast<f32x4*>(eo + (db * 64 + lane) * 4) = o[db];
      em[lane] = mrun;
      el[lane] = ltot;
    }
    __syncthreads();
    if (wave_in == 0) {
      const float m2 = em[lane];
      const float mn = fmaxf(mall, m2);
      const float mu = (mn == -INFINITY) ? 0.f : mn;
      const float f0 = fast_exp2(mall - mu), f2 = fast_exp2(m2 - mu);
      lsum = lsum * f0 + el[lane] * f2;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) o[db] = o[db] * f0 + *reinterpret_cast<const f32x4*>(eo + (db * 64 + lane) * 4) * f2;
      mall = mn;
    }
    __syncthreads();
  }

  // ---- epilogue (the first wave of each team) ------------------------------------------------
  if (wave_in != 0 || !has_rows || m >= Mq) return;
  const bool empty = !(lsum > 0.f);
  const float sc = empty ? 0.f : 1.f / lsum;
  const float lse = empty ? -INFINITY : (mall + __log2f(lsum)) * kLn2Kr;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  if (it.nsplit == 1) {
    if (a.out_lse && g == 0) a.out_lse[th] = lse;
    if (a.out_bf16) {
      __bf16* dst = static_cast<__bf16*>(a.out) + th * DV;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        bf16x4 v;
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = (__bf16)(o[db][k] * sc);
        *reinterpret_cast<bf16x4*>(dst + 16 * db + 4 * g) = v;
      }
    } else {
      float* dst = static_cast<float*>(a.out) + th * DV;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * g) = o[db] * sc;
    }
  } else {
    if (g == 0) a.partial_lse[th * a.s_max + it.split] = lse;
    if (a.part_bf16) {
      __bf16* dst = static_cast<__bf16*>(a.partial_o) + (th * a.s_max + it.split) * DV;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        bf16x4 v;
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = (__bf16)(o[db][k] * sc);
        *reinterpret_cast<bf16x4*>(dst + 16 * db + 4 * g) = v;
      }
    } else {
      float* dst = static_cast<float*>(a.partial_o) + (th * a.s_max + it.split) * DV;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * g) = o[db] * sc;
    }
  }
}

}  // namespace

int launch_stage1_kr(int dv, int wq, const KrArgs& a, int num_items, void* stream) {
  if (num_items <= 0) return 0;
  const hipStream_t s = (hipStream_t)stream;
  const dim3 grid(num_items), block(256);
  if (dv != 128) return (int)hipErrorInvalidValue;
  if (wq == 1) hipLaunchKernelGGL((stage1_kr_kernel<128, 1>), grid, block, 0, s, a);
  else if (wq == 2) hipLaunchKernelGGL((stage1_kr_kernel<128, 2>), grid, block, 0, s, a);
  else if (wq == 4) hipLaunchKernelGGL((stage1_kr_kernel<128, 4>), grid, block, 0, s, a);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

}  // namespace pa
