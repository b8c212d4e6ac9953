// Stage 1 for the latent cache of multi-head latent attention in its absorbed form (FlashMLA
// PR #54, review thread: the "nope" part in 8 bits with one scale per token and 128
// channels, the rotary part kept in 16 bits).  Keys are [latent (512), rotary (64)]: the
// latent as e4m3 codes with a float32 scale per (token, 128 channels), the rotary part a
// bf16 cache of its own; the value is the latent itself.  Queries: latent e4m3 with a scale
// per (row, head, 128 channels), rotary part bf16.
//
// One workgroup (4 waves) per work item (request, KV head, split, group of WQ = 1, 2 or 4
// 16-row query blocks); each block is run by a team of WT = 4 / WQ waves.  Tiles of 64
// tokens stream HBM -> registers -> LDS (wave w loads tokens 16 w .. 16 w + 15, one page).
//   QK (swapped, S^T = K Q^T, tokens on the MFMA M axis): a team's waves take the tile's
//     16-token units in turn; per unit, the latent part is one 16x16x128 e4m3 MFMA per
//     128-channel block over the raw codes (exact products, fp32 sums) scaled by the row's
//     and the token's scale of that block, plus two bf16 MFMAs over the rotary part.
//   softmax: log2 domain, per-row causal / window masks.  Each wave keeps its own running
//     maximum and sum over the units it scores, and writes p = 2^(s - m_wave) to LDS with
//     its m_wave.
//   PV: the team splits the 512 value channels (512 / WT per wave), so a wave holds 128 / WT
//     O^T accumulator registers (32 at one block per item) instead of 128.  For every
//     32-token step a wave rebuilds the P^T operand from LDS as
//     bf16(p * 2^(m_src - m_team) * latent_scale[token][block]) and multiplies it with the
//     transposed, exactly upconverted latent codes (ds_read_b64_tr_b8 + e4m3 -> bf16).
//   End: the team combines its waves' sums under the common maximum and writes O / l and
//     the LSE for its channel slices.
#include "common.hpp"
#include "fair_share.hpp"
#include "row_store.hpp"
#include "kv_addr.hpp"

namespace pa {

namespace {

typedef int i32x4m __attribute__((ext_vector_type(4)));
typedef int i32x8m __attribute__((ext_vector_type(8)));

constexpr float kLog2eM = 1.4426950408889634f;
constexpr float kLn2M = 0.6931471805599453f;

// 16x16x128 with e4m3 A and B (32 bytes per lane: A lane l holds row l%16, B lane l column
// l%16, both over the same 32 K positions of lane group l/16); no extra scaling.
__device__ __forceinline__ f32x4 mfma_e4m3_k128(i32x8m a, i32x8m b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

struct MlaCfg {
  static constexpr int DV = 512;                    // latent channels (= value width)
  static constexpr int DR = 64;                     // rotary channels
  static constexpr int NBLK = DV / 128;             // latent scale blocks
  static constexpr int BN = 64;                     // tokens per tile
  static constexpr int NU = BN / 16;                // 16-token units per tile (one per wave's load)
  static constexpr int KS = BN / 32;                // 32-token P.V steps per tile
  static constexpr int CPR_L = DV / 16;             // 16-byte chunks per latent row
  static constexpr int CPR_R = DR * 2 / 16;         // ... per rotary row
  // LDS rows are padded by 16 bytes: 16 consecutive tokens then start in 16 different
  // 16-byte bank groups, which keeps the row-wise reads of QK (16 tokens x one chunk) and
  // the transposing reads of P.V (8 tokens x one chunk) free of bank conflicts, while every
  // chunk of a row stays at a constant offset from the row (immediate offsets, no swizzle
  // arithmetic per read).
  static constexpr int LSTR = DV + 16;              // latent row stride in bytes
  static constexpr int RSTR = DR * 2 + 16;          // rotary row stride in bytes
  static constexpr int LAT = 0;                     // LDS: latent codes [BN][LSTR]
  static constexpr int ROPE = LAT + BN * LSTR;      //      rotary rows [BN][RSTR]
  static constexpr int SCL = ROPE + BN * RSTR;      //      latent scales [NBLK][BN]
  static constexpr int PST = BN + 4;                //      P row stride in floats (padding vs bank conflicts)
  static constexpr int PBUF = SCL + NBLK * BN * 4;  //      p [WQ][16][PST] fp32
  static constexpr int PBLK = 16 * PST * 4;
  template <int WQ> static constexpr int MX = PBUF + WQ * PBLK;   // per-wave row maxima [4][16]
  template <int WQ> static constexpr int FIN = MX<WQ> + 4 * 16 * 4; // end: (m, l) per wave [4][2][16]
  template <int WQ> static constexpr int BYTES = FIN<WQ> + 4 * 2 * 16 * 4;
};

template <int WQ>
__global__ __launch_bounds__(256, WQ == 4 ? 1 : 2) void stage1_mla_kernel(KrArgs a) {
  using C = MlaCfg;
  constexpr int WT = 4 / WQ;                 // waves per query block
  constexpr int CW = C::DV / WT;             // value channels per wave
  constexpr int DBW = CW / 16;               // 16-channel output blocks per wave
  constexpr int NBW = (CW + 127) / 128;      // latent scale blocks a wave's channels span
  constexpr int UPW = C::NU / WT;            // units a wave scores per tile (= WQ)
  static_assert(WQ == 1 || WQ == 2 || WQ == 4, "one, two or four query blocks per item");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::BYTES<WQ>];

  const PaItem it = a.items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int team = wave / WT;
  const int wave_in = wave % WT;
  const int L16 = lane & 15;
  const int g = lane >> 4;
  const int G = a.group;
  const int Mq = it.nrows * G;
  const int tb0 = it.tok_begin;
  const int te = it.tok_end;
  const int shift = a.page_shift;

  // ---- this team's query block: rows, limits, operands -----------------------------------
  const int qb = it.qblk0 + team;
  const bool has_rows = 16 * qb < Mq;
  const int m = 16 * qb + L16;
  const int mr = min(m, Mq - 1);                       // rows past Mq repeat the last real row
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
  const int64_t th = (int64_t)(it.row0 + r) * a.hq + (int64_t)it.kvh * G + hl;    // (row, query head)

  i32x8m qc[C::NBLK];                        // latent codes: 32 per lane and block (B operand)
  float qs[C::NBLK];
  bf16x8 qr[C::DR / 32];
  {
    const uint8_t* qp = static_cast<const uint8_t*>(a.q) + th * C::DV;
#pragma unroll
    for (int b = 0; b < C::NBLK; ++b) {
      const i32x4m c0 = *reinterpret_cast<const i32x4m*>(qp + 128 * b + 32 * g);
      const i32x4m c1 = *reinterpret_cast<const i32x4m*>(qp + 128 * b + 32 * g + 16);
      qc[b] = __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
      qs[b] = a.q_scale[th * C::NBLK + b];
    }
    const __bf16* qrp = static_cast<const __bf16*>(a.q_rope) + th * C::DR;
#pragma unroll
    for (int kc = 0; kc < C::DR / 32; ++kc) qr[kc] = *reinterpret_cast<const bf16x8*>(qrp + kc * 32 + 8 * g);
  }
  const float qk_scale = a.sm_scale * kLog2eM;

  f32x4 o[DBW];
#pragma unroll
  for (int d = 0; d < DBW; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_w = -INFINITY, l_w = 0.f;          // this wave's running max / sum over its units
  float m_team = -INFINITY;                  // the team's common maximum O is scaled to

  // ---- tile loads: wave w fetches tokens 16 w .. 16 w + 15 --------------------------------
  const LatentSpanLoads<C::DV> ld(lane, it.kvh, a.m_sp, a.m_sh, a.m_ss, a.r_sp, a.r_sh, a.r_ss, a.s_sp, a.s_sh,
                                  a.s_ss);
  using AL = LatentSpanLoads<C::DV>::AL;
  using AR = LatentSpanLoads<C::DV>::AR;
  static_assert(AL::NG == 8 && AR::NG == 2, "16 tokens per wave");
  const AL& al = ld.al;
  const AR& ar = ld.ar;
  const cint32* pidx = (const cint32*)(a.page_indices) + it.page_base;
  const uint8_t* lbase = static_cast<const uint8_t*>(a.k_main);
  const uint8_t* rbase = static_cast<const uint8_t*>(a.k_rope);
  u32x4 lreg[AL::NG], rreg[AR::NG];
  float sreg;
  // (spans wholly before the split's end take one page and no clamp; see LatentSpanLoads)
  auto load_tile = [&](int tile0) __attribute__((always_inline)) {
    ld.tile(pidx, tile0 + 16 * wave, te, shift,
            [&](auto part, int i, int64_t off, int, int) __attribute__((always_inline)) {
              constexpr int PART = decltype(part)::value;
              if constexpr (PART == 0) lreg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(lbase + off));
              else if constexpr (PART == 1) rreg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rbase + off));
              else sreg = __builtin_nontemporal_load(a.k_scale + off);
            });
  };
  // LDS: chunk c of token t sits at byte t * stride + 16 c.
  auto store_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < AL::NG; ++i) {
      const int t = 16 * wave + AL::GT * i + al.lt;
      *reinterpret_cast<u32x4*>(smem + C::LAT + t * C::LSTR + 16 * al.cpos) = lreg[i];
    }
#pragma unroll
    for (int i = 0; i < AR::NG; ++i) {
      const int t = 16 * wave + AR::GT * i + ar.lt;
      *reinterpret_cast<u32x4*>(smem + C::ROPE + t * C::RSTR + 16 * ar.cpos) = rreg[i];
    }
    reinterpret_cast<float*>(smem + C::SCL)[(lane & 3) * C::BN + 16 * wave + (lane >> 2)] = sreg;
  };

  const float* scl = reinterpret_cast<const float*>(smem + C::SCL);
  float* pbuf = reinterpret_cast<float*>(smem + C::PBUF) + team * (16 * C::PST);
  float* mx = reinterpret_cast<float*>(smem + C::MX<WQ>);

  // ---- scores of this wave's units, softmax against the wave's own maximum, p -> LDS ------
  auto score_tile = [&](int tile0) __attribute__((always_inline)) {
    float x[UPW][4];
#pragma unroll
    for (int k = 0; k < UPW; ++k) {
      const int u = wave_in + WT * k;
      const int t = 16 * u + L16;            // K row (token) of this lane in the tile
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < C::DR / 32; ++kc) {
        const bf16x8 kv = *reinterpret_cast<const bf16x8*>(smem + C::ROPE + t * C::RSTR + 16 * (4 * kc + g));
        acc = mfma_bf16(kv, qr[kc], acc);
      }
#pragma unroll
      for (int b = 0; b < C::NBLK; ++b) {
        const uint8_t* kr = smem + C::LAT + t * C::LSTR + 16 * (8 * b + 2 * g);
        const i32x4m k0 = *reinterpret_cast<const i32x4m*>(kr);
        const i32x4m k1 = *reinterpret_cast<const i32x4m*>(kr + 16);
        const f32x4 sb = mfma_e4m3_k128(__builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7), qc[b],
                                        f32x4{0.f, 0.f, 0.f, 0.f});
        // accumulator rows are tokens 16 u + 4 g + k: their scales of block b
        const f32x4 ks = *reinterpret_cast<const f32x4*>(scl + b * C::BN + 16 * u + 4 * g);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc[kk] = fmaf(sb[kk], qs[b] * ks[kk], acc[kk]);
      }
      const int c0 = tile0 + 16 * u;
      const bool need_mask = !(c0 >= vis_lo_all && c0 + 15 <= vis_hi_all);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        float v = acc[kk] * qk_scale;
        if (need_mask) {
          const int j = c0 + 4 * g + kk;
          v = (j >= lim_lo && j <= lim_hi) ? v : -INFINITY;
        }
        x[k][kk] = v;
      }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int k = 0; k < UPW; ++k)
      mt = fmaxf(mt, fmaxf(fmaxf(x[k][0], x[k][1]), fmaxf(x[k][2], x[k][3])));
    mt = wave_max_xor_16_32(mt);
    const float mnew = fmaxf(m_w, mt);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    l_w *= fast_exp2(m_w - muse);            // (0 * 0 while everything so far is masked)
    m_w = mnew;
#pragma unroll
    for (int k = 0; k < UPW; ++k) {
      f32x4 pv;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        pv[kk] = fast_exp2(x[k][kk] - muse);
        l_w += pv[kk];
      }
      *reinterpret_cast<f32x4*>(pbuf + L16 * C::PST + 16 * (wave_in + WT * k) + 4 * g) = pv;
    }
    if (g == 0) mx[wave * 16 + L16] = m_w;
  };

  // ---- O^T += V^T P^T over the tile for this wave's channels ------------------------------
  auto pv_tile = [&]() __attribute__((always_inline)) {
    float msrc[WT];
    float mt = m_team;
#pragma unroll
    for (int w2 = 0; w2 < WT; ++w2) {
      msrc[w2] = mx[(team * WT + w2) * 16 + L16];
      mt = fmaxf(mt, msrc[w2]);
    }
    const float muse = mt == -INFINITY ? 0.f : mt;
    if (__builtin_amdgcn_ballot_w64(mt != m_team) != 0) {
      const float alpha = fast_exp2(m_team - muse);
#pragma unroll
      for (int d = 0; d < DBW; ++d) o[d] *= alpha;
      m_team = mt;
    }
    float f[WT];                             // 2^(m_src - m_team) per source wave
#pragma unroll
    for (int w2 = 0; w2 < WT; ++w2) f[w2] = fast_exp2(msrc[w2] - muse);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      // lane group g holds tokens 32 ks + 8 g .. + 7 (K positions 8 g .. 8 g + 7)
      const int tok = 32 * ks + 8 * g;
      const int src = (tok >> 4) % WT;       // the team wave that scored this unit
      float fs = f[0];
#pragma unroll
      for (int w2 = 1; w2 < WT; ++w2) fs = src == w2 ? f[w2] : fs;
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(pbuf + L16 * C::PST + tok);
      const f32x4 p1 = *reinterpret_cast<const f32x4*>(pbuf + L16 * C::PST + tok + 4);
      const int tv = tok + (L16 >> 1);       // token row this lane addresses for the transposing read
#pragma unroll
      for (int bb = 0; bb < NBW; ++bb) {
        const int b = (wave_in * CW) / 128 + bb;
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(scl + b * C::BN + tok);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(scl + b * C::BN + tok + 4);
        bf16x8 pb;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          pb[kk] = (__bf16)(p0[kk] * fs * s0[kk]);
          pb[4 + kk] = (__bf16)(p1[kk] * fs * s1[kk]);
        }
        constexpr int DPB = CW < 128 ? CW / 16 : 8;   // output blocks of this scale block
#pragma unroll
        for (int dd = 0; dd < DPB; ++dd) {
          const int db = (wave_in * CW) / 16 + 8 * bb + dd;   // global 16-channel block
          const uint32_t addr = tv * C::LSTR + 16 * db + 8 * (L16 & 1);
          const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((PA_LDS i32x2*)(smem + C::LAT + addr));
          o[8 * bb + dd] = mfma_bf16(fp8x8_to_bf16x8((uint32_t)w[0], (uint32_t)w[1]), pb, o[8 * bb + dd]);
        }
      }
    }
  };

  const int ntiles = te > tb0 ? (te - tb0 + C::BN - 1) / C::BN : 0;
  if (ntiles > 0) {
    load_tile(tb0);
    store_tile();
    __syncthreads();
  }
  // issue-priority balance within the CU (not for one block per item: measured 3% slower)
  const FairShare fs(WQ > 1 && a.fair != 0, ntiles);
  for (int ti = 0; ti < ntiles; ++ti) {
    fs.at(ti);
    const int tile0 = tb0 + ti * C::BN;
    const bool more = ti + 1 < ntiles;
    if (more) load_tile(tile0 + C::BN);      // next tile in flight during this one
    if (has_rows) score_tile(tile0);
    __syncthreads();                         // p and the maxima of every wave are in LDS
    if (has_rows) pv_tile();
    __syncthreads();                         // every wave is done with this tile's LDS
    if (more) {
      store_tile();
      __syncthreads();
    }
  }

  // ---- end: the team's sums under its common maximum, O / l, LSE ---------------------------
  const float lsum_w = wave_sum_xor_16_32(l_w);
  float* fin = reinterpret_cast<float*>(smem + C::FIN<WQ>);
  if (g == 0) {
    fin[(wave * 2) * 16 + L16] = m_w;
    fin[(wave * 2 + 1) * 16 + L16] = lsum_w;
  }
  __syncthreads();
  if (!has_rows || m >= Mq) return;
  float mall = -INFINITY;
#pragma unroll
  for (int w2 = 0; w2 < WT; ++w2) mall = fmaxf(mall, fin[((team * WT + w2) * 2) * 16 + L16]);
  const float mu = mall == -INFINITY ? 0.f : mall;
  float lsum = 0.f;
#pragma unroll
  for (int w2 = 0; w2 < WT; ++w2)
    lsum += fin[((team * WT + w2) * 2 + 1) * 16 + L16] * fast_exp2(fin[((team * WT + w2) * 2) * 16 + L16] - mu);
  // O was scaled to m_team, which equals mall once the last tile is in
  const bool empty = !(lsum > 0.f);
  const float sc = empty ? 0.f : 1.f / lsum;
  const float lse = empty ? -INFINITY : (mall + __log2f(lsum)) * kLn2M;
  const int ch0 = wave_in * CW;
  const bool final_out = it.nsplit == 1;
  if (g == 0 && wave_in == 0) {
    if (final_out) {
      if (a.out_lse) a.out_lse[th] = lse;
    } else {
      a.partial_lse[th * a.s_max + it.split] = lse;
    }
  }
  void* dstv = final_out ? a.out : a.partial_o;
  const int64_t row = final_out ? th : th * a.s_max + it.split;
  const bool bf = final_out ? a.out_bf16 : a.part_bf16;
  if (bf) {
    store_row_bf16_x16(static_cast<__bf16*>(dstv) + row * C::DV + ch0, o, sc, g);
  } else {
    float* dst = static_cast<float*>(dstv) + row * C::DV + ch0;
#pragma unroll
    for (int d = 0; d < DBW; ++d) *reinterpret_cast<f32x4*>(dst + 16 * d + 4 * g) = o[d] * sc;
  }
}

}  // namespace

int launch_stage1_mla(int wq, const KrArgs& a, int num_items, void* stream) {
  if (num_items <= 0) return 0;
  const hipStream_t s = (hipStream_t)stream;
  const dim3 grid(num_items), block(256);
  if (wq == 1) hipLaunchKernelGGL(stage1_mla_kernel<1>, grid, block, 0, s, a);
  else if (wq == 2) hipLaunchKernelGGL(stage1_mla_kernel<2>, grid, block, 0, s, a);
  else if (wq == 4) hipLaunchKernelGGL(stage1_mla_kernel<4>, grid, block, 0, s, a);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

}  // namespace pa
