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
// Per tile, each wave owns 32 tokens x (its query blocks):
//   QK:  bf16 MFMA 16x16x32 (bf16 Q; FP8 K upconverted exactly), or fp8 MFMA
//        16x16x32 when Q is FP8 (exact products);
//   softmax: scores scaled into the log2 domain with the dequant scales folded in
//        (FlashInfer PR #869 item 3), per-row causal/window masks, online max/sum;
//   PV:  bf16 KV -> P split in two bf16 terms (hi + lo); per-token-head FP8 V ->
//        v_scale folded into P, V upconverted, two bf16 terms; per-tensor FP8 V ->
//        P requantised to e4m3 after scaling by the format maximum 448 (FlashInfer
//        PR #869 item 2), as a hi term plus a lo term of the residual x16, with the
//        per-tensor v_scale / 448 applied in the final normaliser.
// Waves that split the tokens of a tile merge their (max, sum, O) in LDS at the end.
#include "common.hpp"

namespace pa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int DH, bool QF8, bool KVF8, bool PT, int WQ, int NQB>
struct S1Cfg {
  static constexpr int WT = 4 / WQ;                 // waves splitting the tokens of a tile
  static constexpr int BN = 32 * WT;                // tokens per tile
  static constexpr int KVB = KVF8 ? 1 : 2;          // bytes per cached element
  static constexpr int ROWB = DH * KVB + 32;        // padded LDS row stride (bytes)
  static constexpr int TILEB = BN * ROWB;
  static constexpr int CPR = DH * KVB / 16;         // 16-byte chunks per token row
  static constexpr int CPT = BN * CPR / 256;        // chunks per thread per tile (K or V)
  static constexpr int KC = DH / 32;                // K-steps of q.k
  static constexpr int DB = DH / 16;                // 16-wide d blocks of P.V
  static constexpr bool PV_FP8 = KVF8 && !PT;       // per-tensor FP8 V: fp8 MFMA for P.V
  static constexpr int SCALEB = PT ? 2 * BN * 4 : 0;
  static constexpr int MAINB = 2 * TILEB + SCALEB;
  static constexpr int EPIB = (WT > 1) ? (4 * NQB * DB * 256 * 4 + 4 * NQB * 64 * 2 * 4) : 0;
  static constexpr int LDSB = MAINB > EPIB ? MAINB : EPIB;
  static_assert(CPT >= 1, "tile too small for 256 threads");
  static_assert(WT == 1 || NQB == 1, "query blocks per wave > 1 only without token split");
};

template <bool QF8>
struct QOperand;
template <>
struct QOperand<false> { using T = bf16x8; };
template <>
struct QOperand<true> { using T = long; };

template <int DH, bool QF8, bool KVF8, bool PT, int WQ, int NQB>
__global__ __launch_bounds__(256) void stage1_kernel(Stage1Args a) {
  using C = S1Cfg<DH, QF8, KVF8, PT, WQ, NQB>;
  using QT = typename QOperand<QF8>::T;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDSB];
  uint8_t* Kl = smem;
  uint8_t* Vl = smem + C::TILEB;
  float* ksl = reinterpret_cast<float*>(smem + 2 * C::TILEB);
  float* vsl = ksl + C::BN;

  const PaItem it = a.items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wq = wave % WQ;
  const int wt = wave / WQ;
  const int L16 = lane & 15;
  const int g = lane >> 4;
  const int G = a.group;
  const int Hq = a.hq;
  const int Mq = it.nrows * G;
  const int tb0 = it.tok_begin;
  const int te = it.tok_end;

  // ---- query operand, per-row limits ------------------------------------------
  QT qop[NQB][C::KC];
  int lim_lo[NQB], lim_hi[NQB];
  bool qvalid[NQB];
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    const int qb = wq + WQ * i;
    qvalid[i] = 16 * qb < Mq;
    const int m = 16 * qb + L16;
    const int mr = m < Mq ? m : Mq - 1;
    const int r = mr / G;
    const int hl = mr - r * G;
    const int p = it.kv_len - it.nrows + r;
    const int lo = it.window > 0 ? max(0, p - it.window + 1) : 0;
    lim_lo[i] = max(lo, tb0);
    lim_hi[i] = min(p, te - 1);
    const int64_t qrow = ((int64_t)(it.row0 + r) * Hq + (int64_t)it.kvh * G + hl) * DH;
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      if constexpr (QF8) {
        long v = 0;
        if (m < Mq) v = *reinterpret_cast<const long*>(static_cast<const uint8_t*>(a.q) + qrow + kc * 32 + 8 * g);
        qop[i][kc] = v;
      } else {
        bf16x8 v = {};
        if (m < Mq)
          v = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.q) + qrow + kc * 32 + 8 * g);
        qop[i][kc] = v;
      }
    }
  }
  // Tokens every real row of the item sees (fast path: no masking inside).
  const int p_first = it.kv_len - it.nrows;
  const int lo_last = it.window > 0 ? max(0, it.kv_len - 1 - it.window + 1) : 0;
  const int vis_lo_all = max(lo_last, tb0);
  const int vis_hi_all = min(p_first, te - 1);

  float qk_scale = a.sm_scale * kLog2e;
  if constexpr (QF8) qk_scale *= *a.q_scale;
  if constexpr (KVF8 && !PT) qk_scale *= *a.k_scale;
  float out_scale = 1.0f;
  if constexpr (C::PV_FP8) out_scale = *a.v_scale * (1.0f / 448.0f);

  f32x4 o[NQB][C::DB];
  f32x4 olo[C::PV_FP8 ? NQB : 1][C::PV_FP8 ? C::DB : 1];
  float mrun[NQB], lrun[NQB];
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    mrun[i] = -INFINITY;
    lrun[i] = 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[i][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (C::PV_FP8) {
#pragma unroll
    for (int i = 0; i < NQB; ++i)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) olo[i][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- tile staging ----------------------------------------------------------------
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k);
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v);
  uint4 kst[C::CPT], vst[C::CPT];
  float ksc = 0.f, vsc = 0.f;
  auto load_tile = [&](int tile0) {
#pragma unroll
    for (int c = 0; c < C::CPT; ++c) {
      const int chunk = tid + 256 * c;
      const int tok = chunk / C::CPR;
      const int col = chunk % C::CPR;
      const int j = tile0 + tok;
      if (j < te) {
        const int32_t pg = token_page(a.page_indices, it.page_base, j, a.page_shift);
        const int32_t sl = token_slot(j, a.page_shift);
        const int64_t off = ((int64_t)pg * a.kv_sp + (int64_t)it.kvh * a.kv_sh + (int64_t)sl * a.kv_ss) * C::KVB + col * 16;
        kst[c] = *reinterpret_cast<const uint4*>(kbase + off);
        vst[c] = *reinterpret_cast<const uint4*>(vbase + off);
      } else {
        kst[c] = uint4{0u, 0u, 0u, 0u};
        vst[c] = uint4{0u, 0u, 0u, 0u};
      }
    }
    if constexpr (PT) {
      if (tid < C::BN) {
        const int j = tile0 + tid;
        if (j < te) {
          const int32_t pg = token_page(a.page_indices, it.page_base, j, a.page_shift);
          const int32_t sl = token_slot(j, a.page_shift);
          const int64_t so = (int64_t)pg * a.sc_sp + (int64_t)it.kvh * a.sc_sh + (int64_t)sl * a.sc_ss;
          ksc = a.k_scale[so];
          vsc = a.v_scale[so];
        } else {
          ksc = 0.f;
          vsc = 0.f;
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int c = 0; c < C::CPT; ++c) {
      const int chunk = tid + 256 * c;
      const int tok = chunk / C::CPR;
      const int col = chunk % C::CPR;
      *reinterpret_cast<uint4*>(Kl + tok * C::ROWB + col * 16) = kst[c];
      *reinterpret_cast<uint4*>(Vl + tok * C::ROWB + col * 16) = vst[c];
    }
    if constexpr (PT) {
      if (tid < C::BN) {
        ksl[tid] = ksc;
        vsl[tid] = vsc;
      }
    }
  };

  const int ntiles = te > tb0 ? (te - tb0 + C::BN - 1) / C::BN : 0;
  if (ntiles > 0) load_tile(tb0);

  for (int ti = 0; ti < ntiles; ++ti) {
    const int tile0 = tb0 + ti * C::BN;
    store_tile();
    __syncthreads();
    if (ti + 1 < ntiles) load_tile(tile0 + C::BN);

    const int c0 = tile0 + wt * 32;          // first token of this wave's 32-token chunk
    if (c0 < te) {
      // ---- S^T = K Q^T for 2 x 16 tokens ------------------------------------------
      f32x4 s[NQB][2];
#pragma unroll
      for (int i = 0; i < NQB; ++i) s[i][0] = s[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const uint8_t* krow = Kl + (wt * 32 + tb * 16 + L16) * C::ROWB;
#pragma unroll
        for (int kc = 0; kc < C::KC; ++kc) {
          if constexpr (!KVF8) {
            const bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + (kc * 32 + 8 * g) * 2);
#pragma unroll
            for (int i = 0; i < NQB; ++i)
              if (qvalid[i]) s[i][tb] = mfma_bf16(ka, qop[i][kc], s[i][tb]);
          } else {
            const uint2 raw = *reinterpret_cast<const uint2*>(krow + kc * 32 + 8 * g);
            if constexpr (QF8) {
              const long ka = (long)raw.x | ((long)raw.y << 32);
#pragma unroll
              for (int i = 0; i < NQB; ++i)
                if (qvalid[i]) s[i][tb] = mfma_fp8(ka, qop[i][kc], s[i][tb]);
            } else {
              const bf16x8 ka = fp8x8_to_bf16x8(raw.x, raw.y);
#pragma unroll
              for (int i = 0; i < NQB; ++i)
                if (qvalid[i]) s[i][tb] = mfma_bf16(ka, qop[i][kc], s[i][tb]);
            }
          }
        }
      }

      // ---- scale, mask, online softmax, P operand ------------------------------------
      const bool need_mask = !(c0 >= vis_lo_all && c0 + 31 <= vis_hi_all);
      float ks[8], vs[8];
      if constexpr (PT) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          ks[k] = ksl[wt * 32 + 4 * g + k];
          ks[4 + k] = ksl[wt * 32 + 16 + 4 * g + k];
          vs[k] = vsl[wt * 32 + 4 * g + k];
          vs[4 + k] = vsl[wt * 32 + 16 + 4 * g + k];
        }
      }
      bf16x8 phi[C::PV_FP8 ? 1 : NQB], plo[C::PV_FP8 ? 1 : NQB];
      long phi8[C::PV_FP8 ? NQB : 1], plo8[C::PV_FP8 ? NQB : 1];
#pragma unroll
      for (int i = 0; i < NQB; ++i) {
        if (!qvalid[i]) continue;
        float x[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[k] = s[i][0][k] * qk_scale;
          x[4 + k] = s[i][1][k] * qk_scale;
        }
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
        float mx = x[0];
#pragma unroll
        for (int k = 1; k < 8; ++k) mx = fmaxf(mx, x[k]);
        mx = wave_max_xor_16_32(mx);
        const float mnew = fmaxf(mrun[i], mx);
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = fast_exp2(mrun[i] - muse);
        mrun[i] = mnew;
        float pv[8];
        float ps = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          pv[k] = fast_exp2(x[k] - muse);
          ps += pv[k];
        }
        lrun[i] = lrun[i] * alpha + ps;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) o[i][db] *= alpha;
        if constexpr (C::PV_FP8) {
#pragma unroll
          for (int db = 0; db < C::DB; ++db) olo[i][db] *= alpha;
          float y[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) y[k] = pv[k] * 448.0f;
          const uint32_t h0 = f32x4_to_fp8x4(y[0], y[1], y[2], y[3]);
          const uint32_t h1 = f32x4_to_fp8x4(y[4], y[5], y[6], y[7]);
          const f32x2 d0 = fp8x2_to_f32x2<false>(h0), d1 = fp8x2_to_f32x2<true>(h0);
          const f32x2 d2 = fp8x2_to_f32x2<false>(h1), d3 = fp8x2_to_f32x2<true>(h1);
          const uint32_t l0 = f32x4_to_fp8x4((y[0] - d0[0]) * 16.f, (y[1] - d0[1]) * 16.f,
                                             (y[2] - d1[0]) * 16.f, (y[3] - d1[1]) * 16.f);
          const uint32_t l1 = f32x4_to_fp8x4((y[4] - d2[0]) * 16.f, (y[5] - d2[1]) * 16.f,
                                             (y[6] - d3[0]) * 16.f, (y[7] - d3[1]) * 16.f);
          phi8[i] = (long)h0 | ((long)h1 << 32);
          plo8[i] = (long)l0 | ((long)l1 << 32);
        } else {
          bf16x8 hv, lv;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float y = PT ? pv[k] * vs[k] : pv[k];
            const __bf16 h = (__bf16)y;
            hv[k] = h;
            lv[k] = (__bf16)(y - (float)h);
          }
          phi[i] = hv;
          plo[i] = lv;
        }
      }

      // ---- O^T += V^T P^T --------------------------------------------------------------
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        if constexpr (!KVF8) {
          const uint8_t* b1 = Vl + (wt * 32 + 4 * g + (L16 >> 2)) * C::ROWB + (16 * db + 4 * (L16 & 3)) * 2;
          const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4*)(b1));
          const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4*)(b1 + 16 * C::ROWB));
          bf16x8 va;
          const __bf16* p1 = reinterpret_cast<const __bf16*>(&v1);
          const __bf16* p2 = reinterpret_cast<const __bf16*>(&v2);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            va[k] = p1[k];
            va[4 + k] = p2[k];
          }
#pragma unroll
          for (int i = 0; i < NQB; ++i) {
            if (!qvalid[i]) continue;
            o[i][db] = mfma_bf16(va, phi[i], o[i][db]);
            o[i][db] = mfma_bf16(va, plo[i], o[i][db]);
          }
        } else {
          const int jr = L16 >> 1;
          const int tok = jr < 4 ? 4 * g + jr : 16 + 4 * g + (jr - 4);
          const uint8_t* b1 = Vl + (wt * 32 + tok) * C::ROWB + 16 * db + 8 * (L16 & 1);
          const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((PA_LDS i32x2*)(b1));
          if constexpr (C::PV_FP8) {
            const long va = (long)(uint32_t)w[0] | ((long)(uint32_t)w[1] << 32);
#pragma unroll
            for (int i = 0; i < NQB; ++i) {
              if (!qvalid[i]) continue;
              o[i][db] = mfma_fp8(va, phi8[i], o[i][db]);
              olo[i][db] = mfma_fp8(va, plo8[i], olo[i][db]);
            }
          } else {
            const bf16x8 va = fp8x8_to_bf16x8((uint32_t)w[0], (uint32_t)w[1]);
#pragma unroll
            for (int i = 0; i < NQB; ++i) {
              if (!qvalid[i]) continue;
              o[i][db] = mfma_bf16(va, phi[i], o[i][db]);
              o[i][db] = mfma_bf16(va, plo[i], o[i][db]);
            }
          }
        }
      }
    }
    __syncthreads();
  }

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
    const int m = 16 * (wq + WQ * i) + L16;
    if (m >= Mq) continue;
    const int r = m / G;
    const int hl = m - r * G;
    const int64_t th = (int64_t)(it.row0 + r) * Hq + (int64_t)it.kvh * G + hl;
    const bool empty = !(ltot[i] > 0.f);
    const float sc = empty ? 0.f : out_scale / ltot[i];
    if (it.nsplit == 1) {
      if (a.out_bf16) {
        __bf16* dst = static_cast<__bf16*>(a.out) + th * DH;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 v;
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = (__bf16)(o[i][db][k] * sc);
          *reinterpret_cast<bf16x4*>(dst + 16 * db + 4 * g) = v;
        }
      } else {
        float* dst = static_cast<float*>(a.out) + th * DH;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * g) = o[i][db] * sc;
      }
    } else {
      float* dst = a.partial_o + (th * a.s_max + it.split) * DH;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * g) = o[i][db] * sc;
      if (g == 0)
        a.partial_lse[th * a.s_max + it.split] = empty ? -INFINITY : (mrun[i] + __log2f(ltot[i])) * kLn2;
    }
  }
}

template <int DH, bool QF8, bool KVF8, bool PT, int WQ, int NQB>
static int launch_one(const Stage1Args& a, int num_items, void* stream) {
  hipLaunchKernelGGL((stage1_kernel<DH, QF8, KVF8, PT, WQ, NQB>), dim3(num_items), dim3(256), 0,
                     (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

// Largest query-block count per wave instantiated for a mode: per-tensor FP8 V keeps
// a second (lo) accumulator, which does not fit in registers for more blocks.
template <int DH, bool KVF8, bool PT>
constexpr int max_nqb() {
  constexpr bool pv_fp8 = KVF8 && !PT;
  if constexpr (DH == 128) return pv_fp8 ? 2 : 3;
  else return pv_fp8 ? 1 : 2;
}

template <int DH, bool QF8, bool KVF8, bool PT>
static int dispatch_tiles(const KernelCfg& c, const Stage1Args& a, int n, void* s) {
  constexpr int NMAX = max_nqb<DH, KVF8, PT>();
  if (c.wq == 1 && c.nqb == 1) return launch_one<DH, QF8, KVF8, PT, 1, 1>(a, n, s);
  if (c.wq == 2 && c.nqb == 1) return launch_one<DH, QF8, KVF8, PT, 2, 1>(a, n, s);
  if (c.wq == 4 && c.nqb == 1) return launch_one<DH, QF8, KVF8, PT, 4, 1>(a, n, s);
  if constexpr (NMAX >= 2) {
    if (c.wq == 4 && c.nqb == 2) return launch_one<DH, QF8, KVF8, PT, 4, 2>(a, n, s);
  }
  if constexpr (NMAX >= 3) {
    if (c.wq == 4 && c.nqb == 3) return launch_one<DH, QF8, KVF8, PT, 4, 3>(a, n, s);
  }
  return (int)hipErrorInvalidValue;
}

template <int DH>
static int dispatch_modes(const KernelCfg& c, const Stage1Args& a, int n, void* s) {
  if (!c.qf8 && !c.kvf8) return dispatch_tiles<DH, false, false, false>(c, a, n, s);
  if (c.qf8 && c.kvf8 && !c.pt) return dispatch_tiles<DH, true, true, false>(c, a, n, s);
  if (c.qf8 && c.kvf8 && c.pt) return dispatch_tiles<DH, true, true, true>(c, a, n, s);
  if (!c.qf8 && c.kvf8 && !c.pt) return dispatch_tiles<DH, false, true, false>(c, a, n, s);
  if (!c.qf8 && c.kvf8 && c.pt) return dispatch_tiles<DH, false, true, true>(c, a, n, s);
  return (int)hipErrorInvalidValue;
}

bool stage1_cfg_supported(const KernelCfg& c) {
  if (c.dh != 128 && c.dh != 256) return false;
  if (c.qf8 && !c.kvf8) return false;
  if (!c.kvf8 && c.pt) return false;
  const bool pv_fp8 = c.kvf8 && !c.pt;
  const int nmax = c.dh == 128 ? (pv_fp8 ? 2 : 3) : (pv_fp8 ? 1 : 2);
  if (c.nqb == 1) return c.wq == 1 || c.wq == 2 || c.wq == 4;
  return c.wq == 4 && c.nqb >= 2 && c.nqb <= nmax;
}

int launch_stage1(const KernelCfg& c, const Stage1Args& a, int num_items, void* stream) {
  if (num_items <= 0) return 0;
  if (c.dh == 128) return dispatch_modes<128>(c, a, num_items, stream);
  if (c.dh == 256) return dispatch_modes<256>(c, a, num_items, stream);
  return (int)hipErrorInvalidValue;
}

}  // namespace pa
