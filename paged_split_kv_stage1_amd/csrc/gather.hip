// Test hooks: run stage 1's KV address code (kv_addr.hpp) over every tile of every work
// item, with stage 1's tile geometry for the plan's kernel configuration, and record
// the byte offset of every 16-byte K/V chunk (and the element offset of every scale)
// that stage 1 loads, indexed by (item, token - tok_begin, chunk) -- for the equal-width
// kernel and for the two wider-key kernels.
#include "common.hpp"
#include "kv_addr.hpp"

namespace pa {

template <int DH, int KVB, int WQ, bool PT>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  constexpr int CPR = DH * KVB / 16;
  constexpr int BN = 32 * (4 / WQ);                     // tokens per tile, as in stage 1
  constexpr int NP = BN / 16 + 1;
  using KA = KvTileAddr<CPR, BN, KVB>;
  const PaItem it = a.items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const KA ka(lane, a.kv_ss);
  const cint32* pidx = (const cint32*)(a.page_indices) + it.page_base;
  const int64_t head_off = (int64_t)it.kvh * a.kv_sh;
  const int shift = a.page_shift;
  const int pmask = (1 << shift) - 1;
  const int tb0 = it.tok_begin, te = it.tok_end;
  const int ntiles = te > tb0 ? (te - tb0 + BN - 1) / BN : 0;
  const int64_t base = (int64_t)blockIdx.x * a.max_tok;
  for (int ti = 0; ti < ntiles; ++ti) {
    const int tile0 = tb0 + ti * BN;
#pragma unroll
    for (int i = 0; i < KA::CPT; ++i) {
      const int jb = KA::group_token(tile0, wave, i, te);
      const int32_t page = KA::group_page(pidx, jb, shift);
      const int64_t off = KA::row_offset(page, jb, a.kv_sp, head_off, a.kv_ss, pmask) + ka.lane_offset(jb, te, a.kv_ss);
      a.kv_off[(base + ka.lane_token(jb, te) - tb0) * CPR + ka.cpos] = off;
    }
    if constexpr (PT) {
      if (tid < 2 * BN) {
        const ScaleTileAddr<BN, NP> sa(pidx, tile0, te, shift, tid, it.kvh, a.sc_sp, a.sc_sh, a.sc_ss);
        a.sc_off[(base + sa.token - tb0) * 2 + (sa.is_v ? 1 : 0)] = sa.off;
      }
    }
  }
}

template <int DH, int KVB>
static int launch_dk(const KernelCfg& c, const GatherArgs& a, int n, hipStream_t s) {
  if (c.wq == 1 && !c.pt) hipLaunchKernelGGL((gather_kernel<DH, KVB, 1, false>), dim3(n), dim3(256), 0, s, a);
  else if (c.wq == 1) hipLaunchKernelGGL((gather_kernel<DH, KVB, 1, true>), dim3(n), dim3(256), 0, s, a);
  else if (c.wq == 2 && !c.pt) hipLaunchKernelGGL((gather_kernel<DH, KVB, 2, false>), dim3(n), dim3(256), 0, s, a);
  else if (c.wq == 2) hipLaunchKernelGGL((gather_kernel<DH, KVB, 2, true>), dim3(n), dim3(256), 0, s, a);
  else if (c.wq == 4 && !c.pt) hipLaunchKernelGGL((gather_kernel<DH, KVB, 4, false>), dim3(n), dim3(256), 0, s, a);
  else if (c.wq == 4) hipLaunchKernelGGL((gather_kernel<DH, KVB, 4, true>), dim3(n), dim3(256), 0, s, a);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

// The same for the two wider-key kernels: every 16-byte load (and latent scale load) of
// every wave's span of every tile, through the load enumerators the kernels themselves
// call (RopeQuarterLoads, LatentSpanLoads), recorded at column (part offset + chunk) of
// token (token - tok_begin) of the item.
template <int DV, bool MLA>
__global__ __launch_bounds__(256) void gather_rope_kernel(GatherRopeArgs a) {
  constexpr int BN = MLA ? 64 : 128;                    // tokens per tile, as in the kernels
  constexpr int SPAN = MLA ? 16 : 32;                   // tokens one wave loads per tile
  constexpr int C0 = MLA ? DV / 16 : DV * 2 / 16;       // columns of part 0 (latent / K main)
  constexpr int C1 = 8;                                 // rotary row: 64 bf16
  constexpr int NE = C0 + C1 + (MLA ? DV / 128 : DV * 2 / 16);
  const PaItem it = a.items[blockIdx.x];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const cint32* pidx = (const cint32*)(a.page_indices) + it.page_base;
  const int tb0 = it.tok_begin, te = it.tok_end;
  const int ntiles = te > tb0 ? (te - tb0 + BN - 1) / BN : 0;
  const int64_t base = (int64_t)blockIdx.x * a.max_tok;
  auto rec = [&](auto part, int, int64_t off, int token, int chunk) {
    constexpr int PART = decltype(part)::value;
    const int col = (PART == 0 ? 0 : PART == 1 ? C0 : C0 + C1) + chunk;
    a.off[(base + token - tb0) * NE + col] = off;
  };
  if constexpr (MLA) {
    const LatentSpanLoads<DV> ld(lane, it.kvh, a.m_sp, a.m_sh, a.m_ss, a.r_sp, a.r_sh, a.r_ss, a.s_sp, a.s_sh, a.s_ss);
    for (int ti = 0; ti < ntiles; ++ti) ld.tile(pidx, tb0 + ti * BN + SPAN * wave, te, a.page_shift, rec);
  } else {
    const RopeQuarterLoads<DV> ld(lane, it.kvh, a.m_sp, a.m_sh, a.m_ss, a.r_sp, a.r_sh, a.r_ss, a.v_sp, a.v_sh,
                                  a.v_ss);
    for (int ti = 0; ti < ntiles; ++ti) ld.tile(pidx, tb0 + ti * BN + SPAN * wave, te, a.page_shift, rec);
  }
}

int launch_gather_rope(const KernelCfg& c, const GatherRopeArgs& a, int num_items, void* stream) {
  if (num_items <= 0) return 0;
  const hipStream_t s = (hipStream_t)stream;
  if (c.mla && c.dv == 512) hipLaunchKernelGGL((gather_rope_kernel<512, true>), dim3(num_items), dim3(256), 0, s, a);
  else if (!c.mla && c.dv == 128) hipLaunchKernelGGL((gather_rope_kernel<128, false>), dim3(num_items), dim3(256), 0, s, a);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int launch_gather(const KernelCfg& c, const GatherArgs& a, int num_items, void* stream) {
  if (num_items <= 0) return 0;
  const hipStream_t s = (hipStream_t)stream;
  const int kvb = c.kvf8 ? 1 : 2;
  if (c.dh == 128) return kvb == 1 ? launch_dk<128, 1>(c, a, num_items, s) : launch_dk<128, 2>(c, a, num_items, s);
  if (c.dh == 256) return kvb == 1 ? launch_dk<256, 1>(c, a, num_items, s) : launch_dk<256, 2>(c, a, num_items, s);
  if (c.dh == 512) return kvb == 1 ? launch_dk<512, 1>(c, a, num_items, s) : launch_dk<512, 2>(c, a, num_items, s);
  return (int)hipErrorInvalidValue;
}

}  // namespace pa
