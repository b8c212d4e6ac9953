// Output rows of the stage-1 kernels as bf16 with 16-byte stores.
#pragma once

#include "common.hpp"

namespace pa {

// One output row held as an MFMA O^T accumulator: lane group g (lane / 16) of the row's
// lanes holds channels 16 db + 4g .. +3 of every 16-channel block db, as o[db][0..3].
// For each pair of blocks the lane groups 2h and 2h+1 exchange one half through
// v_permlane16_swap, so that each lane writes 8 contiguous channels: one 16-byte store
// per pair instead of two 8-byte ones (measured: the stores of an item's last tile queue
// behind the other workgroup's loads, and half the instructions take half the time).
// dst points at the row's first channel (16-byte aligned); NDB is even; lanes l and
// l ^ 16 (the same row) must both be active.
template <int NDB>
__device__ __forceinline__ void store_row_bf16_x16(__bf16* dst, const f32x4 (&o)[NDB], float sc, int g) {
  static_assert(NDB % 2 == 0, "pairs of 16-channel blocks");
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bool odd = (g & 1) != 0;
  const int h = g >> 1;
#pragma unroll
  for (int db = 0; db < NDB; db += 2) {
    uint32_t keep[2], got[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const bf16x2 pa = {(__bf16)(o[db][2 * w] * sc), (__bf16)(o[db][2 * w + 1] * sc)};
      const bf16x2 pb = {(__bf16)(o[db + 1][2 * w] * sc), (__bf16)(o[db + 1][2 * w + 1] * sc)};
      const uint32_t ua = __builtin_bit_cast(uint32_t, pa), ub = __builtin_bit_cast(uint32_t, pb);
      const uint32_t send = odd ? ua : ub;
      const auto r = __builtin_amdgcn_permlane16_swap(send, send, false, false);
      got[w] = odd ? r[0] : r[1];       // odd: the even lane's half of block db+1; even: the odd lane's of db
      keep[w] = odd ? ub : ua;
    }
    const uint4 v = odd ? uint4{got[0], got[1], keep[0], keep[1]} : uint4{keep[0], keep[1], got[0], got[1]};
    *reinterpret_cast<uint4*>(dst + 16 * (db + (odd ? 1 : 0)) + 8 * h) = v;
  }
}

}  // namespace pa
