// Issue-priority balance between the workgroups of the stage-1 kernels that share a
// compute unit.
#pragma once

namespace pa {
// Issue priority of two workgroups sharing a compute unit.  Measured on the stage-1
// kernels: the workgroup in slot 0 of its CU (HW_ID.TG_ID) wins the SIMDs' issue
// arbitration against the one in slot 1 and finishes its item 15-20% earlier; the other
// then runs alone for the rest.  When every item of a launch runs at once (two per CU,
// items of about equal cost), the slot-1 workgroup raises its wave priority for the first
// half of its tiles and the slot-0 one for the second half, so both finish together.
// at() is called at tile indices that are multiples of step, in a loop that reaches the
// middle tile whenever ntiles >= 4 step (shorter items keep the default priority).
struct FairShare {
  bool slot1;
  int tswitch;                        // tile index at which the priorities swap, -1: never
  __device__ __forceinline__ FairShare(bool fair, int ntiles, int step = 1) {
    constexpr int kHwRegHwId = (31 << 11) | 4;            // s_getreg: all of HW_ID
    fair = fair && ntiles >= 4 * step;
    slot1 = fair && ((__builtin_amdgcn_s_getreg(kHwRegHwId) >> 16) & 1) != 0;
    tswitch = fair ? (ntiles / 2) / step * step : -1;
    if (slot1) __builtin_amdgcn_s_setprio(1);
  }
  __device__ __forceinline__ void at(int ti) const {
    if (ti == tswitch) {
      if (slot1) __builtin_amdgcn_s_setprio(0);
      else __builtin_amdgcn_s_setprio(1);
    }
  }
};

}  // namespace pa
