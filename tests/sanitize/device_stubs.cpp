// Host-only stand-ins for the device side of the library, so that the planner in api.cpp
// can be built with the host compiler's address and undefined-behaviour sanitizers.  The
// fuzz driver calls only pa_plan_splits with a given CU count, so none of these runs.
#include <hip/hip_runtime_api.h>

#include "kv_append.hpp"
#include "pa_internal.hpp"

namespace pa {
int launch_stage1(const KernelCfg&, const Stage1Args&, int, void*) { return 1; }
int launch_stage1_kr(int, int, const KrArgs&, int, void*) { return 1; }
int launch_stage1_mla(int, const KrArgs&, int, void*) { return 1; }
int launch_gather_rope(const KernelCfg&, const GatherRopeArgs&, int, void*) { return 1; }
int launch_merge(const MergeArgs&, void*) { return 1; }
int launch_gather(const KernelCfg&, const GatherArgs&, int, void*) { return 1; }
int launch_quant(const void*, int, int64_t, int, int, int, uint8_t*, float*, void*) { return 1; }
int launch_append(const AppendArgs&, int, int, int, void*) { return 1; }
int launch_quant_heads(const void*, int, int64_t, int, int, uint8_t*, float*, void*) { return 1; }
}  // namespace pa

extern "C" {
hipError_t hipGetDevice(int* d) { *d = 0; return hipErrorNoDevice; }
hipError_t hipDeviceGetAttribute(int*, hipDeviceAttribute_t, int) { return hipErrorNoDevice; }
const char* hipGetErrorString(hipError_t) { return "no device (host-only build)"; }
}
