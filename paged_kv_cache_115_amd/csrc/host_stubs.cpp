// Host-only build of libpagedkv for the address and undefined-behaviour
// sanitizers (g++ cannot compile the HIP kernels): the C ABI, the block
// manager, the planner and the validation calls are the real sources; this
// file stands in for the kernel launchers and the two entry points that live
// in device-code files.  Every GPU entry point still runs all of its host-side
// checks and then fails with PA_ERR_HIP or PA_ERR_UNSUPPORTED: nothing is
// computed here.  Never part of the GPU library.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "launch.h"

namespace pagedkv {

hipError_t launch_decode_attention(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_merge(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t decode_resident_workgroups_per_cu(int*) { return hipErrorNoDevice; }
hipError_t launch_reshape_and_cache(const pa_kv_pool&, const void*, const void*, const int64_t*, int32_t, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_copy_blocks(const pa_kv_pool&, const int32_t*, int32_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_swap_blocks(const void*, const void*, void*, void*, int64_t, const SwapBatch&, int32_t, bool,
                              hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace pagedkv

extern "C" pa_status pa_decode_noalloc(const pa_kv_pool* pool, const void*, void*, int32_t, const int32_t*, int32_t,
                                       const int32_t*, int32_t, int32_t num_q_heads, float, const void*, const void*,
                                       const void*, const pa_decode_plan_info* info, void*) {
  if (pa_status st = pagedkv::noalloc_check(pool, info, num_q_heads, "pa_decode_noalloc")) return st;
  return pagedkv::fail(PA_ERR_UNSUPPORTED, "pa_decode_noalloc: host-only sanitizer build, no kernels");
}

extern "C" pa_status pa_probe_read(const void*, size_t, int32_t, void*, void*) {
  return pagedkv::fail(PA_ERR_UNSUPPORTED, "pa_probe_read: host-only sanitizer build, no kernels");
}
