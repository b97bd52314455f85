// pa_decode_noalloc: pa_decode for callers that cannot allocate device memory
// (code under stream capture, tight serving loops, harnesses that forbid
// allocation).  The decode launches keep the (max, sum, accumulator) records
// of sequences cut into pieces in a workspace; here the workspace is a
// file-scope device array of fixed size instead of a caller buffer.
//
// `scratch` below is a device symbol.  In host code its name is only a
// host-side stand-in, not a device address, so the host never uses it
// directly: on a device's first call the library asks the runtime for that
// device's address of the array (hipGetSymbolAddress, with the device
// current) and keeps it per device; every launch then receives that address
// like any caller workspace.  Each device that runs the call holds its own
// copy of the array until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace pagedkv {
namespace {

static __device__ __align__(256) char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device.
pa_status scratch_address(void** ptr, const char* who) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(PA_ERR_HIP, "%s: no current device", who);
  }
  if (dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "%s: device %d past the %d supported", who, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return fail(PA_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array failed on device %d: %s", who, dev,
                  hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace
}  // namespace pagedkv

extern "C" pa_status pa_decode_noalloc(const pa_kv_pool* pool, const void* q, void* out, int32_t out_dtype,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                       float scale, const void* new_key, const void* new_value, const void* plan,
                                       const pa_decode_plan_info* info, void* stream) {
  const char* who = "pa_decode_noalloc";
  // The size check needs only the plan's info: a plan too large for the
  // array is refused before the device is touched.
  if (pa_status st = pagedkv::noalloc_check(pool, info, num_q_heads, who)) return st;
  if (info->num_jobs == 0 && info->num_merges == 0) return PA_OK;
  void* ws = nullptr;
  if (pa_status st = pagedkv::scratch_address(&ws, who)) return st;
  return pagedkv::decode_stages(pagedkv::kStageAttention | pagedkv::kStageMerge, who, pool, q, out, out_dtype,
                                block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads, scale, new_key,
                                new_value, plan, info, ws, (size_t)PA_NOALLOC_SCRATCH_BYTES, stream);
}
